"""GPU parity of the input-gradient routes added for group sizes 32 and 64 and of the 16x16x32
fallback kernel, against the fp64 oracle, elementwise.

bwd_bsplit: fp16 scales, gs % 64 == 0 or gs == 32, d_out fp32 / bf16 (and fp16 whose scales
cannot be folded).  (code - 8) * scale is split exactly into bf16 hi + lo; fp32 d_out is split into
bf16 hi + lo (|err| <= 2^-18 |d_out|), so the fp32 tolerance of 1e-5 * R holds as on bwd_split.
The 16x16x32 kernel serves fp16 d_out with foldable scales at group sizes 8, 16, 24, 40, 48, ...
"""
import pytest
import torch

from synthetic_inputs import make_linear
from tests.gpu_helpers import TOL, assert_within, dev, lib, oracle_bwd, pack, sample_rows

pytestmark = pytest.mark.gpu

BSPLIT_CASES = [
    # M, N, K, gs, d_out dtype
    (64, 512, 512, 32, "f32"),
    (130, 1000, 384, 64, "f32"),      # ragged M and N (contraction tail inside a chunk)
    (96, 512, 320, 32, "bf16"),       # K tail inside a 256-column block
    (200, 768, 576, 192, "bf16"),     # gs = 3 * 64: one group per wave, groups straddle blocks
    (40, 256, 1024, 64, "f32"),
    (9, 200, 160, 32, "bf16"),        # just past the small-M routes, K ends inside a 256-column block
]


@pytest.mark.parametrize("M,N,K,gs,act", BSPLIT_CASES)
def test_bwd_bsplit(M, N, K, gs, act):
    q = lib()
    case = make_linear(M, K, N, gs, act, "f16", seed=M * 13 + N + K, fwd=False, bwd=True,
                       sigma=0.1 if act == "f32" else 1.0)
    pw = pack(q, case.w)
    g = dev(case.d_out)
    assert q.route(q.OP_BWD_INPUT, pw, M, case.d_out.dtype) == "bwd_bsplit"
    dx = q.linear_bwd_input(pw, g)
    torch.cuda.synchronize()
    ref, norm = oracle_bwd(case.d_out, case.w)
    assert_within(dx, ref, norm, TOL[case.d_out.dtype], f"bwd_bsplit {act} gs={gs}")


def test_bwd_bsplit_fp16_unfoldable():
    """fp16 d_out with a scale that cannot be folded into fp16 (a subnormal one) takes bwd_bsplit,
    whose hi + lo split of (code - 8) * scale stays exact for subnormal fp16 scales."""
    q = lib()
    case = make_linear(72, 384, 640, 64, "f16", "f16", seed=31, fwd=False, bwd=True)
    case.w.scales[1, 5] = torch.tensor(3e-6, dtype=torch.float16)      # subnormal in fp16
    case.w.scales[0, 7] = torch.tensor(0.0, dtype=torch.float16)
    pw = pack(q, case.w)
    assert not pw.foldable
    assert q.route(q.OP_BWD_INPUT, pw, 72, torch.float16) == "bwd_bsplit"
    dx = q.linear_bwd_input(pw, dev(case.d_out))
    torch.cuda.synchronize()
    ref, norm = oracle_bwd(case.d_out, case.w)
    assert_within(dx, ref, norm, TOL[torch.float16], "bwd_bsplit fp16 unfoldable")


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_bwd_bsplit_llama_q_shape(act):
    """The frozen-base input gradient through the Llama Q projection (M = 512, N = K = 2048,
    gs = 32, fp16 scales), checked on sampled rows."""
    q = lib()
    case = make_linear(512, 2048, 2048, 32, act, "f16", seed=7, fwd=False, bwd=True,
                       sigma=0.1 if act == "f32" else 1.0)
    pw = pack(q, case.w)
    info = q.plan(q.OP_BWD_INPUT, pw, 512, case.d_out.dtype)
    assert info["route"] == "bwd_bsplit" and info["tile_rows"] == 128
    dx = q.linear_bwd_input(pw, dev(case.d_out))
    rows = sample_rows(512)
    ref, norm = oracle_bwd(case.d_out, case.w, rows)
    assert_within(dx, ref, norm, TOL[case.d_out.dtype], f"bwd_bsplit llama q {act}", rows)


@pytest.mark.parametrize("splits", [1, 3, 8])
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_bwd_bsplit_forced_splits(act, splits):
    q = lib()
    case = make_linear(100, 320, 1536, 32, act, "f16", seed=splits, fwd=False, bwd=True,
                       sigma=0.1 if act == "f32" else 1.0)
    pw = pack(q, case.w)
    with q.forced_plan(splits=splits):
        info = q.plan(q.OP_BWD_INPUT, pw, 100, case.d_out.dtype)
        dx = q.linear_bwd_input(pw, dev(case.d_out))
        torch.cuda.synchronize()
    assert info["route"] == "bwd_bsplit" and info["splits"] == splits, info
    ref, norm = oracle_bwd(case.d_out, case.w)
    assert_within(dx, ref, norm, TOL[case.d_out.dtype], f"bwd_bsplit splits={splits} {act}")


def _misaligned(t: torch.Tensor) -> torch.Tensor:
    """A copy of t on the GPU whose data starts one element past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 16, dtype=t.dtype, device="cuda")
    view = flat[1:1 + t.numel()].view(t.shape)
    view.copy_(t.cuda())
    return view


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_bwd_bsplit_unaligned(act):
    """d_out one element off 16-byte alignment: fp32 goes through the plane pre-pass's scalar loads,
    bf16 through the GEMM's guarded register loads."""
    q = lib()
    case = make_linear(70, 256, 520, 64, act, "f16", seed=5, fwd=False, bwd=True,
                       sigma=0.1 if act == "f32" else 1.0)
    pw = pack(q, case.w)
    dx = q.linear_bwd_input(pw, _misaligned(case.d_out))
    torch.cuda.synchronize()
    ref, norm = oracle_bwd(case.d_out, case.w)
    assert_within(dx, ref, norm, TOL[case.d_out.dtype], f"bwd_bsplit unaligned {act}")


V1_FOLD_CASES = [
    # M, N, K, gs: fp16 d_out, foldable fp16 scales, group sizes the 32x32 kernels do not take
    (96, 512, 384, 16),
    (40, 256, 240, 24),
    (130, 700, 264, 8),
]


@pytest.mark.parametrize("M,N,K,gs", V1_FOLD_CASES)
def test_bwd_fold_16x16_kernel(M, N, K, gs):
    q = lib()
    case = make_linear(M, K, N, gs, "f16", "f16", seed=M + gs, fwd=False, bwd=True)
    pw = pack(q, case.w)
    assert pw.foldable
    assert q.route(q.OP_BWD_INPUT, pw, M, torch.float16) == "bwd_fold"
    dx = q.linear_bwd_input(pw, dev(case.d_out))
    torch.cuda.synchronize()
    ref, norm = oracle_bwd(case.d_out, case.w)
    assert_within(dx, ref, norm, TOL[torch.float16], f"bwd 16x16x32 fold gs={gs}")
