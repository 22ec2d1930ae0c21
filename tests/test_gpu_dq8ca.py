"""GPU parity of linear_dq8ca_q4gsw (per-row int8 activations, int8 MFMA) against the oracle.

The quantisation decides integers, so its codes, scales and zero points must equal the oracle's
bit for bit (both take every step in fp32).  The linear is compared elementwise with the oracle's
fp64 forward of the dequantised rows: the GPU's group sums are exact in int32, and its only
roundings are the fp32 accumulation of the groups' scaled sums, the row scale and the split
reduction, so |gpu - oracle| <= (groups + splits + 3) 2^-24 R, at least the fp32 tolerance 1e-5 R.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synthetic_inputs import DTYPES, draw_activation, make_linear, make_workload
from tests.conftest import load_golden
from tests.gpu_helpers import THREADS, assert_within, dev, lib, pack, sample_rows

pytestmark = pytest.mark.gpu


def tol(K, gs, splits):
    return max(1e-5, (K // gs + splits + 3) * 2.0 ** -24)


QUANT_CASES = [
    # M, K, dtype, sigma
    (1, 64, "f32", 1.0),
    (7, 1000, "bf16", 3.0),
    (130, 257, "f16", 0.01),
    (64, 8192, "bf16", 1.0),     # the longest row kept in registers between the two passes
    (3, 8200, "bf16", 2.0),      # longer rows read the row a second time
    (2, 16384, "f16", 0.5),
    (33, 96, "f32", 1e-3),
]


@pytest.mark.parametrize("M,K,act,sigma", QUANT_CASES)
def test_quantize_bit_exact(M, K, act, sigma):
    q = lib()
    g = torch.Generator().manual_seed(M + K)
    x = draw_activation(g, M, K, act, sigma)
    x[M // 2, ::3] = 0.0
    if M > 2:
        x[1] = x[1].abs()                 # a row with no negative values
        x[2] = -x[2].abs()                # and one with no positive values
    print(f"dq8ca quantize M={M} K={K} {act}", flush=True)
    gq, gs_, gz = q.dq8ca_quantize(dev(x))
    torch.cuda.synchronize()
    oq, os_, oz = O.dq8ca_quantize(x, THREADS)
    assert np.array_equal(gq.cpu().numpy(), oq)
    assert np.array_equal(gs_.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(gz.cpu().numpy(), oz)


def test_quantize_golden_rows():
    """The hand-worked rows of tests/golden/dq8ca_rows.txt (ties to even, one-signed rows, zeros)."""
    q = lib()
    g = load_golden("dq8ca_rows.txt")
    for row in "abcd":
        for act in (("f32",) if row == "a" else tuple(DTYPES)):   # row a holds 0.3, exact in fp32 only
            x = torch.tensor([[float(v) for v in g[f"{row}_x"][0]]], dtype=DTYPES[act])
            gq, gs_, gz = q.dq8ca_quantize(dev(x))
            torch.cuda.synchronize()
            assert gq.cpu().tolist()[0] == [int(v) for v in g[f"{row}_q"][0]], (row, act)
            assert float(gs_.item()) == g[f"{row}_scale"], (row, act)
            assert int(gz.item()) == int(g[f"{row}_zp"]), (row, act)


LINEAR_CASES = [
    # M, N, K, gs, act, scale dtype
    (4, 32, 64, 32, "f32", "f32"),
    (9, 256, 512, 64, "bf16", "f16"),
    (130, 512, 1024, 128, "f16", "f16"),
    (64, 300, 256, 32, "f32", "f16"),       # N tail inside a block
    (200, 264, 384, 64, "bf16", "f32"),
    (1, 2048, 2048, 32, "f16", "f16"),
    (257, 128, 192, 64, "f32", "f16"),      # K = 192: chunks past K hold code 8 and zero activations
    (5, 64, 8320, 64, "bf16", "f16"),       # rows past 8192 columns: the quantisation reads them twice
]


def _check_linear(q, case, pw, w, rows=None, splits=None, label=""):
    x = dev(case.x)
    y = q.linear_dq8ca(pw, x)
    torch.cuda.synchronize()
    info = q.plan(q.OP_DQ8CA, pw, case.M, case.x.dtype)
    assert info["route"] == "dq8ca", info
    xs = case.x if rows is None else case.x[rows].contiguous()
    ref, norm = O.linear_dq8ca(xs, w.codes, w.scales, w.group_size, THREADS)
    assert_within(y, ref, norm, tol(w.K, w.group_size, splits or info["splits"]), label, rows)


@pytest.mark.parametrize("M,N,K,gs,act,sdt", LINEAR_CASES)
def test_linear_dq8ca(M, N, K, gs, act, sdt):
    q = lib()
    case = make_linear(M, K, N, gs, act, sdt, seed=M + N + gs, s_lo=0.005 if sdt == "f32" else 0.002)
    pw = pack(q, case.w)
    print(f"dq8ca linear M={M} N={N} K={K} gs={gs} {act} {sdt}", flush=True)
    _check_linear(q, case, pw, case.w, label=f"dq8ca M={M} gs={gs}")


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_linear_dq8ca_forced_splits(splits):
    q = lib()
    case = make_linear(100, 1536, 512, 128, "bf16", "f16", seed=splits)
    pw = pack(q, case.w)
    with q.forced_plan(splits=splits):
        assert q.plan(q.OP_DQ8CA, pw, 100, case.x.dtype)["splits"] == splits
        y = q.linear_dq8ca(pw, dev(case.x))
        torch.cuda.synchronize()
    ref, norm = O.linear_dq8ca(case.x, case.w.codes, case.w.scales, 128, THREADS)
    assert_within(y, ref, norm, tol(1536, 128, splits), f"dq8ca splits={splits}")


def test_linear_dq8ca_prefill_shape():
    """The prefill workload (M=512, K=8192, N=2048, gs=128, bf16 x) through dq8ca, sampled rows."""
    q = lib()
    case = make_workload("prefill")
    pw = pack(q, case.w)
    _check_linear(q, case, pw, case.w, rows=sample_rows(case.M), label="dq8ca prefill")


def test_linear_dq8ca_code8_zero_and_zero_rows():
    """Code 8 everywhere gives exact zeros; an all-zero row gives an exactly zero output row."""
    q = lib()
    case = make_linear(40, 256, 320, 64, "f16", "f16", seed=4)
    case.x[5] = 0.0
    pw = pack(q, case.w)
    y = q.linear_dq8ca(pw, dev(case.x))
    eight = pack(q, type(case.w)(torch.full_like(case.w.codes, 8), case.w.scales, 64))
    y8 = q.linear_dq8ca(eight, dev(case.x))
    torch.cuda.synchronize()
    assert torch.equal(y[5], torch.zeros_like(y[5]))
    assert torch.equal(y8, torch.zeros_like(y8))
