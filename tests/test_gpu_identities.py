"""GPU checks against closed forms and identities (exact where the arithmetic is exact)."""
import numpy as np
import pytest
import torch

from synthetic_inputs import DTYPES, Weight, draw_activation, draw_codes, make_linear
from tests.conftest import load_golden
from tests.gpu_helpers import TOL, assert_within, dev, lib, oracle_bwd, oracle_fwd, pack

pytestmark = pytest.mark.gpu

FAMILIES = ("auto", "generic", "gemv", "gemm_fold")


def each_route(q, fn):
    for fam in FAMILIES:
        try:
            if fam == "auto":
                yield fam, fn()
            else:
                with q.forced_route(fam):
                    r = fn()
                yield fam, r
        except q.Q4gswError as e:
            if e.status != 11:
                raise


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("sdt", ["f32", "f16"])
@pytest.mark.parametrize("M", [2, 16])
def test_golden_worked_example(act, sdt, M):
    """The hand-worked example, tiled to M rows; every value is exact in every dtype."""
    q = lib()
    g = load_golden("worked_example_4x2.txt")
    gs = int(g["group_size"])
    codes = torch.tensor(g["codes"], dtype=torch.uint8)
    scales = torch.tensor(g["scales"], dtype=torch.float64).to(DTYPES[sdt])
    reps = M // 2
    x = torch.tensor(g["x"], dtype=torch.float64).repeat(reps, 1).to(DTYPES[act])
    d_out = torch.tensor(g["d_out"], dtype=torch.float64).repeat(reps, 1).to(DTYPES[act])
    y_want = torch.tensor(g["y"], dtype=torch.float32).repeat(reps, 1)
    dx_want = torch.tensor(g["d_x"], dtype=torch.float32).repeat(reps, 1)
    pw = q.pack(codes.cuda(), scales.cuda(), gs)
    for fam, y in each_route(q, lambda: q.linear_fwd(pw, x.cuda())):
        assert torch.equal(y.cpu(), y_want), (fam, y)
    for fam, dx in each_route(q, lambda: q.linear_bwd_input(pw, d_out.cuda())):
        assert torch.equal(dx.cpu(), dx_want), (fam, dx)


@pytest.mark.parametrize("sdt", ["f32", "f16"])
def test_golden_embedding(sdt):
    """The hand-worked embedding rows of the example (one id out of range), bit for bit."""
    q = lib()
    g = load_golden("worked_example_4x2.txt")
    codes = torch.tensor(g["codes"], dtype=torch.uint8)
    scales = torch.tensor(g["scales"], dtype=torch.float64).to(DTYPES[sdt])
    pw = q.pack(codes.cuda(), scales.cuda(), int(g["group_size"]))
    ids = torch.tensor([int(v) for v in g["ids"][0]], dtype=torch.int64)
    e = q.embedding(pw, ids.cuda())
    torch.cuda.synchronize()
    assert torch.equal(e.cpu(), torch.tensor(g["embedding"], dtype=torch.float32)), e


@pytest.mark.parametrize("M,act", [(1, "f16"), (6, "f32"), (64, "bf16"), (64, "f16"), (40, "f32")])
def test_code8_is_zero(M, act):
    q = lib()
    N, K, gs = 256, 256, 128
    x = draw_activation(torch.Generator().manual_seed(1), M, K, act)
    g = draw_activation(torch.Generator().manual_seed(2), M, N, act)
    codes = torch.full((N, K), 8, dtype=torch.uint8)
    scales = torch.rand(K // gs, N).to(torch.float16) + 0.01
    pw = q.pack(codes.cuda(), scales.cuda(), gs)
    for fam, y in each_route(q, lambda: q.linear_fwd(pw, x.cuda())):
        assert torch.count_nonzero(y) == 0, fam
    for fam, dx in each_route(q, lambda: q.linear_bwd_input(pw, g.cuda())):
        assert torch.count_nonzero(dx) == 0, fam


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
def test_one_hot_reads_every_code(act):
    """x = identity with power-of-two scales: y[m, n] = (code[n, m] - 8) * scale exactly."""
    q = lib()
    N, K, gs = 96, 256, 32
    gen = torch.Generator().manual_seed(5)
    codes = draw_codes(gen, N, K)
    expo = torch.tensor([[((gi * N + n) % 9) - 4 for n in range(N)] for gi in range(K // gs)],
                        dtype=torch.float64)
    scales = torch.pow(2.0, expo).to(torch.float16)
    x = torch.eye(K, dtype=DTYPES[act])
    want = ((codes.to(torch.float64) - 8) * scales.to(torch.float64).repeat_interleave(gs, dim=0).T).T
    pw = q.pack(codes.cuda(), scales.cuda(), gs)
    for fam, y in each_route(q, lambda: q.linear_fwd(pw, x.cuda())):
        assert torch.equal(y.cpu().to(torch.float64), want), fam
    eyeN = torch.eye(N, dtype=DTYPES[act])
    wantb = (codes.to(torch.float64) - 8) * scales.to(torch.float64).repeat_interleave(gs, dim=0).T
    for fam, dx in each_route(q, lambda: q.linear_bwd_input(pw, eyeN.cuda())):
        assert torch.equal(dx.cpu().to(torch.float64), wantb), fam


@pytest.mark.parametrize("M,act", [(1, "f16"), (4, "f32"), (100, "bf16"), (100, "f16"), (100, "f32")])
def test_scale_times_two_is_bitwise(M, act):
    q = lib()
    case = make_linear(M, 512, 256, 128, act, "f16", seed=9, fwd=True, bwd=True)
    w = case.w
    pw1 = pack(q, w)
    pw2 = q.pack(w.codes.cuda(), (w.scales * 2).cuda(), w.group_size)
    for fam, y1 in each_route(q, lambda: q.linear_fwd(pw1, case.x.cuda())):
        with (q.forced_route(fam) if fam != "auto" else _null()):
            y2 = q.linear_fwd(pw2, case.x.cuda())
        assert torch.equal(y2, 2 * y1), fam
    for fam, d1 in each_route(q, lambda: q.linear_bwd_input(pw1, case.d_out.cuda())):
        with (q.forced_route(fam) if fam != "auto" else _null()):
            d2 = q.linear_bwd_input(pw2, case.d_out.cuda())
        assert torch.equal(d2, 2 * d1), fam


class _null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


@pytest.mark.parametrize("M,act", [(3, "f32"), (64, "f16"), (96, "bf16"), (130, "f32")])
def test_adjoint_identity(M, act):
    q = lib()
    case = make_linear(M, 384, 512, 128, act, "f16", seed=13, fwd=True, bwd=True)
    pw = pack(q, case.w)
    y = q.linear_fwd(pw, dev(case.x)).cpu().double()
    dx = q.linear_bwd_input(pw, dev(case.d_out)).cpu().double()
    lhs = float((case.d_out.double() * y).sum())
    rhs = float((dx * case.x.double()).sum())
    _, rf = oracle_fwd(case.x, case.w)
    T = float((case.d_out.double().abs().numpy() * rf).sum())
    tol = TOL[case.x.dtype]
    assert abs(lhs - rhs) <= 2 * tol * T, (lhs, rhs, T)


def test_one_packed_weight_serves_every_M():
    """Shrink and regrow M on one packed buffer (no re-pack between calls)."""
    q = lib()
    K, N, gs = 1024, 768, 64
    gen = torch.Generator().manual_seed(21)
    w = Weight(draw_codes(gen, N, K), (torch.rand(K // gs, N, generator=gen) * 0.02 + 0.002).half(), gs)
    pw = pack(q, w)
    for M in (512, 128, 508, 1, 9, 512):
        for act in ("f16", "bf16", "f32"):
            x = draw_activation(torch.Generator().manual_seed(M), M, K, act)
            y = q.linear_fwd(pw, x.cuda())
            ref, norm = oracle_fwd(x, w)
            assert_within(y, ref, norm, TOL[x.dtype], f"fwd M={M} {act}")
            g = draw_activation(torch.Generator().manual_seed(M + 1), M, N, act)
            dx = q.linear_bwd_input(pw, g.cuda())
            ref, norm = oracle_bwd(g, w)
            assert_within(dx, ref, norm, TOL[g.dtype], f"bwd M={M} {act}")
