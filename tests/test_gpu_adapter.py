"""GPU parity of the adapter step around the frozen base (low-rank adapter forward and
gradients, AdamW) against the oracle.

Rounding bounds (u = 2^-24; R is the oracle's normaliser, the sum of |products| behind each
output).  The frozen-weight term keeps the forward's / input gradient's own tolerance TOL[dtype].
The low-rank terms run in fp32 with a fixed summation order:
  * t = x A^T, u = d_out B over C columns: each lane adds at most 32 products in order, a
    64-lane tree adds 6 levels and the column chunks (at most C / 256) are added in order:
    a chain of at most C / 256 + 40 roundings;
  * y += alpha t B^T, d_x += alpha u A: r products in order, then one fma: r + 2 more (the
    one-split forward adds them in its GEMM epilogue on fp32 MFMAs: alpha t rounded once, then r
    products onto the accumulator, r + 1);
  * d_A = alpha u^T x, d_B = alpha d_out^T t: each wave adds a quarter of a slab's rows in
    order, the 4 waves are added in order, then at most 64 slabs and alpha: at most
    M / 4 + 70 roundings, on top of the error of u or t.
So |gpu - oracle| <= max(TOL, n u) R with n the chain length of that output.  With a weight of
code 8 everywhere the frozen term is exactly zero and the low-rank bound applies alone, in
every activation dtype.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from synthetic_inputs import ADAPTER_ALPHA, make_adamw_state, make_adapter, make_workload
from tests.gpu_helpers import THREADS, TOL, assert_within, dev, lib, pack, sample_rows

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def contract_chain(C):
    return C / 256 + 40


def column_chain(M):
    return math.ceil(M / 4) + 70


def tol_y(case, r):
    return max(TOL[case.x.dtype], (contract_chain(case.w.K) + r + 2) * U)


def tol_dx(case, r):
    return max(TOL[case.x.dtype], (contract_chain(case.w.N) + r + 2) * U)


def tol_dA(case):
    return (contract_chain(case.w.N) + column_chain(case.M)) * U


def tol_dB(case):
    return (contract_chain(case.w.K) + column_chain(case.M)) * U


def t_norm(x, A):
    """sum_k |x[m,k]| |A[j,k]| in fp64 (the normaliser of t)."""
    return np.abs(x.double().numpy()) @ np.abs(A.double().numpy()).T


def run_adapter(q, case, alpha, pw=None):
    pw = pack(q, case.w) if pw is None else pw
    x, d = dev(case.x), dev(case.d_out)
    A, B = dev(case.A), dev(case.B)
    y, t = q.adapter_fwd(pw, x, A, B, alpha)
    dx, dA, dB = q.adapter_bwd(pw, x, d, A, B, alpha, t)
    torch.cuda.synchronize()
    return y, t, dx, dA, dB


CASES = [
    # M, N, K, gs, act, scale dtype, rank, alpha
    (1, 64, 128, 32, "f32", "f16", 1, 1.0),
    (4, 256, 512, 64, "bf16", "f16", 4, 2.0),
    (37, 300, 256, 32, "f16", "f32", 5, -0.5),       # ragged N, rank inside the 8 bucket
    (130, 512, 1024, 128, "bf16", "f16", 16, 0.25),
    (70, 128, 192, 64, "f32", "f16", 33, 1.0),       # rank 33 in the 64 bucket
    (200, 264, 384, 64, "f16", "f16", 64, 0.125),    # the largest rank
    (1000, 256, 512, 32, "bf16", "f16", 8, 1.0),     # d_A and d_B over several row slabs
    (9, 96, 2048, 32, "f32", "f32", 17, 3.0),
    (33, 257, 256, 32, "f16", "f16", 3, 1.0),       # odd N: rows of y, d_out and B^T without whole quads
]


@pytest.mark.parametrize("M,N,K,gs,act,sdt,r,alpha", CASES)
def test_adapter_parity(M, N, K, gs, act, sdt, r, alpha):
    q = lib()
    case = make_adapter(M, K, N, gs, act, sdt, r, seed=M + N + r)
    print(f"adapter M={M} N={N} K={K} gs={gs} {act}/{sdt} r={r}", flush=True)
    y, t, dx, dA, dB = run_adapter(q, case, alpha)
    w = case.w
    oy, ot, ry = O.lora_fwd(case.x, w.codes, w.scales, gs, case.A, case.B, alpha, threads=THREADS)
    assert_within(y, oy, ry, tol_y(case, r), "y")
    assert_within(t, ot, t_norm(case.x, case.A), contract_chain(K) * U, "t")
    g = O.lora_bwd(case.x, case.d_out, w.codes, w.scales, gs, case.A, case.B, alpha, threads=THREADS)
    assert_within(dx, g["dx"], g["r_dx"], tol_dx(case, r), "d_x")
    assert_within(dA, g["dA"], g["r_dA"], tol_dA(case), "d_A")
    assert_within(dB, g["dB"], g["r_dB"], tol_dB(case), "d_B")


# Forward shapes whose GEMM plans one K split (K = 128 is one chunk) on the exact-code group route
# with 128-column chunks (bf16 x, fp16 scales, gs 128): the low-rank term goes through the GEMM's
# epilogue.  Rows past M, columns past N (inside a wave and whole idle waves), odd rank, rank 1
# and the largest rank.
EPI_CASES = [
    # M, N, K, rank, alpha
    (70, 300, 128, 33, 1.0),
    (130, 520, 128, 64, -0.5),
    (257, 96, 128, 1, 2.0),
    (64, 256, 128, 16, 0.25),
]


@pytest.mark.parametrize("M,N,K,r,alpha", EPI_CASES)
def test_adapter_fwd_epilogue(M, N, K, r, alpha):
    q = lib()
    case = make_adapter(M, K, N, 128, "bf16", "f16", r, seed=7 * M + N + r)
    print(f"adapter forward epilogue M={M} N={N} K={K} r={r}", flush=True)
    pw = pack(q, case.w)
    pl = q.plan(q.OP_FWD, pw, M, case.x.dtype)
    assert pl["route"] == "gemm_group" and pl["splits"] == 1, pl
    y, t = q.adapter_fwd(pw, dev(case.x), dev(case.A), dev(case.B), alpha)
    torch.cuda.synchronize()
    w = case.w
    oy, ot, ry = O.lora_fwd(case.x, w.codes, w.scales, 128, case.A, case.B, alpha, threads=THREADS)
    assert_within(y, oy, ry, tol_y(case, r), "y")
    assert_within(t, ot, t_norm(case.x, case.A), contract_chain(K) * U, "t")


def _offset_copy(t):
    """t on the GPU, one element past the start of its allocation (misaligned for vector loads)."""
    big = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    v = big[1:].view(t.shape)
    v.copy_(t)
    return v


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_adapter_unaligned_operands(act):
    """x, d_out, A, B and t one element off their allocations: every low-rank kernel takes its
    element-wise path, with the same results as the oracle."""
    q = lib()
    M, N, K, r, alpha = 70, 320, 512, 12, -1.25
    case = make_adapter(M, K, N, 64, act, "f16", r, seed=90 + len(act))
    pw = pack(q, case.w)
    x, d = _offset_copy(case.x), _offset_copy(case.d_out)
    A, B = _offset_copy(case.A), _offset_copy(case.B)
    y, t = q.adapter_fwd(pw, x, A, B, alpha)
    t_off = _offset_copy(t)
    dx, dA, dB = q.adapter_bwd(pw, x, d, A, B, alpha, t_off)
    torch.cuda.synchronize()
    w = case.w
    oy, ot, ry = O.lora_fwd(case.x, w.codes, w.scales, 64, case.A, case.B, alpha, threads=THREADS)
    assert_within(y, oy, ry, tol_y(case, r), "y")
    assert_within(t, ot, t_norm(case.x, case.A), contract_chain(K) * U, "t")
    g = O.lora_bwd(case.x, case.d_out, w.codes, w.scales, 64, case.A, case.B, alpha, threads=THREADS)
    assert_within(dx, g["dx"], g["r_dx"], tol_dx(case, r), "d_x")
    assert_within(dA, g["dA"], g["r_dA"], tol_dA(case), "d_A")
    assert_within(dB, g["dB"], g["r_dB"], tol_dB(case), "d_B")


def test_cases_cover_both_backward_paths():
    """When the input gradient of the frozen term ends in a split reduction (MFMA routes with K
    splits), that launch also adds alpha u A; otherwise (small M, one split) a separate launch
    does.  The parity cases above run both."""
    q = lib()
    fused = set()
    for M, N, K, gs, act, sdt, r, alpha in CASES:
        case = make_adapter(M, K, N, gs, act, sdt, r, seed=0)
        pl = q.plan(q.OP_BWD_INPUT, pack(q, case.w), M, case.x.dtype)
        fused.add(pl["route"] in ("bwd_split", "bwd_bsplit", "bwd_fold") and pl["splits"] > 1)
    assert fused == {True, False}


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,N,K,r", [(3, 128, 256, 8), (77, 320, 640, 16), (260, 192, 1088, 64)])
def test_adapter_terms_alone(act, M, N, K, r):
    """A weight of code 8 everywhere dequantises to zero: the frozen term is exactly 0 and the
    outputs are the low-rank terms, held to their own fp32 bound in every dtype."""
    q = lib()
    case = make_adapter(M, K, N, 64, act, "f16", r, seed=7 * M + r)
    case.w.codes.fill_(8)
    print(f"adapter terms alone M={M} N={N} K={K} r={r} {act}", flush=True)
    y, t, dx, dA, dB = run_adapter(q, case, -0.75)
    w = case.w
    oy, ot, ry = O.lora_fwd(case.x, w.codes, w.scales, 64, case.A, case.B, -0.75, threads=THREADS)
    assert_within(y, oy, ry, (contract_chain(K) + r + 2) * U, "y")
    g = O.lora_bwd(case.x, case.d_out, w.codes, w.scales, 64, case.A, case.B, -0.75, threads=THREADS)
    assert_within(dx, g["dx"], g["r_dx"], (contract_chain(N) + r + 2) * U, "d_x")
    assert_within(dA, g["dA"], g["r_dA"], tol_dA(case), "d_A")
    assert_within(dB, g["dB"], g["r_dB"], tol_dB(case), "d_B")


@pytest.mark.parametrize("M,N,K,act", [(1, 256, 512, "f16"), (64, 512, 1024, "bf16"), (300, 384, 256, "f32")])
def test_zero_factors_leave_the_base_bit_for_bit(M, N, K, act):
    """B = 0: y is the plain forward bit for bit.  A = 0: t = 0, y is the plain forward, d_x the
    plain input gradient and d_B = 0, bit for bit.  A = B = 0: d_A = 0 as well."""
    q = lib()
    case = make_adapter(M, K, N, 32, act, "f16", 8, seed=M)
    pw = pack(q, case.w)
    x, d = dev(case.x), dev(case.d_out)
    base_y = q.linear_fwd(pw, x)
    base_dx = q.linear_bwd_input(pw, d)
    A, B = dev(case.A), dev(case.B)
    zA, zB = torch.zeros_like(A), torch.zeros_like(B)
    y, t = q.adapter_fwd(pw, x, A, zB, 1.5)
    assert torch.equal(y, base_y)
    y, t = q.adapter_fwd(pw, x, zA, B, 1.5)
    assert torch.equal(y, base_y) and not torch.any(t)
    dx, dA, dB = q.adapter_bwd(pw, x, d, zA, B, 1.5, t)
    assert torch.equal(dx, base_dx) and not torch.any(dB)
    dx, dA, dB = q.adapter_bwd(pw, x, d, zA, zB, 1.5, t)
    assert torch.equal(dx, base_dx) and not torch.any(dA) and not torch.any(dB)


def test_adapter_is_deterministic():
    """Two runs of the same step give the same bits (every sum has one fixed order)."""
    q = lib()
    case = make_adapter(500, 384, 768, 64, "bf16", "f16", 16, seed=3)
    pw = pack(q, case.w)
    first = run_adapter(q, case, 0.5, pw)
    second = run_adapter(q, case, 0.5, pw)
    for a, b, name in zip(first, second, ("y", "t", "d_x", "d_A", "d_B")):
        assert torch.equal(a, b), name


def test_adapter_prefill_size():
    """The MLP up projection's adapter step at its prefill size (M=512, K=2048, N=8192, gs=128,
    bf16, rank 16), as the benchmark launches it: y and d_x on sampled rows against the full
    oracle, t, d_A and d_B (every element) against the oracle's adapter term alone."""
    q = lib()
    case = make_workload("adapter")
    w, r, a = case.w, case.A.shape[0], ADAPTER_ALPHA
    print("adapter prefill M=512 K=2048 N=8192 r=16", flush=True)
    y, t, dx, dA, dB = run_adapter(q, case, a)
    rows = sample_rows(case.M)
    xs, ds = case.x[rows].contiguous(), case.d_out[rows].contiguous()
    oy, _, ry = O.lora_fwd(xs, w.codes, w.scales, w.group_size, case.A, case.B, a, threads=THREADS)
    assert_within(y, oy, ry, tol_y(case, r), "y", rows=rows)
    _, ot, _ = O.lora_fwd(case.x, None, None, w.group_size, case.A, case.B, a)
    assert_within(t, ot, t_norm(case.x, case.A), contract_chain(w.K) * U, "t")
    g = O.lora_bwd(xs, ds, w.codes, w.scales, w.group_size, case.A, case.B, a, threads=THREADS)
    assert_within(dx, g["dx"], g["r_dx"], tol_dx(case, r), "d_x", rows=rows)
    g = O.lora_bwd(case.x, case.d_out, None, None, w.group_size, case.A, case.B, a)
    assert_within(dA, g["dA"], g["r_dA"], tol_dA(case), "d_A")
    assert_within(dB, g["dB"], g["r_dB"], tol_dB(case), "d_B")


# ---- AdamW -----------------------------------------------------------------------------------

def f32(values):
    """The hyperparameters as the call receives them (fp32 fields), given to the oracle alike."""
    return [float(np.float32(v)) for v in values]


HYPER = [
    # lr, beta1, beta2, eps, weight decay
    (1e-3, 0.9, 0.999, 1e-8, 0.01),
    (3e-2, 0.8, 0.99, 1e-6, 0.1),
    (5e-4, 0.0, 0.9999, 1e-8, 0.0),
]


def check_adamw(state_in, got, ref, lr, b1, b2, eps, step, label):
    """The moments within 3 u of the sum of their two terms' magnitudes (b m + (1 - b) g, no
    cancellation bound needed beyond that); p within 12 u of |p| plus the update's magnitude
    taken with that first-moment magnitude (decay, two roundings of the moments, square root,
    bias factors, fma and division each add at most one or two)."""
    p0, g0, m0, v0 = (t.double().numpy() for t in state_in)
    gp, gm, gv = (t.cpu().double().numpy() for t in got)
    rp, rm, rv = ref
    mag_m = np.abs(b1 * m0) + np.abs((1 - b1) * g0)
    mag_v = np.abs(b2 * v0) + (1 - b2) * g0 * g0
    upd = lr * (mag_m / (1 - b1 ** step)) / (np.sqrt(rv / (1 - b2 ** step)) + eps)
    for name, g_, r_, bound in (("p", gp, rp, 12 * U * (np.abs(p0) + upd)),
                                ("m", gm, rm, 3 * U * mag_m),
                                ("v", gv, rv, 3 * U * mag_v)):
        err = np.abs(g_ - r_)
        bad = err > bound
        assert not np.any(bad), (label, name, int(bad.sum()), float(np.max(err - bound)))


@pytest.mark.parametrize("n,offset", [(1, 0), (3, 0), (4096, 0), (4099, 0), (4096, 1), (4 * 256 * 2048 * 2 + 4, 0)])
@pytest.mark.parametrize("hyper", range(len(HYPER)))
def test_adamw_parity(n, offset, hyper):
    """Several steps in a row, each checked against the oracle's step from the GPU's previous
    state; offset 1 takes views 4 bytes into larger tensors (the per-element path), n % 4 != 0
    likewise, and the largest n runs the grid-stride loop."""
    q = lib()
    lr, b1, b2, eps, wd = f32(HYPER[hyper])
    p, gr, m, v = make_adamw_state(n, 1, seed=n + hyper)
    gr[:: 7] = 0.0                                      # zero gradients: only the decay moves p
    bufs = [torch.zeros(n + offset, device="cuda") for _ in range(4)]
    P, G, Mm, V = (b[offset:] for b in bufs)
    for dst, src in zip((P, G, Mm, V), (p, gr, m, v)):
        dst.copy_(src)
    print(f"adamw n={n} offset={offset} hyper={hyper}", flush=True)
    for step in (1, 2, 3, 10):
        state = [t.cpu() for t in (P, G, Mm, V)]
        q.adamw_step(P, G, Mm, V, step, lr, b1, b2, eps, wd)
        torch.cuda.synchronize()
        ref = O.adamw(*state, lr, b1, b2, eps, wd, step)
        check_adamw(state, (P, Mm, V), ref, lr, b1, b2, eps, step, f"step {step}")
        G.copy_(torch.randn(n, generator=torch.Generator().manual_seed(step)) * 0.1)


def test_adamw_from_random_moments():
    """A later step (step 250) from nonzero moments."""
    q = lib()
    p, gr, m, v = make_adamw_state(10000, 250, seed=5)
    P, G, Mm, V = (dev(t) for t in (p, gr, m, v))
    lr, b1, b2, eps, wd = f32((1e-3, 0.9, 0.999, 1e-8, 0.05))
    q.adamw_step(P, G, Mm, V, 250, lr, b1, b2, eps, wd)
    torch.cuda.synchronize()
    ref = O.adamw(p, gr, m, v, lr, b1, b2, eps, wd, 250)
    check_adamw((p, gr, m, v), (P, Mm, V), ref, lr, b1, b2, eps, 250, "step 250")
