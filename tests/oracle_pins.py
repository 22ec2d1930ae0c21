"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` takes a loaded ``oracle.oracle.Oracle`` and raises AssertionError if
the oracle disagrees with the fact it pins.  test_oracle.py runs them on the real
oracle; test_oracle_mutants.py runs them on copies of oracle.c with one planted
mistake each and checks that some pin fails.

The facts:
  * hand-worked examples (tests/golden) of the definition on the pages;
  * the code -> value table of the dequantisation formula (tests/golden);
  * IEEE decoding of every fp16 / bf16 bit pattern, against numpy and torch;
  * pure-Python brute force on tiny inputs (same summation order: bitwise);
  * numpy fp64 matmul of an explicitly dequantised matrix (<= 1e-12 R);
  * code 8 contributes exactly zero; outputs are linear in the scales;
  * the adjoint identity <d_out, fwd(x)> = <bwd(d_out), x>;
  * one-hot closed forms that read back every code and scale address;
  * QKV equals three forwards; thread-count invariance; R >= |y| with equality
    when every term has one sign;
  * the embedding gather equals rows of the numpy-dequantised matrix and the
    backward of a one-hot output gradient; ids outside [0, N) give zero rows;
  * dq8ca (per-row int8 activations): hand-worked rows (tests/golden); PyTorch's own
    quantizer reproduces the codes from the oracle's scale and zero point; nearest-grid,
    span, zero and monotonicity properties; on-grid rows give exactly the plain forward;
    the linear against a numpy matmul of the dequantised rows.
  * the adapter step (a low-rank adapter beside the frozen weight, and AdamW): zero
    adapters reduce to the plain forward and input gradient bit for bit; a numpy matmul of
    the dense matrices; the adjoint identities that define the three gradients (the output
    is linear in x, in A and in B separately); PyTorch's own torch.optim.AdamW on the same
    state; closed forms of a first step and of a decay-only step.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import torch

from synthetic_inputs import DTYPES, Weight, draw_activation, draw_codes, draw_scales
from tests.conftest import ROOT, load_golden

ACT_DTYPES = ("f32", "f16", "bf16")
SCALE_DTYPES = ("f32", "f16")


def _t(rows, dtype):
    return torch.tensor(rows, dtype=torch.float64).to(DTYPES[dtype]).contiguous()


def _case(seed, M, N, K, gs, act="f32", sdt="f32", s_lo=0.005, s_hi=0.02, sigma=1.0):
    g = torch.Generator().manual_seed(seed)
    x = draw_activation(g, M, K, act, sigma)
    d_out = draw_activation(g, M, N, act, sigma)
    codes = draw_codes(g, N, K)
    scales = draw_scales(g, K // gs, N, sdt, s_lo, s_hi)
    return x, d_out, codes, scales


def _dense(codes, scales, gs):
    """Explicit dequantised [N, K] float64 matrix built with numpy (a library route)."""
    c = codes.numpy().astype(np.float64) - 8.0
    s = scales.to(torch.float64).numpy()            # [G, N]
    return c * np.repeat(s.T, gs, axis=1)           # [N, K]


# ---------------------------------------------------------------------------------------------
def pin_worked_example(o):
    g = load_golden("worked_example_4x2.txt")
    gs = int(g["group_size"])
    codes = torch.tensor(g["codes"], dtype=torch.uint8)
    for act, sdt in itertools.product(ACT_DTYPES, SCALE_DTYPES):
        scales = _t(g["scales"], sdt)
        y, ry = o.linear_fwd(_t(g["x"], act), codes, scales, gs)
        assert np.array_equal(y, np.array(g["y"])), (act, sdt, y)
        assert np.array_equal(ry, np.array(g["y_norm"])), (act, sdt, ry)
        dx, rdx = o.linear_bwd_input(_t(g["d_out"], act), codes, scales, gs)
        assert np.array_equal(dx, np.array(g["d_x"])), (act, sdt, dx)
        assert np.array_equal(rdx, np.array(g["d_x_norm"])), (act, sdt, rdx)
    ids = torch.tensor([int(v) for v in g["ids"][0]], dtype=torch.int64)
    for sdt in SCALE_DTYPES:
        e = o.embedding(ids, codes, _t(g["scales"], sdt), gs)
        assert np.array_equal(e, np.array(g["embedding"])), (sdt, e)


def pin_code_table(o):
    pairs = []
    with open(os.path.join(ROOT, "tests", "golden", "dequant_codes.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                pairs.append((int(c), float(v)))
    assert len(pairs) == 16
    codes = torch.tensor([[c for c, _ in pairs]], dtype=torch.uint8)     # N=1, K=16
    for sdt in SCALE_DTYPES:
        scales = torch.ones(1, 1, dtype=DTYPES[sdt])                      # gs = 16, one group
        for k, (_, v) in enumerate(pairs):
            assert o.dequant(codes, scales, 16, 0, k) == v
        half = torch.full((1, 1), 0.5, dtype=DTYPES[sdt])
        for k, (_, v) in enumerate(pairs):
            assert o.dequant(codes, half, 16, 0, k) == v * 0.5


def pin_decoders(o):
    bits = np.arange(65536, dtype=np.uint16)
    ref16 = bits.view(np.float16).astype(np.float64)
    refbf = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for b in range(0, 65536, 1):
        v = o.f16_to_f64(b)
        r = ref16[b]
        assert (v == r) or (math.isnan(v) and math.isnan(r)), ("f16", b, v, r)
        v = o.bf16_to_f64(b)
        r = refbf[b]
        assert (v == r) or (math.isnan(v) and math.isnan(r)), ("bf16", b, v, r)
    rng = np.random.default_rng(1)
    specials = np.array([0, 1, 0x7FFFFF, 0x800000, 0x3F800000, 0x7F7FFFFF, 0x7F800000,
                         0x80000001, 0xFF800000, 0x00400000], dtype=np.uint32)
    sample = np.concatenate([specials, rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32)])
    with np.errstate(invalid="ignore"):
        ref32 = sample.view(np.float32).astype(np.float64)
    for b, r in zip(sample.tolist(), ref32.tolist()):
        v = o.f32_to_f64(b)
        assert (v == r) or (math.isnan(v) and math.isnan(r)), ("f32", b, v, r)


def pin_brute_force(o):
    """Pure-Python loops on tiny inputs; k (resp. n) ascending, so equality is bitwise."""
    seed = 10
    for (M, N, K, gs) in [(1, 1, 8, 8), (2, 3, 8, 2), (3, 5, 12, 4), (2, 4, 16, 1), (1, 3, 24, 8),
                          (4, 2, 6, 3)]:
        for act, sdt in [("f32", "f32"), ("f16", "f16"), ("bf16", "f16"), ("f32", "f16")]:
            seed += 1
            x, d_out, codes, scales = _case(seed, M, N, K, gs, act, sdt)
            xs, ds = x.tolist(), d_out.tolist()
            cs, ss = codes.tolist(), scales.tolist()
            D = [[(cs[n][k] - 8) * ss[k // gs][n] for k in range(K)] for n in range(N)]
            y, ry = o.linear_fwd(x, codes, scales, gs)
            dx, rdx = o.linear_bwd_input(d_out, codes, scales, gs)
            for m in range(M):
                for n in range(N):
                    acc = 0.0
                    nrm = 0.0
                    for k in range(K):
                        acc += xs[m][k] * D[n][k]
                        nrm += abs(xs[m][k]) * abs(D[n][k])
                    assert y[m, n] == acc and ry[m, n] == nrm, (M, N, K, gs, act, sdt, m, n)
                for k in range(K):
                    acc = 0.0
                    nrm = 0.0
                    for n in range(N):
                        acc += ds[m][n] * D[n][k]
                        nrm += abs(ds[m][n]) * abs(D[n][k])
                    assert dx[m, k] == acc and rdx[m, k] == nrm, (M, N, K, gs, act, sdt, m, k)


def pin_numpy_matmul(o):
    for seed, (M, N, K, gs, act, sdt) in enumerate([(7, 33, 96, 32, "f16", "f16"),
                                                    (5, 40, 128, 16, "bf16", "f16"),
                                                    (3, 24, 64, 64, "f32", "f32")]):
        x, d_out, codes, scales = _case(100 + seed, M, N, K, gs, act, sdt)
        D = _dense(codes, scales, gs)
        xd = x.to(torch.float64).numpy()
        dd = d_out.to(torch.float64).numpy()
        y, ry = o.linear_fwd(x, codes, scales, gs)
        assert np.all(np.abs(y - xd @ D.T) <= 1e-12 * ry + 1e-300)
        assert np.allclose(ry, np.abs(xd) @ np.abs(D).T, rtol=1e-12, atol=0)
        dx, rdx = o.linear_bwd_input(d_out, codes, scales, gs)
        assert np.all(np.abs(dx - dd @ D) <= 1e-12 * rdx + 1e-300)
        assert np.allclose(rdx, np.abs(dd) @ np.abs(D), rtol=1e-12, atol=0)


def pin_code8_zero(o):
    x, d_out, codes, scales = _case(200, 3, 6, 32, 8, "f32", "f16")
    eights = torch.full_like(codes, 8)
    y, ry = o.linear_fwd(x, eights, scales, 8)
    assert np.all(y == 0) and np.all(ry == 0)
    dx, rdx = o.linear_bwd_input(d_out, eights, scales, 8)
    assert np.all(dx == 0) and np.all(rdx == 0)
    # a column of code 8 makes y blind to that activation column
    c2 = codes.clone()
    c2[:, 5] = 8
    y0, _ = o.linear_fwd(x, c2, scales, 8)
    x2 = x.clone()
    x2[:, 5] = 1000.0
    y1, _ = o.linear_fwd(x2, c2, scales, 8)
    assert np.array_equal(y0, y1)
    # a row of code 8 makes d_x blind to that output-gradient column
    c3 = codes.clone()
    c3[2, :] = 8
    dx0, _ = o.linear_bwd_input(d_out, c3, scales, 8)
    d2 = d_out.clone()
    d2[:, 2] = -777.0
    dx1, _ = o.linear_bwd_input(d2, c3, scales, 8)
    assert np.array_equal(dx0, dx1)
    # and a code other than 8 is not blind
    y2, _ = o.linear_fwd(x2, codes, scales, 8)
    assert not np.array_equal(y2, o.linear_fwd(x, codes, scales, 8)[0])


def pin_scale_linearity(o):
    x, d_out, codes, scales = _case(300, 4, 8, 64, 16, "bf16", "f16")
    y, ry = o.linear_fwd(x, codes, scales, 16)
    dx, rdx = o.linear_bwd_input(d_out, codes, scales, 16)
    for p in (2.0, 0.5, 8.0):
        s2 = (scales.to(torch.float64) * p).to(scales.dtype)
        y2, ry2 = o.linear_fwd(x, codes, s2, 16)
        assert np.array_equal(y2, y * p) and np.array_equal(ry2, ry * p)
        dx2, rdx2 = o.linear_bwd_input(d_out, codes, s2, 16)
        assert np.array_equal(dx2, dx * p) and np.array_equal(rdx2, rdx * p)
    # additivity: s = s_a + s_b with both parts exact in fp32
    sa = (scales.to(torch.float32) * 0.75).contiguous()
    sb = (scales.to(torch.float32) * 0.25).contiguous()
    s_sum = (sa + sb).contiguous()
    ya, ra = o.linear_fwd(x, codes, sa, 16)
    yb, _ = o.linear_fwd(x, codes, sb, 16)
    ys, rs = o.linear_fwd(x, codes, s_sum, 16)
    assert np.all(np.abs(ys - (ya + yb)) <= 1e-12 * rs)


def pin_adjoint(o):
    for seed, (M, N, K, gs, act) in enumerate([(3, 40, 64, 16, "f32"), (6, 17, 48, 8, "f16"),
                                               (2, 64, 32, 32, "bf16")]):
        x, d_out, codes, scales = _case(400 + seed, M, N, K, gs, act, "f16")
        y, ry = o.linear_fwd(x, codes, scales, gs)
        dx, _ = o.linear_bwd_input(d_out, codes, scales, gs)
        xd = x.to(torch.float64).numpy()
        dd = d_out.to(torch.float64).numpy()
        lhs = float(np.sum(dd * y))
        rhs = float(np.sum(dx * xd))
        T = float(np.sum(np.abs(dd) * ry))
        assert abs(lhs - rhs) <= 1e-12 * T, (lhs, rhs, T)


def pin_one_hot(o):
    """x = identity reads back every dequantised element: y[m, n] = (code[n, m] - 8) * scale."""
    N, K, gs = 12, 48, 8
    g = torch.Generator().manual_seed(500)
    codes = draw_codes(g, N, K)
    eye = torch.eye(K, dtype=torch.float32)
    ones = torch.ones(K // gs, N, dtype=torch.float16)
    y, _ = o.linear_fwd(eye, codes, ones, gs)
    assert np.array_equal(y, (codes.numpy().astype(np.float64) - 8).T)
    # distinct power-of-two scale per (group, n): pins the scale's row and column index
    expo = torch.tensor([[((gi * N + n) % 13) - 6 for n in range(N)] for gi in range(K // gs)],
                        dtype=torch.float64)
    pscales = torch.pow(2.0, expo).to(torch.float16)
    y, _ = o.linear_fwd(eye, codes, pscales, gs)
    for m in range(K):
        for n in range(N):
            want = (int(codes[n, m]) - 8) * 2.0 ** (((m // gs) * N + n) % 13 - 6)
            assert y[m, n] == want, (m, n, y[m, n], want)
    # one-hot output gradients read back rows: d_x[m, k] = dequant(W[m, k])
    eyeN = torch.eye(N, dtype=torch.bfloat16)
    dx, _ = o.linear_bwd_input(eyeN, codes, pscales, gs)
    for m in range(N):
        for k in range(K):
            want = (int(codes[m, k]) - 8) * 2.0 ** (((k // gs) * N + m) % 13 - 6)
            assert dx[m, k] == want, (m, k, dx[m, k], want)


def pin_qkv(o):
    g = torch.Generator().manual_seed(600)
    x = draw_activation(g, 5, 64, "f16")
    ws = [Weight(draw_codes(g, n, 64), draw_scales(g, 2, n, "f16", 0.002, 0.02), 32) for n in (32, 8, 8)]
    outs = o.qkv(x, ws)
    for (yo, ro), w in zip(outs, ws):
        y, r = o.linear_fwd(x, w.codes, w.scales, 32)
        assert np.array_equal(yo, y) and np.array_equal(ro, r)
    # the triple equals one forward over the row-stacked weight
    cat_codes = torch.cat([w.codes for w in ws], dim=0)
    cat_scales = torch.cat([w.scales for w in ws], dim=1).contiguous()
    y, _ = o.linear_fwd(x, cat_codes, cat_scales, 32)
    assert np.array_equal(np.concatenate([yo for yo, _ in outs], axis=1), y)


def pin_threads(o):
    x, d_out, codes, scales = _case(700, 9, 37, 64, 16, "f16", "f16")
    a = o.linear_fwd(x, codes, scales, 16, threads=1)
    b = o.linear_fwd(x, codes, scales, 16, threads=3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    a = o.linear_bwd_input(d_out, codes, scales, 16, threads=1)
    b = o.linear_bwd_input(d_out, codes, scales, 16, threads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def pin_normaliser(o):
    x, d_out, codes, scales = _case(800, 4, 10, 32, 8, "f32", "f32")
    y, ry = o.linear_fwd(x, codes, scales, 8)
    assert np.all(ry >= np.abs(y))
    dx, rdx = o.linear_bwd_input(d_out, codes, scales, 8)
    assert np.all(rdx >= np.abs(dx))
    # one sign everywhere: x >= 0, code >= 8, scale > 0 gives R == y exactly
    xp = x.abs().contiguous()
    cp = (codes % 8 + 8).to(torch.uint8).contiguous()
    y, ry = o.linear_fwd(xp, cp, scales, 8)
    assert np.array_equal(y, ry)
    dp = d_out.abs().contiguous()
    dx, rdx = o.linear_bwd_input(dp, cp, scales, 8)
    assert np.array_equal(dx, rdx)


def pin_embedding(o):
    """Row gather: rows of the numpy-dequantised matrix, the power-of-two address pin, the
    one-hot backward, code 8 giving zero rows, and rows of zeros for ids outside [0, N)."""
    N, K, gs = 11, 64, 16
    g = torch.Generator().manual_seed(900)
    codes = draw_codes(g, N, K)
    scales = draw_scales(g, K // gs, N, "f16", 0.002, 0.02)
    ids = torch.tensor([3, 0, 10, 3, 7, 1, 9, 2], dtype=torch.int64)
    e = o.embedding(ids, codes, scales, gs)
    assert e.shape == (len(ids), K)
    assert np.array_equal(e, _dense(codes, scales, gs)[ids.numpy()])
    # distinct power-of-two scale per (group, n) and distinct codes: pins row, group and column
    expo = torch.tensor([[((gi * N + n) % 13) - 6 for n in range(N)] for gi in range(K // gs)],
                        dtype=torch.float64)
    pscales = torch.pow(2.0, expo).to(torch.float16)
    e = o.embedding(ids, codes, pscales, gs)
    for t, n in enumerate(ids.tolist()):
        for k in range(K):
            assert e[t, k] == (int(codes[n, k]) - 8) * 2.0 ** (((k // gs) * N + n) % 13 - 6), (t, k)
    # one-hot output gradient: the backward reads back the same rows
    onehot = torch.zeros(len(ids), N, dtype=torch.float32)
    onehot[torch.arange(len(ids)), ids] = 1.0
    dx, _ = o.linear_bwd_input(onehot, codes, pscales, gs)
    assert np.array_equal(e, dx)
    # code 8 is exactly zero
    eight = torch.full((N, K), 8, dtype=torch.uint8)
    assert np.array_equal(o.embedding(ids, eight, scales, gs), np.zeros((len(ids), K)))
    # ids outside [0, N) give zero rows; valid ids beside them are unaffected
    mixed = torch.tensor([-1, 4, N, 2**40, -2**40], dtype=torch.int64)
    e = o.embedding(mixed, codes, scales, gs)
    assert np.array_equal(e[[0, 2, 3, 4]], np.zeros((4, K)))
    assert np.array_equal(e[1], _dense(codes, scales, gs)[4])
    # no ids: an empty result
    assert o.embedding(torch.zeros(0, dtype=torch.int64), codes, scales, gs).shape == (0, K)


def pin_dq8ca_golden(o):
    g = load_golden("dq8ca_rows.txt")
    for row in "abcd":
        x = [float(v) for v in g[f"{row}_x"][0]]
        acts = ("f32",) if row == "a" else ACT_DTYPES      # row a holds 0.3, exact in fp32 only
        for act in acts:
            q, scale, zp = o.dq8ca_quantize(_t([x], act))
            assert q[0].tolist() == [int(v) for v in g[f"{row}_q"][0]], (row, act, q)
            assert float(scale[0]) == g[f"{row}_scale"], (row, act, scale)
            assert int(zp[0]) == int(g[f"{row}_zp"]), (row, act, zp)


def _dq8ca_rows(seed):
    """Rows of several magnitudes and sign mixes (some all positive, all negative, with zeros)."""
    g = torch.Generator().manual_seed(seed)
    rows = []
    for i in range(24):
        r = torch.randn(1, 96, generator=g) * (10.0 ** (i % 7 - 3))
        if i % 4 == 1:
            r = r.abs()
        elif i % 4 == 2:
            r = -r.abs()
        if i % 6 == 3:
            r[0, ::5] = 0.0
        rows.append(r)
    return torch.cat(rows)


def pin_dq8ca_library(o):
    """PyTorch's quantize_per_tensor (its own implementation) maps each row to the same int8
    codes from the oracle's scale and zero point."""
    x = _dq8ca_rows(5)
    q, scale, zp = o.dq8ca_quantize(x)
    for m in range(x.shape[0]):
        ref = torch.quantize_per_tensor(x[m], float(scale[m]), int(zp[m]), torch.qint8).int_repr().numpy()
        assert np.array_equal(ref, q[m]), (m, np.nonzero(ref != q[m]))


def pin_dq8ca_properties(o):
    """Facts of an 8-bit asymmetric grid that spans each row, whatever the formulas: zero is a
    grid point, every value is within half a step of its grid value (plus the fp32 roundings of the
    step, its reciprocal and x / step carried over at most 255 steps: 255 * 3 * 2^-24 of a step),
    the 255 steps span [min(0, row min), max(0, row max)], the row's extreme below zero takes code
    -128, codes are monotone."""
    for act in ACT_DTYPES:
        x = _dq8ca_rows(6).to(DTYPES[act])
        q, scale, zp = o.dq8ca_quantize(x)
        xf = x.to(torch.float64).numpy()
        for m in range(xf.shape[0]):
            s = float(scale[m])
            lo, hi = min(0.0, xf[m].min()), max(0.0, xf[m].max())
            assert abs(s * 255 - (hi - lo)) <= 2 ** -21 * (hi - lo), (act, m)
            back = s * (q[m].astype(np.float64) - zp[m])
            assert np.all(np.abs(back - xf[m]) <= s * (0.5 + 255 * 3 * 2 ** -24)), (act, m)
            assert np.all(back[xf[m] == 0] == 0.0)
            assert np.all(np.diff(q[m][np.argsort(xf[m], kind="stable")].astype(int)) >= 0)
            if lo < 0:
                assert q[m][np.argmin(xf[m])] == -128
    z = torch.zeros(2, 8)
    q, scale, zp = o.dq8ca_quantize(z)
    assert np.all(q == -128) and np.all(zp == -128) and np.all(scale > 0)


def pin_dq8ca_linear(o):
    """Rows already on the grid (scale 1/64) give exactly the plain forward; random rows match
    a numpy matmul of the dequantised rows; code 8 contributes zero."""
    g = torch.Generator().manual_seed(8)
    M, N, K, gs = 5, 7, 64, 16
    j = torch.randint(-128, 128, (M, K), generator=g)
    j[:, 0], j[:, 1] = -128, 127                       # each row spans [-2, 127/64]: scale 1/64, zp 0
    x = (j.to(torch.float64) / 64).to(torch.float32)
    codes = draw_codes(g, N, K)
    for sdt in SCALE_DTYPES:
        scales = draw_scales(g, K // gs, N, sdt, 0.005, 0.02)
        y, r = o.linear_dq8ca(x, codes, scales, gs)
        y0, r0 = o.linear_fwd(x, codes, scales, gs)
        assert np.array_equal(y, y0) and np.array_equal(r, r0), sdt
    x = _dq8ca_rows(9)[:, :64].contiguous()
    scales = draw_scales(g, K // gs, N, "f16", 0.005, 0.02)
    y, r = o.linear_dq8ca(x, codes, scales, gs)
    q, scale, zp = o.dq8ca_quantize(x)
    xt = scale.astype(np.float64)[:, None] * (q.astype(np.float64) - zp[:, None])
    ref = xt @ _dense(codes, scales, gs).T
    assert np.all(np.abs(y - ref) <= 1e-12 * r + 1e-300)
    assert np.allclose(r, np.abs(xt) @ np.abs(_dense(codes, scales, gs)).T, rtol=1e-12, atol=0)
    eight = torch.full((N, K), 8, dtype=torch.uint8)
    assert np.array_equal(o.linear_dq8ca(x, eight, scales, gs)[0], np.zeros((x.shape[0], N)))


def _lora_case(seed, M, N, K, gs, r, act="f32", sdt="f16"):
    g = torch.Generator().manual_seed(seed)
    x = draw_activation(g, M, K, act)
    d_out = draw_activation(g, M, N, act)
    codes = draw_codes(g, N, K)
    scales = draw_scales(g, K // gs, N, sdt, 0.005, 0.02)
    A = (torch.randn(r, K, generator=g) * 0.05).to(torch.float32)
    B = (torch.randn(N, r, generator=g) * 0.05).to(torch.float32)
    return x, d_out, codes, scales, A, B


def pin_lora_zero_adapter(o):
    """With B = 0 (or A = 0) the adapter forward is the plain forward and the adapter input
    gradient the plain input gradient, bit for bit; the vanishing factor's partner gets a zero
    gradient and the other one the product of the remaining terms."""
    for act in ACT_DTYPES:
        x, d, codes, scales, A, B = _lora_case(31, 4, 12, 32, 8, 3, act)
        y0, r0 = o.linear_fwd(x, codes, scales, 8)
        dx0, rd0 = o.linear_bwd_input(d, codes, scales, 8)
        zb = torch.zeros_like(B)
        y, t, r = o.lora_fwd(x, codes, scales, 8, A, zb, 0.75)
        assert np.array_equal(y, y0) and np.array_equal(r, r0), act
        g = o.lora_bwd(x, d, codes, scales, 8, A, zb, 0.75)
        assert np.array_equal(g["dx"], dx0) and np.array_equal(g["r_dx"], rd0), act
        assert not np.any(g["dA"]), act                  # u = d_out B = 0
        za = torch.zeros_like(A)
        y, t, r = o.lora_fwd(x, codes, scales, 8, za, B, 0.75)
        assert np.array_equal(y, y0) and not np.any(t), act
        g = o.lora_bwd(x, d, codes, scales, 8, za, B, 0.75)
        assert np.array_equal(g["dx"], dx0) and not np.any(g["dB"]), act


def pin_lora_numpy(o):
    """Against numpy fp64 matmuls of the dense matrices: y = x W^T + a (x A^T) B^T,
    dx = d W + a (d B) A, dA = a (d B)^T x, dB = a d^T (x A^T)."""
    x, d, codes, scales, A, B = _lora_case(32, 5, 24, 64, 16, 4, "bf16", "f32")
    a = -1.25
    W = _dense(codes, scales, 16)
    X, D = x.double().numpy(), d.double().numpy()
    An, Bn = A.double().numpy(), B.double().numpy()
    y, t, r = o.lora_fwd(x, codes, scales, 16, A, B, a)
    assert np.all(np.abs(y - (X @ W.T + a * (X @ An.T) @ Bn.T)) <= 1e-12 * r + 1e-300)
    assert np.allclose(t, X @ An.T, rtol=1e-13, atol=1e-300)
    g = o.lora_bwd(x, d, codes, scales, 16, A, B, a)
    assert np.all(np.abs(g["dx"] - (D @ W + a * (D @ Bn) @ An)) <= 1e-12 * g["r_dx"] + 1e-300)
    assert np.all(np.abs(g["dA"] - a * (D @ Bn).T @ X) <= 1e-12 * g["r_dA"] + 1e-300)
    assert np.all(np.abs(g["dB"] - a * D.T @ (X @ An.T)) <= 1e-12 * g["r_dB"] + 1e-300)
    assert np.allclose(g["r_dB"], abs(a) * np.abs(D).T @ (np.abs(X) @ np.abs(An).T), rtol=1e-12, atol=0)


def pin_lora_adjoint(o):
    """The three gradients by their definition: y is linear in x, in A and in B, so for the
    loss <d, y>: <d, y(x)> = <dx, x>, <d, y(A) - y(0)> = <dA, A>, <d, y(B) - y(0)> = <dB, B>."""
    x, d, codes, scales, A, B = _lora_case(33, 6, 20, 48, 16, 5, "f16", "f16")
    a = 0.5
    D, X = d.double().numpy(), x.double().numpy()
    y, _, r = o.lora_fwd(x, codes, scales, 16, A, B, a)
    g = o.lora_bwd(x, d, codes, scales, 16, A, B, a)
    scale = float((np.abs(D) * r).sum())
    assert abs(float((D * y).sum()) - float((g["dx"] * X).sum())) <= 1e-12 * scale
    y0, _, _ = o.lora_fwd(x, codes, scales, 16, A, torch.zeros_like(B), a)
    lhs = float((D * (y - y0)).sum())
    assert abs(lhs - float((g["dA"] * A.double().numpy()).sum())) <= 1e-12 * scale
    assert abs(lhs - float((g["dB"] * B.double().numpy()).sum())) <= 1e-12 * scale


def pin_lora_adapter_only(o):
    """Leaving the frozen weight out (codes None) leaves the adapter term alone: against numpy
    fp64 matmuls y = a (x A^T) B^T and dx = a (d B) A, t unchanged, and dA, dB (which do not
    involve the weight) bit for bit those of the full call."""
    x, d, codes, scales, A, B = _lora_case(35, 7, 20, 48, 16, 6, "bf16", "f16")
    a = 1.5
    X, D = x.double().numpy(), d.double().numpy()
    An, Bn = A.double().numpy(), B.double().numpy()
    y, t, r = o.lora_fwd(x, None, None, 16, A, B, a)
    _, t_full, _ = o.lora_fwd(x, codes, scales, 16, A, B, a)
    assert np.all(np.abs(y - a * (X @ An.T) @ Bn.T) <= 1e-12 * r + 1e-300)
    assert np.allclose(r, abs(a) * (np.abs(X) @ np.abs(An).T) @ np.abs(Bn).T, rtol=1e-12, atol=0)
    assert np.array_equal(t, t_full)
    g = o.lora_bwd(x, d, None, None, 16, A, B, a)
    full = o.lora_bwd(x, d, codes, scales, 16, A, B, a)
    assert np.all(np.abs(g["dx"] - a * (D @ Bn) @ An) <= 1e-12 * g["r_dx"] + 1e-300)
    assert np.allclose(g["r_dx"], abs(a) * (np.abs(D) @ np.abs(Bn)) @ np.abs(An), rtol=1e-12, atol=0)
    for k in ("dA", "dB", "r_dA", "r_dB"):
        assert np.array_equal(g[k], full[k]), k


def pin_adamw_torch(o):
    """One AdamW step from an fp32 state equals torch.optim.AdamW's on the same state (fp64
    tensors), at several step counts and hyperparameters."""
    g = torch.Generator().manual_seed(34)
    for step, lr, b1, b2, eps, wd in [(1, 1e-3, 0.9, 0.999, 1e-8, 0.01), (7, 3e-2, 0.8, 0.99, 1e-6, 0.1),
                                     (250, 5e-4, 0.95, 0.9999, 1e-8, 0.0)]:
        p = torch.randn(64, generator=g).to(torch.float32)
        gr = (torch.randn(64, generator=g) * 0.1).to(torch.float32)
        m = (torch.randn(64, generator=g) * 0.05).to(torch.float32) if step > 1 else torch.zeros(64)
        v = (torch.rand(64, generator=g) * 0.01).to(torch.float32) if step > 1 else torch.zeros(64)
        pr, mr, vr = o.adamw(p, gr, m, v, lr, b1, b2, eps, wd, step)
        param = torch.nn.Parameter(p.double().clone())
        opt = torch.optim.AdamW([param], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
        param.grad = gr.double().clone()
        opt.state[param] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                            "exp_avg": m.double().clone(), "exp_avg_sq": v.double().clone()}
        opt.step()
        st = opt.state[param]
        assert np.allclose(pr, param.detach().numpy(), rtol=1e-13, atol=1e-15), step
        assert np.allclose(mr, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-18), step
        assert np.allclose(vr, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-20), step


def pin_adamw_closed_forms(o):
    """A first step from zero moments without decay moves each parameter by lr g / (|g| + eps)
    against its gradient; a zero gradient with zero moments only decays: p (1 - lr wd)."""
    p = torch.tensor([1.0, -2.0, 0.5, 3.0])
    gr = torch.tensor([0.5, -0.25, 2.0, -1.0])
    z = torch.zeros(4)
    lr, eps = 1e-2, 1e-8
    pr, mr, vr = o.adamw(p, gr, z, z, lr, 0.9, 0.999, eps, 0.0, 1)
    want = p.double().numpy() - lr * gr.double().numpy() / (np.abs(gr.double().numpy()) + eps)
    assert np.allclose(pr, want, rtol=1e-14, atol=0)
    assert np.allclose(mr, 0.1 * gr.double().numpy(), rtol=1e-15, atol=0)
    assert np.allclose(vr, 0.001 * gr.double().numpy() ** 2, rtol=1e-15, atol=0)
    pr, mr, vr = o.adamw(p, z, z, z, lr, 0.9, 0.999, eps, 0.25, 3)
    assert np.array_equal(pr, p.double().numpy() * (1.0 - lr * 0.25))
    assert not np.any(mr) and not np.any(vr)


PINS = [pin_worked_example, pin_code_table, pin_decoders, pin_brute_force, pin_numpy_matmul,
        pin_code8_zero, pin_scale_linearity, pin_adjoint, pin_one_hot, pin_qkv, pin_threads,
        pin_normaliser, pin_embedding, pin_dq8ca_golden, pin_dq8ca_library, pin_dq8ca_properties,
        pin_dq8ca_linear, pin_lora_zero_adapter, pin_lora_numpy, pin_lora_adjoint, pin_lora_adapter_only, pin_adamw_torch,
        pin_adamw_closed_forms]
