"""GPU parity: every entry point and route against the fp64 oracle, elementwise.

Acceptance: |gpu - oracle| <= tol * R with R = sum |activation| * |dequant(W)| over the
contraction; tol = 1e-5 for fp32 activations and 2e-3 for fp16 / bf16.
"""
import numpy as np
import pytest
import torch

from synthetic_inputs import make_linear, make_qkv, make_workload
from tests.gpu_helpers import (TOL, assert_within, dev, lib, oracle_bwd, oracle_fwd, pack, sample_rows)

pytestmark = pytest.mark.gpu

ROUTE_FAMILIES = ("auto", "generic", "gemv", "gemm_fold")


def run_routes(q, fn, family_list=ROUTE_FAMILIES):
    """Yield (family, result) for every route family that can serve the call."""
    out = []
    for fam in family_list:
        try:
            if fam == "auto":
                res = fn()
            else:
                with q.forced_route(fam):
                    res = fn()
        except q.Q4gswError as e:
            if e.status == 11:          # E_ROUTE: this family cannot serve the shape
                continue
            raise
        torch.cuda.synchronize()
        out.append((fam, res))
    return out


FWD_CASES = [
    # M, N, K, gs, act, scale
    (4, 32, 64, 16, "f32", "f32"),        # tiny workload
    (1, 200, 256, 32, "f16", "f16"),
    (3, 384, 200, 8, "bf16", "f16"),
    (8, 256, 512, 64, "f32", "f32"),
    (5, 130, 136, 8, "f16", "f32"),
    (9, 256, 512, 32, "f16", "f16"),
    (17, 300, 256, 32, "bf16", "f16"),
    (130, 512, 1024, 128, "bf16", "f16"),
    (64, 256, 384, 64, "f16", "f32"),
    (33, 256, 256, 32, "f32", "f16"),
    (200, 640, 512, 16, "f16", "f16"),
    (100, 192, 96, 12, "f16", "f16"),
    (20, 128, 104, 8, "bf16", "f16"),
    (2, 40, 44, 4, "f32", "f16"),
    (257, 136, 320, 64, "bf16", "f32"),
]


@pytest.mark.parametrize("M,N,K,gs,act,sdt", FWD_CASES)
def test_forward_all_routes(M, N, K, gs, act, sdt):
    q = lib()
    case = make_linear(M, K, N, gs, act, sdt, seed=M * 7 + N, s_lo=0.005 if sdt == "f32" else 0.002)
    w = case.w
    pw = pack(q, w)
    x = dev(case.x)
    ref, norm = oracle_fwd(case.x, w)
    tol = TOL[case.x.dtype]
    ran = run_routes(q, lambda: q.linear_fwd(pw, x))
    assert ran and ran[0][0] == "auto"
    for fam, y in ran:
        assert_within(y, ref, norm, tol, f"fwd {fam} route={q.route(q.OP_FWD, pw, M, case.x.dtype)}")


BWD_CASES = [
    (4, 32, 64, 16, "f32", "f32"),        # tiny workload
    (2, 300, 256, 32, "f16", "f16"),
    (8, 256, 200, 8, "f32", "f16"),
    (64, 512, 512, 128, "f32", "f16"),
    (130, 1000, 256, 128, "bf16", "f16"),
    (96, 512, 384, 32, "f16", "f16"),
    (40, 384, 256, 256, "f16", "f32"),
    (50, 100, 96, 32, "f32", "f16"),
    (12, 64, 72, 24, "bf16", "f16"),
    (7, 136, 512, 128, "bf16", "f32"),
    (200, 200, 384, 128, "f16", "f16"),
]


@pytest.mark.parametrize("M,N,K,gs,act,sdt", BWD_CASES)
def test_backward_all_routes(M, N, K, gs, act, sdt):
    q = lib()
    case = make_linear(M, K, N, gs, act, sdt, seed=M * 11 + K, fwd=False, bwd=True,
                       sigma=0.1 if act == "f32" else 1.0)
    w = case.w
    pw = pack(q, w)
    g = dev(case.d_out)
    ref, norm = oracle_bwd(case.d_out, w)
    tol = TOL[case.d_out.dtype]
    ran = run_routes(q, lambda: q.linear_bwd_input(pw, g))
    assert ran and ran[0][0] == "auto"
    for fam, dx in ran:
        assert_within(dx, ref, norm, tol, f"bwd {fam} route={q.route(q.OP_BWD_INPUT, pw, M, case.d_out.dtype)}")


QKV_CASES = [
    (128, 2048, (2048, 512, 512), 32, "f16"),     # the Llama projection triple at M = 128
    (20, 96, (64, 40, 24), 32, "bf16"),
    (9, 256, (256, 128, 128), 64, "f32"),
    (3, 128, (128, 64, 64), 16, "f16"),
    (300, 512, (384, 128, 200), 128, "f16"),
]


@pytest.mark.parametrize("M,K,Ns,gs,act", QKV_CASES)
def test_qkv_fused(M, K, Ns, gs, act):
    q = lib()
    case = make_qkv(M, K, Ns, gs, act, "f16", seed=M + K)
    pws = [pack(q, w) for w in case.weights]
    x = dev(case.x)
    rows = sample_rows(M, 24) if M > 128 else None
    refs = [oracle_fwd(case.x, w, rows) for w in case.weights]
    tol = TOL[case.x.dtype]
    for fam, outs in run_routes(q, lambda: q.qkv_fused(*pws, x)):
        for name, o, (ref, norm) in zip("qkv", outs, refs):
            assert_within(o, ref, norm, tol, f"qkv {fam} {name}", rows)
    # fused against three separate forwards: both within tol of the oracle, so within 2 tol of each other
    fused = q.qkv_fused(*pws, x)
    for o, pw, (_, norm) in zip(fused, pws, refs):
        sep = q.linear_fwd(pw, x)
        diff = (o - sep).abs().cpu().numpy().astype(np.float64)
        if rows is not None:
            diff = diff[rows]
        assert np.all(diff <= 2 * tol * norm + 1e-30)


# ---- the suite's workloads at full size (sampled rows where the oracle would be slow) ----------

def test_workload_tiny():
    q = lib()
    case = make_workload("tiny")
    pw = pack(q, case.w)
    y = q.linear_fwd(pw, dev(case.x))
    ref, norm = oracle_fwd(case.x, case.w)
    assert_within(y, ref, norm, 1e-5, "tiny fwd")
    dx = q.linear_bwd_input(pw, dev(case.d_out))
    ref, norm = oracle_bwd(case.d_out, case.w)
    assert_within(dx, ref, norm, 1e-5, "tiny bwd")


def test_workload_decode():
    q = lib()
    case = make_workload("decode")
    pw = pack(q, case.w)
    assert q.route(q.OP_FWD, pw, 1, case.x.dtype) == "gemv"
    y = q.linear_fwd(pw, dev(case.x))
    ref, norm = oracle_fwd(case.x, case.w)
    assert_within(y, ref, norm, 2e-3, "decode")


@pytest.mark.parametrize("act", ["bf16", "f16", "f32"])
def test_workload_prefill(act):
    q = lib()
    case = make_workload("prefill", act_dtype=act)
    pw = pack(q, case.w)
    y = q.linear_fwd(pw, dev(case.x))
    rows = sample_rows(case.M)
    ref, norm = oracle_fwd(case.x, case.w, rows)
    assert_within(y, ref, norm, TOL[case.x.dtype], f"prefill {act}", rows)


@pytest.mark.parametrize("M", [128, 508, 512])
def test_workload_qkv(M):
    q = lib()
    case = make_workload("qkv", M=M)
    pws = [pack(q, w) for w in case.weights]
    assert q.route(q.OP_QKV, pws[0], M, case.x.dtype) == "qkv_fused"
    outs = q.qkv_fused(*pws, dev(case.x))
    rows = sample_rows(M)
    for name, o, w in zip("qkv", outs, case.weights):
        ref, norm = oracle_fwd(case.x, w, rows)
        assert_within(o, ref, norm, 2e-3, f"qkv M={M} {name}", rows)


@pytest.mark.parametrize("act", ["f32", "f16", "bf16"])
def test_workload_bwd(act):
    q = lib()
    case = make_workload("bwd")
    d_out = case.d_out if act == "f32" else case.d_out.to({"f16": torch.float16, "bf16": torch.bfloat16}[act])
    pw = pack(q, case.w)
    dx = q.linear_bwd_input(pw, dev(d_out))
    rows = sample_rows(case.M)
    ref, norm = oracle_bwd(d_out, case.w, rows)
    assert_within(dx, ref, norm, TOL[d_out.dtype], f"bwd {act}", rows)


# ---- both forward block tiles (64 and 128 rows), forced, on every forward precision route ------

TILE_CASES = [
    # M, N, K, gs, act, scale
    (130, 512, 1024, 128, "bf16", "f16"),     # group route, ragged M over both tile heights
    (200, 640, 512, 32, "f16", "f16"),        # fold route, two scale slots per chunk
    (96, 256, 320, 8, "f16", "f16"),          # fold route, a scale slot per k-octet
    (257, 264, 256, 64, "f16", "f32"),        # group route with fp32 scales and an N tail
    (65, 256, 384, 64, "f32", "f16"),         # split route (fp32 x)
    (40, 512, 256, 32, "f32", "f32"),         # split route, gs = 32, fp32 scales
]


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("M,N,K,gs,act,sdt", TILE_CASES)
def test_forward_tiles(M, N, K, gs, act, sdt, rows):
    q = lib()
    case = make_linear(M, K, N, gs, act, sdt, seed=M * 11 + N + rows, s_lo=0.005 if sdt == "f32" else 0.002)
    pw = pack(q, case.w)
    x = dev(case.x)
    ref, norm = oracle_fwd(case.x, case.w)
    with q.forced_plan(tile_rows=rows):
        # fp32 activations have no 128-row tile: a forced 128 plans 64
        assert q.plan(q.OP_FWD, pw, M, case.x.dtype)["tile_rows"] == (64 if act == "f32" else rows)
        y = q.linear_fwd(pw, x)
        torch.cuda.synchronize()
    assert_within(y, ref, norm, TOL[case.x.dtype], f"fwd tile {rows} route={q.route(q.OP_FWD, pw, M, case.x.dtype)}")


# fp16 activations with foldable fp16 scales and gs % 32 == 0 run 128-column chunks: a last chunk
# only partly inside K, two or four scale slots per chunk (gs 64, gs 96 with groups not aligned to
# chunks) and a group across two chunks (gs 256), at both tile heights and with K splits.
WIDE_FOLD_CASES = [
    # M, N, K, gs
    (70, 264, 320, 32),
    (130, 300, 448, 64),
    (64, 256, 576, 96),
    (96, 520, 768, 256),
]


@pytest.mark.parametrize("M,N,K,gs", WIDE_FOLD_CASES)
@pytest.mark.parametrize("rows,splits", [(64, 1), (128, 1), (64, 3)])
def test_forward_fold_wide_chunks(M, N, K, gs, rows, splits):
    q = lib()
    case = make_linear(M, K, N, gs, "f16", "f16", seed=M * 13 + K + gs)
    pw = pack(q, case.w)
    x = dev(case.x)
    ref, norm = oracle_fwd(case.x, case.w)
    print(f"fold wide chunks M={M} N={N} K={K} gs={gs} rows={rows} splits={splits}", flush=True)
    with q.forced_plan(tile_rows=rows, splits=splits):
        info = q.plan(q.OP_FWD, pw, M, case.x.dtype)
        assert info["route"] == "gemm_fold" and info["tile_rows"] == rows, info
        y = q.linear_fwd(pw, x)
        torch.cuda.synchronize()
    assert_within(y, ref, norm, TOL[case.x.dtype], f"fwd fold gs={gs} K={K} rows={rows} splits={info['splits']}")


@pytest.mark.parametrize("rows", [64, 128])
def test_qkv_tiles(rows):
    q = lib()
    case = make_qkv(M=200, K=512, Ns=(512, 256, 136), group_size=32, act_dtype="f16", scale_dtype="f16", seed=rows)
    pws = [pack(q, w) for w in case.weights]
    x = dev(case.x)
    refs = [oracle_fwd(case.x, w) for w in case.weights]
    with q.forced_plan(tile_rows=rows):
        assert q.plan(q.OP_QKV, pws[0], 200, case.x.dtype, pws[1], pws[2])["tile_rows"] == rows
        outs = q.qkv_fused(*pws, x)
        torch.cuda.synchronize()
    for name, o, (ref, norm) in zip("qkv", outs, refs):
        assert_within(o, ref, norm, 2e-3, f"qkv tile {rows} {name}")


# ---- forced split counts: every split count gives the oracle's result within tol ----------------

SPLIT_CASES = [
    # kind, M, N, K, gs, act, scale, tile rows, splits
    ("fwd", 130, 512, 1024, 128, "bf16", "f16", 128, 4),
    ("fwd", 64, 264, 2048, 32, "f16", "f16", 64, 8),
    ("fwd", 40, 512, 1536, 64, "f32", "f32", 64, 3),
    ("qkv", 128, None, 2048, 32, "f16", "f16", 64, 2),
    ("qkv", 100, None, 1280, 64, "bf16", "f16", 128, 5),
]


@pytest.mark.parametrize("kind,M,N,K,gs,act,sdt,rows,splits", SPLIT_CASES)
def test_forced_splits(kind, M, N, K, gs, act, sdt, rows, splits):
    q = lib()
    if kind == "qkv":
        case = make_qkv(M=M, K=K, Ns=(512, 128, 136), group_size=gs, act_dtype=act, scale_dtype=sdt, seed=M + K)
        ws_list = case.weights
    else:
        case = make_linear(M, K, N, gs, act, sdt, seed=M + N + K, s_lo=0.005 if sdt == "f32" else 0.002)
        ws_list = [case.w]
    pws = [pack(q, w) for w in ws_list]
    x = dev(case.x)
    with q.forced_plan(tile_rows=rows, splits=splits):
        if kind == "qkv":
            info = q.plan(q.OP_QKV, pws[0], M, case.x.dtype, pws[1], pws[2])
            outs = q.qkv_fused(*pws, x)
        else:
            info = q.plan(q.OP_FWD, pws[0], M, case.x.dtype)
            outs = (q.linear_fwd(pws[0], x),)
        torch.cuda.synchronize()
    assert info["splits"] == splits and info["tile_rows"] == rows, f"forced plan not taken: {info}"
    tol = TOL[case.x.dtype]
    for o, w in zip(outs, ws_list):
        ref, norm = oracle_fwd(case.x, w)
        assert_within(o, ref, norm, tol, f"{kind} splits={splits} rows={rows}")


# ---- forced split counts of the 32x32 input-gradient routes -------------------------------------

BWD_SPLIT_CASES = [
    # M, N, K, gs, d_out dtype, scale dtype, splits; route bwd_split unless noted
    (130, 1024, 512, 128, "f32", "f16", 3),       # ragged M, two scale groups per block
    (64, 2048, 256, 256, "bf16", "f16", 5),       # one scale group per block
    (200, 1536, 384, 128, "f32", "f32", 5),       # fp32 scales, K tail inside a block
    (96, 1024, 512, 64, "f16", "f16", 4),         # bwd_fold
    (40, 1024, 96, 32, "f16", "f16", 3),          # bwd_fold, K = 96 inside one padded 128-column tile
]


@pytest.mark.parametrize("M,N,K,gs,act,sdt,splits", BWD_SPLIT_CASES)
def test_forced_bwd_splits(M, N, K, gs, act, sdt, splits):
    q = lib()
    case = make_linear(M, K, N, gs, act, sdt, seed=M + N + K + splits, fwd=False, bwd=True,
                       s_lo=0.005 if sdt == "f32" else 0.002)
    pw = pack(q, case.w)
    g = dev(case.d_out)
    with q.forced_plan(splits=splits):
        info = q.plan(q.OP_BWD_INPUT, pw, M, case.d_out.dtype)
        dx = q.linear_bwd_input(pw, g)
        torch.cuda.synchronize()
    assert info["splits"] == splits, f"forced split count not taken: {info}"
    ref, norm = oracle_bwd(case.d_out, case.w)
    assert_within(dx, ref, norm, TOL[case.d_out.dtype], f"bwd splits={splits} route={info['route']}")


# ---- row-octet decode (M = 1, fp16 x, K = 512 U with U <= 4) ---------------------------------

ROW_DECODE_CASES = [
    # N, K, gs, scale dtype
    (200, 512, 32, "f16"),       # U = 1, N tail inside the last row-octet block
    (1000, 1024, 64, "f32"),     # U = 2, fp32 scales
    (136, 1536, 8, "f16"),       # U = 3, a scale group per k-octet
    (520, 2048, 128, "f32"),     # U = 4, fp32 scales
    (203, 1024, 32, "f16"),      # U = 2, N ends inside a row-octet
    (2048, 8192, 128, "f16"),    # U = 16, four waves per row-octet
    (300, 4096, 64, "f32"),      # U = 8, fp32 scales, N tail
    (8, 8192, 8, "f16"),         # U = 16, a single row-octet, a scale group per k-octet
]


@pytest.mark.parametrize("N,K,gs,sdt", ROW_DECODE_CASES)
def test_decode_row_octet_path(N, K, gs, sdt):
    q = lib()
    case = make_linear(1, K, N, gs, "f16", sdt, seed=N + K + gs, s_lo=0.005 if sdt == "f32" else 0.002)
    pw = pack(q, case.w)
    assert q.route(q.OP_FWD, pw, 1, torch.float16) == "gemv"
    y = q.linear_fwd(pw, dev(case.x))
    torch.cuda.synchronize()
    ref, norm = oracle_fwd(case.x, case.w)
    assert_within(y, ref, norm, TOL[torch.float16], f"decode row-octet N={N} K={K} gs={gs} {sdt}")


# ---- activations one element off 16-byte alignment take each kernel's guarded fallback --------

def _misaligned(t: torch.Tensor) -> torch.Tensor:
    """A contiguous device copy of t whose data starts one element past an aligned allocation."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
    v = buf[1:].view(t.shape)
    v.copy_(t.cuda())
    assert v.is_contiguous() and v.data_ptr() % 16 != 0
    return v


UNALIGNED_CASES = [
    # kind, M, N, K, gs, act, scale
    ("fwd", 1, 256, 1024, 32, "f16", "f16"),      # decode GEMV (the row-octet path needs alignment)
    ("fwd", 3, 192, 256, 32, "bf16", "f16"),      # GEMV, M = 3
    ("fwd", 64, 256, 512, 32, "f16", "f16"),      # MFMA fold
    ("fwd", 70, 256, 512, 128, "bf16", "f16"),    # MFMA group
    ("fwd", 40, 256, 384, 64, "f32", "f32"),      # MFMA split (fp32 x)
    ("bwd", 2, 256, 512, 32, "f16", "f16"),       # GEMV input gradient
    ("bwd", 64, 512, 256, 64, "f16", "f16"),      # bwd_fold
    ("bwd", 50, 512, 256, 128, "f32", "f16"),     # bwd_split
]


@pytest.mark.parametrize("kind,M,N,K,gs,act,sdt", UNALIGNED_CASES)
def test_unaligned_activation(kind, M, N, K, gs, act, sdt):
    q = lib()
    case = make_linear(M, K, N, gs, act, sdt, seed=M + N + K + gs, fwd=kind == "fwd", bwd=kind == "bwd",
                       s_lo=0.005 if sdt == "f32" else 0.002)
    pw = pack(q, case.w)
    if kind == "fwd":
        got = q.linear_fwd(pw, _misaligned(case.x))
        ref, norm = oracle_fwd(case.x, case.w)
        dt = case.x.dtype
    else:
        got = q.linear_bwd_input(pw, _misaligned(case.d_out))
        ref, norm = oracle_bwd(case.d_out, case.w)
        dt = case.d_out.dtype
    torch.cuda.synchronize()
    route = q.route(q.OP_FWD if kind == "fwd" else q.OP_BWD_INPUT, pw, M, dt)
    assert_within(got, ref, norm, TOL[dt], f"unaligned {kind} M={M} route={route}")


@pytest.mark.parametrize("M", [40, 1, 5])
def test_unaligned_qkv(M):
    """MFMA QKV (M = 40) and the one-launch small-M GEMV (M = 1 and 5; unaligned x leaves the
    row-octet kernel for the segmented GEMV's guarded loads), each equal to separate forwards."""
    q = lib()
    case = make_qkv(M=M, K=512, Ns=(256, 128, 72), group_size=32, act_dtype="f16", scale_dtype="f16", seed=7)
    pws = [pack(q, w) for w in case.weights]
    x = _misaligned(case.x)
    outs = q.qkv_fused(*pws, x)
    separate = [q.linear_fwd(pw, x) for pw in pws]
    torch.cuda.synchronize()
    for name, o, sep, w in zip("qkv", outs, separate, case.weights):
        ref, norm = oracle_fwd(case.x, w)
        assert_within(o, ref, norm, 2e-3, f"unaligned qkv M={M} {name}")
        if M <= 8:
            assert torch.equal(o, sep), f"unaligned qkv M={M} {name}: fused and separate forwards differ"


# ---- decode-shaped fused QKV: one launch of the row-octet GEMV over the three weights ----------

DECODE_QKV_CASES = [
    # K, Ns, gs, scale dtype
    (4096, (4096, 1024, 1024), 64, "f16"),   # U = 8: four waves per row-octet
    (2048, (2048, 512, 512), 32, "f16"),     # the Llama projection triple at decode
    (512, (200, 72, 136), 64, "f32"),        # ragged N per weight, fp32 scales
    (1536, (256, 128, 8), 8, "f16"),         # a weight of a single row-octet
]


@pytest.mark.parametrize("K,Ns,gs,sdt", DECODE_QKV_CASES)
def test_decode_qkv_one_launch(K, Ns, gs, sdt):
    q = lib()
    case = make_qkv(M=1, K=K, Ns=Ns, group_size=gs, act_dtype="f16", scale_dtype=sdt, seed=K + sum(Ns),
                    s_lo=0.005 if sdt == "f32" else 0.002)
    pws = [pack(q, w) for w in case.weights]
    x = dev(case.x)
    assert q.route(q.OP_QKV, pws[0], 1, torch.float16) == "gemv"
    outs = q.qkv_fused(*pws, x)
    separate = [q.linear_fwd(pw, x) for pw in pws]
    torch.cuda.synchronize()
    for name, o, sep, w in zip("qkv", outs, separate, case.weights):
        ref, norm = oracle_fwd(case.x, w)
        assert_within(o, ref, norm, TOL[torch.float16], f"decode qkv {name}")
        assert torch.equal(o, sep), f"decode qkv {name}: fused and separate forwards differ"


EMB_CASES = [
    # T, N, K, gs, scale dtype
    (1, 200, 256, 32, "f16"),              # one id (decode)
    (37, 130, 136, 8, "f32"),              # ragged K past the packing tile, fp32 scales
    (300, 9, 64, 16, "f16"),               # many repeated ids over a 9-row table
    (19, 40, 44, 4, "f16"),                # K not a multiple of 8, group smaller than an octet
    (5, 100, 96, 12, "f16"),               # group size not a multiple of 8
    (64, 1000, 8192, 128, "f32"),          # long rows, fp32 scales
    (7, 50, 60, 12, "f32"),                # fp32 scales, K not a multiple of 8, gs not of 8
]


def _emb_ref(ids, w):
    from oracle import oracle as O
    return O.embedding(ids, w.codes, w.scales, w.group_size)


@pytest.mark.parametrize("T,N,K,gs,sdt", EMB_CASES)
def test_embedding_rows(T, N, K, gs, sdt):
    """Bit-exact: (code - 8) * scale is one fp32 product, correctly rounded on both sides."""
    from synthetic_inputs import make_embedding
    q = lib()
    case = make_embedding(T, K, N, gs, sdt, seed=T * 31 + N, s_lo=0.005 if sdt == "f32" else 0.002)
    pw = pack(q, case.w)
    out = q.embedding(pw, dev(case.ids))
    torch.cuda.synchronize()
    ref = _emb_ref(case.ids, case.w).astype(np.float32)
    assert out.shape == (T, K)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_embedding_out_of_range_and_misaligned_out():
    """Ids outside [0, N) give zero rows; an output 4 bytes off a 16-byte boundary takes the
    scalar-store path with the same values."""
    q = lib()
    from synthetic_inputs import make_embedding
    case = make_embedding(6, 64, 40, 8, "f16", seed=5)
    ids = torch.tensor([-1, 0, 39, 40, 2**40, -2**40, 17, 17], dtype=torch.int64)
    pw = pack(q, case.w)
    ref = _emb_ref(ids, case.w).astype(np.float32)
    out = q.embedding(pw, dev(ids))
    flat = torch.full((ids.numel() * 64 + 1,), 7.0, dtype=torch.float32, device="cuda")
    mis = flat[1:].view(ids.numel(), 64)
    q.embedding(pw, dev(ids), out=mis)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)
    assert np.array_equal(mis.cpu().numpy(), ref)
    assert flat[0].item() == 7.0
    assert not out[[0, 3, 4, 5]].any()


def test_embedding_equals_one_hot_backward():
    """A one-hot output gradient through the input-gradient kernels reads back the same rows."""
    q = lib()
    from synthetic_inputs import make_embedding
    case = make_embedding(8, 512, 256, 32, "f16", seed=11)
    pw = pack(q, case.w)
    emb = q.embedding(pw, dev(case.ids))
    onehot = torch.zeros(8, 256, dtype=torch.float32)
    onehot[torch.arange(8), case.ids] = 1.0
    dx = q.linear_bwd_input(pw, dev(onehot))
    torch.cuda.synchronize()
    assert torch.equal(emb, dx)


def test_workload_embedding():
    """The tied-embedding table of the suite [128256, 2048], 512 ids, all rows checked."""
    q = lib()
    case = make_workload("embedding")
    pw = pack(q, case.w)
    out = q.embedding(pw, dev(case.ids))
    torch.cuda.synchronize()
    ref = _emb_ref(case.ids, case.w).astype(np.float32)
    assert np.array_equal(out.cpu().numpy(), ref)
    # a decode-sized gather (one id) from the same packed table
    one = q.embedding(pw, dev(case.ids[-1:]))
    torch.cuda.synchronize()
    assert np.array_equal(one.cpu().numpy(), ref[-1:])


SMALL_M_QKV_CASES = [
    # M, K, Ns, gs, activation dtype, scale dtype
    (4, 2048, (2048, 512, 512), 32, "f16", "f16"),     # the Llama triple, small decode batch
    (8, 2048, (2048, 512, 512), 32, "bf16", "f16"),
    (1, 2048, (2048, 512, 512), 32, "bf16", "f16"),    # one row outside the fp16 row-octet path
    (3, 512, (200, 72, 136), 64, "f32", "f32"),        # ragged N per weight, fp32 everywhere
    (5, 1000, (256, 128, 8), 8, "f16", "f16"),         # K past the packing tile, a one-octet weight
    (7, 8192, (256, 64, 64), 128, "f32", "f16"),       # long K: eight waves per row-octet
    (2, 32768, (64, 64, 64), 128, "f16", "f16"),       # K split across blocks: three forwards
]


@pytest.mark.parametrize("M,K,Ns,gs,act,sdt", SMALL_M_QKV_CASES)
def test_small_m_qkv_one_launch(M, K, Ns, gs, act, sdt):
    """QKV at M <= 8: one GEMV launch over the three weights when none splits K, bitwise equal to
    three separate forwards, and within tolerance of the oracle."""
    q = lib()
    case = make_qkv(M=M, K=K, Ns=Ns, group_size=gs, act_dtype=act, scale_dtype=sdt, seed=M * 1000 + K,
                    s_lo=0.005 if sdt == "f32" else 0.002)
    pws = [pack(q, w) for w in case.weights]
    x = dev(case.x)
    assert q.route(q.OP_QKV, pws[0], M, x.dtype) == "gemv"
    outs = q.qkv_fused(*pws, x)
    separate = [q.linear_fwd(pw, x) for pw in pws]
    torch.cuda.synchronize()
    for name, o, sep, w in zip("qkv", outs, separate, case.weights):
        ref, norm = oracle_fwd(case.x, w)
        assert_within(o, ref, norm, TOL[x.dtype], f"small-M qkv {name}")
        assert torch.equal(o, sep), f"small-M qkv {name}: fused and separate forwards differ"


ROW_DECODE_BF16_CASES = [
    # N, K, gs, scale dtype: one bf16 row through the row-octet decode kernel
    (200, 512, 32, "f16"),
    (520, 2048, 128, "f32"),
    (8192, 2048, 32, "f16"),      # the decode workload's weight
    (2048, 8192, 128, "f16"),     # four waves per row-octet
    (203, 1024, 32, "f16"),
]


@pytest.mark.parametrize("N,K,gs,sdt", ROW_DECODE_BF16_CASES)
def test_decode_row_octet_bf16(N, K, gs, sdt):
    q = lib()
    case = make_linear(1, K, N, gs, "bf16", sdt, seed=N + K + 7, s_lo=0.005 if sdt == "f32" else 0.002)
    pw = pack(q, case.w)
    y = q.linear_fwd(pw, dev(case.x))
    torch.cuda.synchronize()
    ref, norm = oracle_fwd(case.x, case.w)
    assert_within(y, ref, norm, TOL[torch.bfloat16], f"bf16 decode row-octet N={N} K={K} gs={gs} {sdt}")
