"""C-ABI checks that need no GPU: exported symbols, host-side validation, route selection.

Every call here fails validation (or is a pure host function) before the library
makes any HIP call, so fabricated descriptors and fake device addresses are safe.
"""
import ctypes
import os
import re

import pytest
import torch

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "q4gsw.h")


@pytest.fixture(scope="module")
def q():
    from bit_group_quantized_q4gsw_amd import build as qbuild
    if not os.path.exists(qbuild.LIB):
        qbuild.build()
    import bit_group_quantized_q4gsw_amd as q
    return q


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4gsw_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("q4gsw_pack", "q4gsw_linear_fwd", "q4gsw_linear_bwd_input", "q4gsw_qkv_fused"):
        assert n in names


def test_library_exports_every_declared_function(q):
    lib = q.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in include/q4gsw.h but not exported"


def test_status_and_route_names(q):
    assert q.status_str(0) == "ok"
    assert "group_size" in q.status_str(4)
    assert q.route_name(2) == "gemv"
    assert q.route_name(99) == "unknown"
    assert q.lib().q4gsw_layout_version() == 2


S_OK, E_NULL, E_SHAPE, E_DTYPE, E_GROUP, E_ALIAS, E_CODE, E_WS, E_DESC, E_HIP, E_BUF, E_ROUTE = range(12)
FAKE = 1 << 40            # never dereferenced: every call below fails validation first


def packed_bytes(q, N, K, gs, sdt):
    out = ctypes.c_uint64()
    st = q.lib().q4gsw_packed_bytes(N, K, gs, sdt, ctypes.byref(out))
    return st, out.value


def test_packed_bytes(q):
    st, b = packed_bytes(q, 8192, 2048, 32, q.F16)
    assert st == S_OK and b == 256 + 8192 * 2048 // 2 + 64 * 8192 * 2
    st, b = packed_bytes(q, 32, 64, 16, q.F32)         # pads to 128 x 128, 8 scale rows
    assert st == S_OK and b == 256 + 128 * 128 // 2 + 8 * 128 * 4
    assert packed_bytes(q, 0, 64, 16, q.F16)[0] == E_SHAPE
    assert packed_bytes(q, 32, 64, 0, q.F16)[0] == E_GROUP
    assert packed_bytes(q, 32, 64, 24, q.F16)[0] == E_GROUP
    assert packed_bytes(q, 32, 64, 16, q.BF16)[0] == E_DTYPE
    assert q.lib().q4gsw_packed_bytes(32, 64, 16, q.F16, None) == E_NULL


def test_pack_validation(q):
    lib = q.lib()
    d = q.WeightDesc()
    _, need = packed_bytes(q, 32, 64, 16, q.F16)
    assert lib.q4gsw_pack(None, FAKE, q.F16, 32, 64, 16, FAKE * 2, need, None, ctypes.byref(d)) == E_NULL
    assert lib.q4gsw_pack(FAKE, FAKE * 3, q.F16, 32, 64, 16, FAKE * 2, need, None, None) == E_NULL
    assert lib.q4gsw_pack(FAKE, FAKE * 3, q.F16, 32, 64, 0, FAKE * 2, need, None, ctypes.byref(d)) == E_GROUP
    assert lib.q4gsw_pack(FAKE, FAKE * 3, q.F16, 32, 60, 16, FAKE * 2, need, None, ctypes.byref(d)) == E_GROUP
    assert lib.q4gsw_pack(FAKE, FAKE * 3, 9, 32, 64, 16, FAKE * 2, need, None, ctypes.byref(d)) == E_DTYPE
    assert lib.q4gsw_pack(FAKE, FAKE * 3, q.F16, -1, 64, 16, FAKE * 2, need, None, ctypes.byref(d)) == E_SHAPE
    assert lib.q4gsw_pack(FAKE, FAKE * 3, q.F16, 32, 64, 16, FAKE * 2, need - 1, None, ctypes.byref(d)) == E_BUF
    # packed buffer overlapping the codes
    assert lib.q4gsw_pack(FAKE, FAKE * 3, q.F16, 32, 64, 16, FAKE + 100, need, None, ctypes.byref(d)) == E_ALIAS


def fake_desc(q, N, K, gs, sdt=1, flags=0, data=FAKE * 4):
    """A descriptor with the layout fields the library expects (as q4gsw_pack fills them)."""
    def rup(v, m):
        return (v + m - 1) // m * m
    n_pad, k_pad = rup(N, 128), rup(K, 128)
    g_pad = (k_pad + gs - 1) // gs
    nib_off = 256
    scale_off = rup(nib_off + n_pad * k_pad // 2, 256)
    total = rup(scale_off + g_pad * n_pad * (2 if sdt == 1 else 4), 256)
    d = q.WeightDesc()
    d.magic, d.version = 0x57534734, 2
    d.N, d.K, d.group_size = N, K, gs
    d.n_pad, d.k_pad, d.g_pad = n_pad, k_pad, g_pad
    d.scale_dtype, d.flags = sdt, flags
    d.data, d.bytes = data, total
    d.nibble_offset, d.scale_offset = nib_off, scale_off
    return d


def test_fake_descriptor_matches_packed_bytes(q):
    for (N, K, gs, sdt) in [(32, 64, 16, 0), (8192, 2048, 32, 1), (100, 200, 8, 1), (2048, 8192, 128, 1)]:
        d = fake_desc(q, N, K, gs, sdt)
        assert packed_bytes(q, N, K, gs, sdt) == (S_OK, d.bytes)


def route(q, op, d, M, dt, forced=None):
    """The route of a plain call, or (forced = a route name) of a call with that route option."""
    if forced is None:
        return q.route_name(q.lib().q4gsw_route(op, ctypes.byref(d), M, dt))
    o = q.binding.Options(q.ROUTES[forced], 0, 0)
    extra = ctypes.byref(d) if op == q.OP_QKV else None
    st, info = plan_info(q, op, d, M, dt, extra, extra, opts=o)
    assert st == S_OK
    return q.route_name(info.route)


def test_route_selection(q):
    fold = 1
    dec = fake_desc(q, 8192, 2048, 32, 1, flags=fold)
    assert route(q, q.OP_FWD, dec, 1, q.F16) == "gemv"
    assert route(q, q.OP_FWD, dec, 8, q.BF16) == "gemv"
    assert route(q, q.OP_FWD, dec, 9, q.F16) == "gemm_fold"
    assert route(q, q.OP_FWD, dec, 512, q.BF16) == "gemm_group"
    assert route(q, q.OP_FWD, dec, 512, q.F32) == "gemm_split"
    nofold = fake_desc(q, 8192, 2048, 32, 1, flags=0)
    assert route(q, q.OP_FWD, nofold, 512, q.F16) == "gemm_group"
    assert route(q, q.OP_QKV, dec, 512, q.F16) == "qkv_fused"
    assert route(q, q.OP_QKV, dec, 4, q.F16) == "gemv"
    pre = fake_desc(q, 2048, 8192, 128, 1, flags=fold)
    assert route(q, q.OP_FWD, pre, 512, q.BF16) == "gemm_group"
    bwd = fake_desc(q, 8192, 2048, 128, 1, flags=fold)
    assert route(q, q.OP_BWD_INPUT, bwd, 512, q.F32) == "bwd_split"
    assert route(q, q.OP_BWD_INPUT, bwd, 512, q.F16) == "bwd_fold"
    assert route(q, q.OP_BWD_INPUT, bwd, 512, q.BF16) == "bwd_split"
    assert route(q, q.OP_BWD_INPUT, bwd, 4, q.F32) == "bwd_gemv"
    # group sizes the fast kernels do not take fall back to the generic route
    odd = fake_desc(q, 64, 96, 12, 1)
    assert route(q, q.OP_FWD, odd, 1, q.F16) == "generic"
    assert route(q, q.OP_FWD, odd, 100, q.F16) == "generic"
    assert route(q, q.OP_BWD_INPUT, odd, 100, q.F32) == "generic"
    small_gs = fake_desc(q, 256, 256, 32, 1, flags=fold)
    assert route(q, q.OP_BWD_INPUT, small_gs, 64, q.F32) == "bwd_bsplit"   # exact bf16 B, gs = 32
    assert route(q, q.OP_BWD_INPUT, small_gs, 64, q.BF16) == "bwd_bsplit"
    assert route(q, q.OP_BWD_INPUT, small_gs, 64, q.F16) == "bwd_fold"
    gs64 = fake_desc(q, 256, 512, 64, 1, flags=0)                           # not foldable
    assert route(q, q.OP_BWD_INPUT, gs64, 64, q.F16) == "bwd_bsplit"
    assert route(q, q.OP_BWD_INPUT, gs64, 64, q.F32) == "bwd_bsplit"
    f32_scales = fake_desc(q, 256, 256, 32, 0)                             # fp32 scales: no exact hi + lo
    assert route(q, q.OP_BWD_INPUT, f32_scales, 64, q.F32) == "generic"
    gs16 = fake_desc(q, 256, 256, 16, 1, flags=fold)
    assert route(q, q.OP_BWD_INPUT, gs16, 64, q.F16) == "bwd_fold"          # the 16x16x32 kernel
    assert route(q, q.OP_BWD_INPUT, gs16, 64, q.F32) == "generic"
    assert route(q, q.OP_FWD, dec, 0, q.F16) == "none"
    assert route(q, q.OP_FWD, dec, 1, 5) == "none"


def test_forced_routes(q):
    """A route option sends one call onto a route family; the next plain call is unaffected (the
    library keeps no routing state)."""
    dec = fake_desc(q, 8192, 2048, 32, 1, flags=1)
    assert route(q, q.OP_FWD, dec, 1, q.F16, forced="generic") == "generic"
    assert route(q, q.OP_BWD_INPUT, dec, 512, q.F32, forced="generic") == "generic"
    assert route(q, q.OP_FWD, dec, 8, q.F16, forced="gemv") == "gemv"
    assert route(q, q.OP_FWD, dec, 9, q.F16, forced="gemv") == "none"     # the small-M kernels stop at M = 8
    assert route(q, q.OP_BWD_INPUT, dec, 3, q.F16, forced="gemv") == "bwd_gemv"
    assert route(q, q.OP_FWD, dec, 1, q.F16, forced="gemm_fold") == "gemm_fold"
    assert route(q, q.OP_FWD, dec, 1, q.BF16, forced="gemm_fold") == "gemm_group"
    assert route(q, q.OP_QKV, dec, 1, q.F16, forced="gemm_fold") == "qkv_fused"
    assert route(q, q.OP_FWD, dec, 1, q.F16) == "gemv"


def test_binding_options_are_per_thread(q):
    """forced_route / forced_plan hold the choice in the calling Python thread only, and restore the
    enclosing choice on exit."""
    import threading
    assert q.binding._opts() is None
    seen = {}
    with q.forced_route("generic"):
        with q.forced_plan(tile_rows=64, splits=3):
            o = q.binding._local.opts
            assert (o.route, o.tile_rows, o.splits) == (1, 64, 3)
            t = threading.Thread(target=lambda: seen.setdefault("other", q.binding._opts()))
            t.start()
            t.join()
        o = q.binding._local.opts
        assert (o.route, o.tile_rows, o.splits) == (1, 0, 0)
    assert seen["other"] is None
    assert q.binding._opts() is None
    with pytest.raises(ValueError):
        with q.forced_plan(tile_rows=96):
            pass


def test_options_validation(q):
    """Out-of-range options are refused before any HIP call: a route outside the enum with E_ROUTE,
    block rows other than 0 / 64 / 128 and split counts outside 0..64 with E_SHAPE."""
    lib = q.lib()
    d = fake_desc(q, 256, 512, 32, 1, flags=1)
    x, y = FAKE * 8, FAKE * 16
    for (r, rows, splits), want in [((12, 0, 0), E_ROUTE), ((-1, 0, 0), E_ROUTE), ((0, 96, 0), E_SHAPE),
                                    ((0, 0, -1), E_SHAPE), ((0, 0, 65), E_SHAPE)]:
        o = q.binding.Options(r, rows, splits)
        assert lib.q4gsw_linear_fwd_ex(ctypes.byref(d), x, q.F16, 64, y, None, 0, ctypes.byref(o), None) == want
        assert lib.q4gsw_linear_bwd_input_ex(ctypes.byref(d), x, q.F16, 64, y, None, 0, ctypes.byref(o),
                                             None) == want
        need = ctypes.c_uint64()
        assert lib.q4gsw_workspace_bytes_ex(q.OP_FWD, ctypes.byref(d), 64, q.F16, ctypes.byref(o),
                                            ctypes.byref(need)) == want
        assert plan_info(q, q.OP_FWD, d, 64, q.F16, opts=o)[0] == want


def test_binding_rejects_bad_outputs(q):
    """Every output tensor a caller hands the binding must be what the kernels write: contiguous
    fp32 of exactly the output shape on the input's device (checked before any library call)."""
    cpu = torch.device("cpu")
    good = torch.empty(3, 5, dtype=torch.float32)
    assert q.binding._out(good, (3, 5), cpu, "out") is good
    assert q.binding._out(None, (3, 5), cpu, "out").shape == (3, 5)
    bad = [torch.empty(3, 5, dtype=torch.float16),              # dtype
           torch.empty(5, 3, dtype=torch.float32).t(),          # strided view
           torch.empty(3, 4, dtype=torch.float32),              # too small
           torch.empty(15, dtype=torch.float32),                # right size, wrong shape
           torch.empty(4, 5, dtype=torch.float32)]              # too large
    for t in bad:
        with pytest.raises(ValueError):
            q.binding._out(t, (3, 5), cpu, "out")
    with pytest.raises(ValueError):
        q.binding._out(good, (3, 5), torch.device("cuda", 0), "out")   # another device


def test_forward_validation(q):
    lib = q.lib()
    d = fake_desc(q, 256, 512, 32, 1, flags=1)
    x, y = FAKE * 8, FAKE * 16
    f = lib.q4gsw_linear_fwd
    bad = fake_desc(q, 256, 512, 32, 1)
    bad.magic = 0
    assert f(ctypes.byref(bad), x, q.F16, 4, y, None, 0, None) == E_DESC
    bad = fake_desc(q, 256, 512, 32, 1)
    bad.k_pad = 640
    assert f(ctypes.byref(bad), x, q.F16, 4, y, None, 0, None) == E_DESC
    bad = fake_desc(q, 256, 512, 32, 1)
    bad.bytes -= 1
    assert f(ctypes.byref(bad), x, q.F16, 4, y, None, 0, None) == E_DESC
    assert f(None, x, q.F16, 4, y, None, 0, None) == E_NULL
    assert f(ctypes.byref(d), None, q.F16, 4, y, None, 0, None) == E_NULL
    assert f(ctypes.byref(d), x, q.F16, 0, y, None, 0, None) == E_SHAPE
    assert f(ctypes.byref(d), x, 7, 4, y, None, 0, None) == E_DTYPE
    assert f(ctypes.byref(d), x, q.F16, 4, x + 64, None, 0, None) == E_ALIAS        # y inside x
    assert f(ctypes.byref(d), x, q.F16, 4, FAKE * 4 + 512, None, 0, None) == E_ALIAS  # y inside the weight
    big = fake_desc(q, 2048, 8192, 128, 1, flags=1)
    need = ctypes.c_uint64()
    assert lib.q4gsw_workspace_bytes(q.OP_FWD, ctypes.byref(big), 512, q.BF16, ctypes.byref(need)) == S_OK
    assert need.value > 0                    # the prefill shape splits K across blocks
    assert f(ctypes.byref(big), x, q.BF16, 512, y, None, 0, None) == E_WS
    assert f(ctypes.byref(big), x, q.BF16, 512, y, FAKE * 32, need.value - 4, None) == E_WS
    assert f(ctypes.byref(big), x, q.BF16, 512, y, y + 256, need.value, None) == E_ALIAS  # ws overlaps y
    assert f(ctypes.byref(big), x, q.BF16, 512, y, FAKE * 32 + 16, need.value, None) == E_WS  # ws not 256-aligned
    o = q.binding.Options(q.ROUTES["gemv"], 0, 0)
    assert lib.q4gsw_linear_fwd_ex(ctypes.byref(d), x, q.F16, 64, y, None, 0, ctypes.byref(o), None) == E_ROUTE


def test_backward_and_qkv_validation(q):
    lib = q.lib()
    d = fake_desc(q, 256, 512, 32, 1)
    g, dx = FAKE * 8, FAKE * 16
    b = lib.q4gsw_linear_bwd_input
    assert b(ctypes.byref(d), g, q.F32, 4, None, None, 0, None) == E_NULL
    assert b(ctypes.byref(d), g, q.F32, -3, dx, None, 0, None) == E_SHAPE
    assert b(ctypes.byref(d), g, q.F32, 4, g + 4, FAKE * 32, 1 << 30, None) == E_ALIAS
    wq = fake_desc(q, 2048, 2048, 32, 1, flags=1, data=FAKE * 4)
    wk = fake_desc(q, 512, 2048, 32, 1, flags=1, data=FAKE * 5)
    wv = fake_desc(q, 512, 2048, 32, 1, flags=1, data=FAKE * 6)
    qf = lib.q4gsw_qkv_fused
    x, o1, o2, o3 = FAKE * 8, FAKE * 16, FAKE * 17, FAKE * 18
    wrong_k = fake_desc(q, 512, 1024, 32, 1, flags=1, data=FAKE * 5)
    assert qf(ctypes.byref(wq), ctypes.byref(wrong_k), ctypes.byref(wv), x, q.F16, 4, o1, o2, o3, None, 0,
              None) == E_DESC
    wrong_gs = fake_desc(q, 512, 2048, 64, 1, flags=1, data=FAKE * 5)
    assert qf(ctypes.byref(wq), ctypes.byref(wrong_gs), ctypes.byref(wv), x, q.F16, 4, o1, o2, o3, None, 0,
              None) == E_DESC
    # outputs that overlap each other
    assert qf(ctypes.byref(wq), ctypes.byref(wk), ctypes.byref(wv), x, q.F16, 4, o1, o1 + 8, o3, FAKE * 40,
              1 << 30, None) == E_ALIAS
    assert qf(ctypes.byref(wq), ctypes.byref(wk), ctypes.byref(wv), x, q.F16, 4, o1, o2, None, None, 0,
              None) == E_NULL
    need = ctypes.c_uint64()
    assert lib.q4gsw_qkv_workspace_bytes(ctypes.byref(wq), ctypes.byref(wk), ctypes.byref(wv), 128, q.F16,
                                         ctypes.byref(need)) == S_OK
    if need.value:
        assert qf(ctypes.byref(wq), ctypes.byref(wk), ctypes.byref(wv), x, q.F16, 128, o1, o2, o3, None, 0,
                  None) == E_WS


def test_python_wrappers_reject_host_tensors(q):
    with pytest.raises(ValueError):
        q.pack(torch.zeros(4, 8, dtype=torch.uint8), torch.ones(1, 4, dtype=torch.float16), 8)


def plan_info(q, op, d, M, dt, dk=None, dv=None, opts=None):
    info = q.binding.PlanInfo()
    refs = [x if x is None or isinstance(x, type(ctypes.byref(d))) else ctypes.byref(x) for x in (dk, dv)]
    st = q.lib().q4gsw_plan(op, ctypes.byref(d), refs[0], refs[1], M, dt,
                            ctypes.byref(opts) if opts is not None else None, ctypes.byref(info))
    return st, info


def test_plan_attestation_and_forcing(q):
    """q4gsw_plan reports the route, block rows and splits; the tile_rows and splits options pin
    the forward block rows and split count of one call (host logic only)."""
    fold = 1
    pre = fake_desc(q, 2048, 8192, 128, 1, flags=fold)
    st, info = plan_info(q, q.OP_FWD, pre, 512, q.BF16)
    assert st == S_OK and q.route_name(info.route) == "gemm_group"
    assert info.tile_rows in (64, 128) and info.splits >= 1
    default = (info.tile_rows, info.splits)
    # null info, and a QKV plan without its other two weights
    assert q.lib().q4gsw_plan(q.OP_FWD, ctypes.byref(pre), None, None, 512, q.BF16, None, None) == 1   # E_NULL
    st, _ = plan_info(q, q.OP_QKV, pre, 512, q.F16)
    assert st == 1
    dec = fake_desc(q, 8192, 2048, 32, 1, flags=fold)
    st, info = plan_info(q, q.OP_FWD, dec, 1, q.F16)
    assert st == S_OK and q.route_name(info.route) == "gemv" and info.tile_rows == 0
    bwd = fake_desc(q, 8192, 2048, 128, 1, flags=fold)
    st, info = plan_info(q, q.OP_BWD_INPUT, bwd, 512, q.F32)
    assert st == S_OK and q.route_name(info.route) == "bwd_split" and info.tile_rows == 128
    for rows, splits in [(64, 3), (128, 16)]:
        st, info = plan_info(q, q.OP_FWD, pre, 512, q.BF16, opts=q.binding.Options(0, rows, splits))
        assert st == S_OK and info.tile_rows == rows and info.splits == splits
    # a requested count is rounded to one without an empty split: 128 chunks in 5 -> 26 per split, 5
    five = q.binding.Options(0, 0, 5)
    assert plan_info(q, q.OP_FWD, pre, 512, q.BF16, opts=five)[1].splits == 5
    # the same options govern the 32x32 input-gradient plan
    assert plan_info(q, q.OP_BWD_INPUT, bwd, 512, q.F32, opts=q.binding.Options(0, 0, 4))[1].splits == 4
    # the workspace size follows the plan of the options: splits x M x n_pad fp32 partials
    need = ctypes.c_uint64()
    assert q.lib().q4gsw_workspace_bytes_ex(q.OP_FWD, ctypes.byref(pre), 512, q.BF16, ctypes.byref(five),
                                            ctypes.byref(need)) == S_OK
    assert need.value == 5 * 512 * 2048 * 4
    # a plain plan right after is the library's own choice again
    info = plan_info(q, q.OP_FWD, pre, 512, q.BF16)[1]
    assert (info.tile_rows, info.splits) == default


def test_noalloc_forward_validation(q):
    """The allocation-free forward validates like q4gsw_linear_fwd and refuses, before any HIP call,
    a call whose split partials would not fit its 32 MiB scratch (E_SCRATCH)."""
    lib = q.lib()
    f = lib.q4gsw_linear_fwd_noalloc
    d = fake_desc(q, 256, 512, 32, 1, flags=1)
    x, y = FAKE * 8, FAKE * 16
    assert f(None, x, q.F16, 4, y, None) == E_NULL
    assert f(ctypes.byref(d), None, q.F16, 4, y, None) == E_NULL
    assert f(ctypes.byref(d), x, q.F16, 0, y, None) == E_SHAPE
    assert f(ctypes.byref(d), x, 7, 4, y, None) == E_DTYPE
    assert f(ctypes.byref(d), x, q.F16, 4, x + 64, None) == E_ALIAS
    pre = fake_desc(q, 2048, 8192, 64, 1, flags=1)    # a prefill-like weight the planner splits K for
    need = ctypes.c_uint64()
    assert lib.q4gsw_workspace_bytes(q.OP_FWD, ctypes.byref(pre), 1536, q.BF16, ctypes.byref(need)) == S_OK
    assert need.value > 32 << 20
    assert f(ctypes.byref(pre), x, q.BF16, 1536, y, None) == 12                       # E_SCRATCH
    assert "32 MiB" in q.status_str(12)


def test_dq8ca_validation(q):
    """linear_dq8ca validates like the forward and refuses group sizes its int8 kernel does not
    take (E_GROUP); the quantize call checks its pointers, sizes, dtype and overlaps."""
    lib = q.lib()
    x, y = FAKE * 8, FAKE * 16
    ok = fake_desc(q, 256, 512, 64, 1, flags=1)
    assert route(q, 3, ok, 100, q.BF16) == "dq8ca"
    for gs in (16, 96):
        d = fake_desc(q, 256, 576 if gs == 96 else 512, gs, 1, flags=1)
        assert lib.q4gsw_linear_dq8ca(ctypes.byref(d), x, q.BF16, 100, y, FAKE * 32, 1 << 30, None) == E_GROUP
        assert route(q, 3, d, 100, q.BF16) == "none"
    need = ctypes.c_uint64()
    assert lib.q4gsw_workspace_bytes(3, ctypes.byref(ok), 100, q.BF16, ctypes.byref(need)) == S_OK
    assert need.value >= 100 * 512                        # the quantised rows live in the workspace
    f = lib.q4gsw_linear_dq8ca
    assert f(ctypes.byref(ok), x, q.BF16, 100, y, None, 0, None) == E_WS
    assert f(ctypes.byref(ok), x, q.BF16, 0, y, FAKE * 32, need.value, None) == E_SHAPE
    assert f(ctypes.byref(ok), x, 9, 100, y, FAKE * 32, need.value, None) == E_DTYPE
    assert f(ctypes.byref(ok), x, q.BF16, 100, x + 8, FAKE * 32, need.value, None) == E_ALIAS
    qz = lib.q4gsw_dq8ca_quantize
    assert qz(None, q.F32, 4, 8, FAKE * 2, FAKE * 3, FAKE * 4, None) == E_NULL
    assert qz(x, q.F32, 0, 8, FAKE * 2, FAKE * 3, FAKE * 4, None) == E_SHAPE
    assert qz(x, 5, 4, 8, FAKE * 2, FAKE * 3, FAKE * 4, None) == E_DTYPE
    assert qz(x, q.F32, 4, 8, x + 16, FAKE * 3, FAKE * 4, None) == E_ALIAS            # codes inside x
    assert qz(x, q.F32, 4, 8, FAKE * 2, FAKE * 3, FAKE * 3 + 8, None) == E_ALIAS       # zero points inside scales


def test_embedding_validation(q):
    lib = q.lib()
    d = fake_desc(q, 256, 512, 32, 1)
    ids, out = FAKE * 8, FAKE * 16
    e = lib.q4gsw_embedding
    assert e(None, ids, 4, out, None) == E_NULL
    assert e(ctypes.byref(d), None, 4, out, None) == E_NULL
    assert e(ctypes.byref(d), ids, 4, None, None) == E_NULL
    bad = fake_desc(q, 256, 512, 32, 1)
    bad.magic = 0
    assert e(ctypes.byref(bad), ids, 4, out, None) == E_DESC
    assert e(ctypes.byref(d), ids, 0, out, None) == E_SHAPE
    assert e(ctypes.byref(d), ids, -1, out, None) == E_SHAPE
    assert e(ctypes.byref(d), ids, (1 << 23) + 1, out, None) == E_SHAPE
    assert e(ctypes.byref(d), ids, 4, ids + 16, None) == E_ALIAS               # out overlaps ids
    assert e(ctypes.byref(d), ids, 4, FAKE * 4 + 512, None) == E_ALIAS       # out inside the weight
    # the launch has T * ceil(ceil(K / 8) / 64) blocks, which must stay below 2^31: K = 2^30 gives
    # 2^21 blocks per id, so 1024 ids are refused before any HIP call
    wide = fake_desc(q, 8, 1 << 30, 1 << 30, 1, data=FAKE * 64)
    assert e(ctypes.byref(wide), ids, 1024, FAKE * 128, None) == E_SHAPE


def test_adapter_validation(q):
    """The adapter calls refuse bad ranks, non-finite alpha, missing factors, a short workspace and
    every output that overlaps an input, the other outputs or the workspace."""
    lib = q.lib()
    d = fake_desc(q, 256, 512, 32, 1, flags=1)
    x, y, A, B, t = FAKE * 8, FAKE * 16, FAKE * 20, FAKE * 24, FAKE * 28
    nan, inf = float("nan"), float("inf")
    need = ctypes.c_uint64()
    wsb = lib.q4gsw_adapter_workspace_bytes
    assert wsb(q.OP_FWD, ctypes.byref(d), 4, q.F16, 8, None) == E_NULL
    assert wsb(q.OP_FWD, ctypes.byref(d), 4, q.F16, 0, ctypes.byref(need)) == E_SHAPE
    assert wsb(q.OP_FWD, ctypes.byref(d), 4, q.F16, 65, ctypes.byref(need)) == E_SHAPE
    assert wsb(q.OP_QKV, ctypes.byref(d), 4, q.F16, 8, ctypes.byref(need)) == E_SHAPE
    assert wsb(q.OP_FWD, ctypes.byref(d), 4, 7, 8, ctypes.byref(need)) == E_DTYPE
    assert wsb(q.OP_BWD_INPUT, ctypes.byref(d), 4, q.F16, 8, ctypes.byref(need)) == S_OK
    assert need.value >= 4 * 8 * 4                      # u = d_out B lives in the workspace
    f = lib.q4gsw_adapter_fwd
    assert wsb(q.OP_FWD, ctypes.byref(d), 4, q.F16, 8, ctypes.byref(need)) == S_OK
    assert need.value >= 4 * 8 * 4                      # and the column-chunk sums of t
    fw, fn = FAKE * 52, need.value
    assert f(ctypes.byref(d), x, q.F16, 4, None, B, 8, 1.0, y, t, fw, fn, None) == E_NULL
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, y, None, fw, fn, None) == E_NULL
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 0, 1.0, y, t, fw, fn, None) == E_SHAPE
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 65, 1.0, y, t, fw, fn, None) == E_SHAPE
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, nan, y, t, fw, fn, None) == E_SHAPE
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, inf, y, t, fw, fn, None) == E_SHAPE
    assert f(ctypes.byref(d), x, 7, 4, A, B, 8, 1.0, y, t, fw, fn, None) == E_DTYPE
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, y, t, None, 0, None) == E_WS
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, y, t, fw, fn - 4, None) == E_WS
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, y, x + 64, fw, fn, None) == E_ALIAS   # t inside x
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, y, y + 64, fw, fn, None) == E_ALIAS   # t inside y
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, A + 64, t, fw, fn, None) == E_ALIAS   # y inside A
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, y, B + 4, fw, fn, None) == E_ALIAS    # t inside B
    assert f(ctypes.byref(d), x, q.F16, 4, A, B, 8, 1.0, y, t, A, fn, None) == E_ALIAS         # ws over A
    big = fake_desc(q, 2048, 8192, 128, 1, flags=1)
    assert wsb(q.OP_FWD, ctypes.byref(big), 512, q.BF16, 16, ctypes.byref(need)) == S_OK
    assert need.value > 0
    assert f(ctypes.byref(big), x, q.BF16, 512, A, B, 16, 1.0, y, t, None, 0, None) == E_WS
    assert f(ctypes.byref(big), x, q.BF16, 512, A, B, 16, 1.0, y, t, t, need.value, None) == E_ALIAS  # ws over t
    g = lib.q4gsw_adapter_bwd
    gx, dx, dA, dB = FAKE * 32, FAKE * 36, FAKE * 40, FAKE * 44
    assert wsb(q.OP_BWD_INPUT, ctypes.byref(d), 4, q.F16, 8, ctypes.byref(need)) == S_OK
    ws = FAKE * 48
    args = lambda **k: [k.get(n, v) for n, v in (("w", ctypes.byref(d)), ("x", x), ("g", gx), ("dt", q.F16),
                                                    ("M", 4), ("A", A), ("B", B), ("r", 8), ("alpha", 1.0),
                                                    ("t", t), ("dx", dx), ("dA", dA), ("dB", dB), ("ws", ws),
                                                    ("wsb", need.value), ("s", None))]
    for k in ("x", "g", "A", "B", "t", "dx", "dA", "dB"):
        assert g(*args(**{k: None})) == E_NULL, k
    assert g(*args(r=0)) == E_SHAPE
    assert g(*args(r=65)) == E_SHAPE
    assert g(*args(M=0)) == E_SHAPE
    assert g(*args(alpha=nan)) == E_SHAPE
    assert g(*args(dt=7)) == E_DTYPE
    assert g(*args(ws=None, wsb=0)) == E_WS
    assert g(*args(wsb=need.value - 4)) == E_WS
    assert g(*args(dA=x + 16)) == E_ALIAS                  # d_A inside x
    assert g(*args(dB=dx + 16)) == E_ALIAS                 # d_B inside d_x
    assert g(*args(dx=t)) == E_ALIAS                       # d_x over t
    assert g(*args(ws=gx)) == E_ALIAS                      # workspace over d_out
    assert g(*args(dx=ws + 256)) == E_ALIAS                # d_x inside the workspace
    assert g(*args(dB=FAKE * 4 + 512)) == E_ALIAS          # d_B inside the weight


def test_adamw_validation(q):
    lib = q.lib()
    p, gr, m, v = FAKE * 8, FAKE * 12, FAKE * 16, FAKE * 20
    hp = lambda **k: ctypes.byref(q.binding.AdamwParams(k.get("lr", 1e-3), k.get("b1", 0.9), k.get("b2", 0.999),
                                                         k.get("eps", 1e-8), k.get("wd", 0.01)))
    f = lib.q4gsw_adamw_step
    assert f(p, gr, m, v, 64, None, 1, None) == E_NULL
    assert f(None, gr, m, v, 64, hp(), 1, None) == E_NULL
    assert f(p, gr, m, None, 64, hp(), 1, None) == E_NULL
    assert f(p, gr, m, v, 64, hp(), 0, None) == E_SHAPE            # steps count from 1
    assert f(p, gr, m, v, -1, hp(), 1, None) == E_SHAPE
    for bad in (dict(lr=-1.0), dict(lr=float("inf")), dict(b1=1.0), dict(b1=-0.1), dict(b2=float("nan")),
                dict(eps=0.0), dict(wd=-0.5)):
        assert f(p, gr, m, v, 64, hp(**bad), 1, None) == E_SHAPE, bad
    assert f(p, p + 128, m, v, 64, hp(), 1, None) == E_ALIAS      # grad overlaps param
    assert f(p, gr, m, m + 4, 64, hp(), 1, None) == E_ALIAS       # second moment overlaps first
    assert f(None, None, None, None, 0, hp(), 1, None) == S_OK    # nothing to update: no HIP call


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says why (no GPU touched)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
