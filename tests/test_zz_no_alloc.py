"""The allocation-free forward (q4gsw_linear_fwd_noalloc) against q4gsw_linear_fwd.

The entry point keeps its K-split partials in the library's per-device scratch instead of a
caller workspace.  Two calls in a row, the second smaller, each must equal q4gsw_linear_fwd's
output bit for bit (same kernels and plan) and the fp64 oracle within the activation's tolerance.
A graph capture of the call replays to the same bits.
"""
import pytest
import torch

from synthetic_inputs import make_linear, make_workload
from tests.gpu_helpers import TOL, assert_within, dev, lib, oracle_fwd, pack, sample_rows

pytestmark = pytest.mark.gpu

SCRATCH = 32 << 20


def _call(q, pw, x, y):
    """q4gsw_linear_fwd_noalloc straight through the C ABI."""
    return q.lib().q4gsw_linear_fwd_noalloc(pw.ref(), x.data_ptr(), q.binding._TORCH_DTYPE[x.dtype], x.shape[0],
                                            y.data_ptr(), q.binding._stream())


def test_noalloc_forward_twice_then_smaller():
    q = lib()
    cases = [
        # the prefill workload: M=512, K=8192, N=2048, gs=128, bf16 x; its plan splits K four ways,
        # so the partials take half of the scratch
        ("prefill", make_workload("prefill")),
        # a smaller forward whose plan also splits K: it reuses what the first call left behind
        ("small", make_linear(96, 2048, 1024, 64, "f16", "f16", seed=5)),
    ]
    for label, case in cases:
        w = case.weights[0]
        pw = pack(q, w)
        x = dev(case.x)
        M = x.shape[0]
        print(f"noalloc case {label}: M={M} N={w.N} K={w.K} gs={w.group_size} x={x.dtype}", flush=True)
        need = q.workspace_bytes(q.OP_FWD, pw, M, x.dtype)
        assert 0 < need <= SCRATCH, (label, need)
        assert q.plan(q.OP_FWD, pw, M, x.dtype)["splits"] > 1
        want = q.linear_fwd(pw, x)
        y = torch.full((M, w.N), float("nan"), dtype=torch.float32, device="cuda")
        assert _call(q, pw, x, y) == 0
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"{label}: differs from q4gsw_linear_fwd"
        rows = sample_rows(M)
        ref, norm = oracle_fwd(case.x, w, rows)
        assert_within(y, ref, norm, TOL[case.x.dtype], f"noalloc {label}", rows=rows)


def test_noalloc_forward_in_a_graph():
    """Captured into a HIP graph (no allocation inside the capture) and replayed, with eager work
    between the replays: every replay equals the eager result."""
    q = lib()
    case = make_linear(130, 1536, 512, 32, "f16", "f16", seed=9)
    w = case.w
    pw = pack(q, w)
    x = dev(case.x)
    print("noalloc graph case: M=130 N=512 K=1536 gs=32 f16", flush=True)
    assert q.plan(q.OP_FWD, pw, 130, x.dtype)["splits"] > 1
    want = q.linear_fwd(pw, x)
    y = torch.empty(130, w.N, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert _call(q, pw, x, y) == 0          # first call on the device outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = _call(q, pw, x, y)
    assert st == 0
    for i in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {i}"
        q.linear_fwd(pw, x)                      # eager work between replays
        torch.cuda.synchronize()
