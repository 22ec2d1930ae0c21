"""HIP-graph capture of every entry point: each replay must equal the eager result bitwise.

The kernels are deterministic (no atomics, fixed reduction order) and record no memset, so a
captured call replayed several times, with other eager work and synchronisations between the
replays, must reproduce the eager output exactly.  The benchmark times its step this way.
"""
import pytest
import torch

from synthetic_inputs import make_adamw_state, make_adapter, make_embedding, make_linear, make_qkv
from tests.gpu_helpers import dev, lib, pack

pytestmark = pytest.mark.gpu

CASES = [
    # kind, M, N, K, gs, act dtype, scale dtype
    ("fwd", 1, 1024, 512, 32, "f16", "f16"),        # decode GEMV route
    ("fwd", 130, 512, 1024, 128, "bf16", "f16"),    # MFMA forward with K splits and reduction
    ("fwd", 64, 256, 384, 32, "f16", "f16"),        # folded fp16 forward
    ("bwd", 3, 512, 256, 32, "f16", "f16"),         # input-gradient GEMV
    ("bwd", 130, 1024, 512, 128, "f32", "f16"),     # input-gradient split route
    ("qkv", 128, None, 512, 32, "f16", "f16"),      # fused QKV
    ("qkv", 1, None, 512, 32, "f16", "f16"),        # decode QKV: one row-octet GEMV launch
    ("qkv", 4, None, 512, 32, "bf16", "f32"),       # small-M QKV: one segmented GEMV launch
    ("emb", 37, 300, 256, 32, None, "f16"),         # embedding row gather
]


def _call(q, kind, pw, a, outs, ws):
    if kind == "emb":
        q.embedding(pw[0], a, out=outs[0])
    elif kind == "fwd":
        q.linear_fwd(pw[0], a, out=outs[0], workspace=ws)
    elif kind == "bwd":
        q.linear_bwd_input(pw[0], a, out=outs[0], workspace=ws)
    else:
        q.qkv_fused(pw[0], pw[1], pw[2], a, outs=outs, workspace=ws)


@pytest.mark.parametrize("kind,M,N,K,gs,act,sdt", CASES)
def test_graph_replay_matches_eager(kind, M, N, K, gs, act, sdt):
    q = lib()
    if kind == "qkv":
        case = make_qkv(M=M, K=K, Ns=(512, 128, 128), group_size=gs, act_dtype=act, scale_dtype=sdt, seed=5)
        ws_list = case.weights
        a = dev(case.x)
    elif kind == "emb":
        case = make_embedding(M, K, N, gs, sdt, seed=9)
        ws_list = [case.w]
        a = dev(case.ids)
    else:
        case = make_linear(M, K, N, gs, act, sdt, seed=M + K, fwd=(kind == "fwd"), bwd=(kind == "bwd"))
        ws_list = [case.w]
        a = dev(case.x if kind == "fwd" else case.d_out)
    pw = [pack(q, w) for w in ws_list]
    if kind in ("bwd", "emb"):
        shapes = [(M, K)]
        op = q.OP_BWD_INPUT
    else:
        shapes = [(M, w.N) for w in ws_list]
        op = q.OP_QKV if kind == "qkv" else q.OP_FWD
    if kind == "qkv":
        need = q.qkv_workspace_bytes(pw[0], pw[1], pw[2], M, a.dtype)
    elif kind == "emb":
        need = 0
    else:
        need = q.workspace_bytes(op, pw[0], M, a.dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    eager = tuple(torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes)
    _call(q, kind, pw, a, eager, ws)
    torch.cuda.synchronize()

    outs = tuple(torch.full(s, float("nan"), dtype=torch.float32, device="cuda") for s in shapes)
    _call(q, kind, pw, a, outs, ws)                 # warm the stream before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(q, kind, pw, a, outs, ws)
    torch.cuda.synchronize()

    other = torch.randn(1 << 16, device="cuda")
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"{kind} replay {rep} differs from the eager result"
        # eager work between replays that reuses the workspace and the stream
        _call(q, kind, pw, a, eager, ws)
        other.mul_(1.0001)
        torch.cuda.synchronize()


def test_graph_replay_adapter_step():
    """The adapter forward and backward captured once and replayed: every replay gives the eager
    t, y, d_x, d_A and d_B bit for bit, with eager calls that reuse the workspaces in between.
    AdamW captured for one step and replayed from a restored state gives the eager step."""
    q = lib()
    M, N, K, r, alpha = 300, 1024, 512, 16, 0.5
    case = make_adapter(M, K, N, 64, "bf16", "f16", r, seed=11)
    pw = pack(q, case.w)
    x, d, A, B = dev(case.x), dev(case.d_out), dev(case.A), dev(case.B)
    wsf = torch.empty(max(q.adapter_workspace_bytes(q.OP_FWD, pw, M, x.dtype, r), 1), dtype=torch.uint8,
                      device="cuda")
    wsb = torch.empty(max(q.adapter_workspace_bytes(q.OP_BWD_INPUT, pw, M, x.dtype, r), 1), dtype=torch.uint8,
                      device="cuda")

    def step(y, t, dx, dA, dB):
        q.adapter_fwd(pw, x, A, B, alpha, out=y, t=t, workspace=wsf)
        q.adapter_bwd(pw, x, d, A, B, alpha, t, d_x=dx, d_A=dA, d_B=dB, workspace=wsb)

    shapes = [(M, N), (M, r), (M, K), (r, K), (N, r)]
    eager = [torch.empty(s, device="cuda") for s in shapes]
    step(*eager)
    torch.cuda.synchronize()
    outs = [torch.full(s, float("nan"), device="cuda") for s in shapes]
    step(*outs)                                     # warm the stream before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*outs)
    torch.cuda.synchronize()
    scratch = [torch.empty(s, device="cuda") for s in shapes]
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, e in zip(("y", "t", "d_x", "d_A", "d_B"), outs, eager):
            assert torch.equal(o, e), f"adapter {name}: replay {rep} differs from the eager result"
        step(*scratch)                              # eager work on the same workspaces
        torch.cuda.synchronize()

    # AdamW: one captured step, replayed from the same starting state each time
    p0, g0, m0, v0 = (dev(t) for t in make_adamw_state(4099, 3, seed=2))
    P, G, Mm, V = (t.clone() for t in (p0, g0, m0, v0))
    q.adamw_step(P, G, Mm, V, 3, 1e-3, 0.9, 0.999, 1e-8, 0.01)
    torch.cuda.synchronize()
    want = (P.clone(), Mm.clone(), V.clone())
    for t, s in zip((P, Mm, V), (p0, m0, v0)):
        t.copy_(s)
    torch.cuda.synchronize()
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        q.adamw_step(P, G, Mm, V, 3, 1e-3, 0.9, 0.999, 1e-8, 0.01)
    for rep in range(3):
        for t, s in zip((P, Mm, V), (p0, m0, v0)):
            t.copy_(s)
        torch.cuda.synchronize()
        ga.replay()
        torch.cuda.synchronize()
        for name, t, w in zip(("param", "exp_avg", "exp_avg_sq"), (P, Mm, V), want):
            assert torch.equal(t, w), f"adamw {name}: replay {rep} differs from the eager step"
