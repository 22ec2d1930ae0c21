"""Benchmark of the q4gsw hot path on one MI355X.

One step = one pass of every op of the Llama-3.2-1B-shaped q4gsw suite, each on its own
seeded synthetic inputs already resident in HBM:
  decode   forward       M=1,   K=2048, N=8192, gs=32,  fp16 x, fp16 scales
  prefill  forward       M=512, K=8192, N=2048, gs=128, bf16 x, fp16 scales
  qkv      fused QKV     M in {128, 508, 512}, K=2048, N=2048+512+512, gs=32, fp16 x
  bwd      input grad    M=512, N=8192, K=2048, gs=128, fp32 d_out ~ N(0, 0.1)
Outputs are fp32.  Several copies of every weight and activation are rotated so the
working set exceeds the 256 MB Infinity Cache and the weight stream comes from HBM.

Prints one JSON line: whole-step TFLOP/s (the step captured as a HIP graph per rotated
input set and replayed), per-op TFLOP/s and weight GB/s with their roofline fractions
(each op alone captured as a HIP graph of at least 32 launches over the rotated sets and
replayed between HIP events on the launch stream; the eager per-op time is kept beside it), the roofline object of the
dominant op and the fp64 CPU oracle timed on a bounded sample of the same step.
"""
import argparse
import copy
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0        # MI355X dense fp16 / bf16 MFMA
INT8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA
MALL_BYTES = 256 << 20
METRIC = "q4gsw linear TFLOP/s + weight GB/s (decode, prefill, QKV, bwd) vs roofline"
QKV_MS = (128, 508, 512)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--ops", default="decode,prefill,qkv,bwd,bwd_h,bwd_gs32,embedding,dq8ca,adapter",
                   help="comma-separated ops (embedding, dq8ca, adapter (its forward, backward and AdamW), "
                        "bwd_h, bwd_gs32 and the decode-shaped QKV are timed outside the step)")
    p.add_argument("--rotate", type=int, default=0, help="input sets rotated (0: enough to exceed the MALL)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=256, help="rows per M=512 op in the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB --steps times (counter calibration)")
    p.add_argument("--ingest-counters", nargs=4, metavar=("OP_FETCH", "OP_WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="rocprofv3 --pmc output dirs (FETCH_SIZE / WRITE_SIZE of a run of --ops OP and of "
                        "--copy-calibration); writes profiles/traffic.json for the op (no GPU needed)")
    p.add_argument("--copy-mib", type=int, default=256, help="size of the calibration copy (with --ingest-counters)")
    p.add_argument("--stream-floor", action="store_true",
                   help="only time a plain streaming read (torch's sum) of the decode weight bytes, cache-cold")
    return p.parse_args()


class Op:
    """One op of the step: its inputs (several rotated copies), flops and algorithmic bytes."""

    def __init__(self, name, kind, case, q, sets):
        import torch
        self.name, self.kind, self.case = name, kind, case
        self.in_step = True              # False: timed per op only, outside the step
        ws = case.weights
        self.M = case.M
        N = sum(w.N for w in ws)
        K = ws[0].K
        self.flops = 2.0 * self.M * N * K
        act = case.x if case.x is not None else case.d_out
        w_bytes = sum(w.N * w.K / 2 + w.scales.numel() * w.scales.element_size() for w in ws)
        self.weight_bytes = w_bytes
        out_elems = self.M * (K if kind == "bwd" else N)
        self.bytes = w_bytes + act.numel() * act.element_size() + 4.0 * out_elems
        self.sets = []
        for s in range(sets):
            pw = [q.pack(w.codes.cuda(), w.scales.cuda(), w.group_size) for w in ws]
            a = act.cuda()
            if kind == "bwd":
                outs = (torch.empty(self.M, K, dtype=torch.float32, device="cuda"),)
            else:
                outs = tuple(torch.empty(self.M, w.N, dtype=torch.float32, device="cuda") for w in ws)
            self.sets.append((pw, a, outs))
        pw0 = self.sets[0][0]
        if kind == "qkv":
            need = q.qkv_workspace_bytes(pw0[0], pw0[1], pw0[2], self.M, act.dtype)
            self.route = q.route(q.OP_QKV, pw0[0], self.M, act.dtype)
        elif kind == "bwd":
            need = q.workspace_bytes(q.OP_BWD_INPUT, pw0[0], self.M, act.dtype)
            self.route = q.route(q.OP_BWD_INPUT, pw0[0], self.M, act.dtype)
        elif kind == "dq8ca":
            need = q.workspace_bytes(q.OP_DQ8CA, pw0[0], self.M, act.dtype)
            self.route = q.route(q.OP_DQ8CA, pw0[0], self.M, act.dtype)
        else:
            need = q.workspace_bytes(q.OP_FWD, pw0[0], self.M, act.dtype)
            self.route = q.route(q.OP_FWD, pw0[0], self.M, act.dtype)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.set_bytes = sum(p.buffer.numel() for p in pw0) + act.numel() * act.element_size()
        # the int8 path runs on int8 MFMA; the others on fp16 / bf16 MFMA
        self.peak = INT8_PEAK_TOPS if kind == "dq8ca" else MFMA_PEAK_TFLOPS
        self.bound = "hbm" if self.flops / self.bytes < self.peak * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"

    def run(self, q, i):
        pw, a, outs = self.sets[i % len(self.sets)]
        if self.kind == "qkv":
            q.qkv_fused(pw[0], pw[1], pw[2], a, outs=outs, workspace=self.ws)
        elif self.kind == "bwd":
            q.linear_bwd_input(pw[0], a, out=outs[0], workspace=self.ws)
        elif self.kind == "dq8ca":
            q.linear_dq8ca(pw[0], a, out=outs[0], workspace=self.ws)
        else:
            q.linear_fwd(pw[0], a, out=outs[0], workspace=self.ws)


class EmbOp:
    """The embedding row gather (outside the step): T ids against a packed [N, K] table.
    Algorithmic bytes per token: the row's codes (K/2) and scales, its id and its fp32 row out."""

    def __init__(self, name, case, q, sets):
        import torch
        self.name, self.kind, self.case = name, "embedding", case
        self.in_step = False
        w = case.w
        self.M = case.M
        self.flops = 0.0
        row = w.K / 2 + (w.K // w.group_size) * w.scales.element_size()
        self.weight_bytes = self.M * row
        self.bytes = self.M * (row + 8 + 4.0 * w.K)
        self.sets = []
        for s in range(sets):
            pw = q.pack(w.codes.cuda(), w.scales.cuda(), w.group_size)
            self.sets.append((pw, case.ids.cuda(), torch.empty(self.M, w.K, dtype=torch.float32, device="cuda")))
        self.route = "embedding"
        self.bound = "hbm"
        self.peak = MFMA_PEAK_TFLOPS

    def run(self, q, i):
        pw, ids, out = self.sets[i % len(self.sets)]
        q.embedding(pw, ids, out=out)


class AdapterOp:
    """The adapter step around the frozen MLP up projection (outside the step): the adapter
    forward (y = x W^T + alpha (x A^T) B^T and t), its backward (d_x, d_A, d_B) or the AdamW
    update of the factors A [r, K] and B [N, r].  Algorithmic bytes are each call's inputs read
    once and outputs written once: forward W + x + A + B + y + t; backward W + d_out + x + A +
    B + t + d_x + d_A + d_B; AdamW 4 reads and 3 writes of the r (K + N) fp32 factor values."""

    def __init__(self, name, kind, case, q, sets):
        import torch
        from synthetic_inputs import ADAPTER_ALPHA
        self.name, self.kind, self.case = name, kind, case
        self.in_step = False
        self.alpha = ADAPTER_ALPHA
        w = case.w
        M, N, K, r = case.M, w.N, w.K, case.A.shape[0]
        self.M = M
        ab = case.x.element_size()
        wb = w.N * w.K / 2 + w.scales.numel() * w.scales.element_size()
        fac = 4.0 * r * (K + N)
        if kind == "adapter_fwd":
            self.flops = 2.0 * M * N * K + 2.0 * M * r * (K + N)
            self.weight_bytes = wb
            self.bytes = wb + M * K * ab + fac + 4.0 * M * N + 4.0 * M * r
        elif kind == "adapter_bwd":
            self.flops = 2.0 * M * N * K + 4.0 * M * r * (K + N)
            self.weight_bytes = wb
            self.bytes = wb + M * (N + K) * ab + fac + 4.0 * M * r + 4.0 * M * K + fac
        else:
            self.flops = 0.0
            self.weight_bytes = 0.0
            self.bytes = 7 * fac
        self.sets = []
        for s in range(sets):
            pw = q.pack(w.codes.cuda(), w.scales.cuda(), w.group_size)
            st = {"pw": pw, "x": case.x.cuda(), "d": case.d_out.cuda(), "A": case.A.cuda(), "B": case.B.cuda()}
            st["y"] = torch.empty(M, N, dtype=torch.float32, device="cuda")
            st["t"] = torch.empty(M, r, dtype=torch.float32, device="cuda")
            st["dx"] = torch.empty(M, K, dtype=torch.float32, device="cuda")
            st["dA"] = torch.empty(r, K, dtype=torch.float32, device="cuda")
            st["dB"] = torch.empty(N, r, dtype=torch.float32, device="cuda")
            # the optimizer state of both factors in one flat buffer each (A's values, then B's)
            n = r * (K + N)
            st["p"] = torch.cat([case.A.reshape(-1), case.B.reshape(-1)]).cuda()
            st["g"] = torch.randn(n, generator=torch.Generator().manual_seed(s)).mul_(1e-3).cuda()
            st["m"] = torch.zeros(n, device="cuda")
            st["v"] = torch.zeros(n, device="cuda")
            self.sets.append(st)
        op = q.OP_FWD if kind == "adapter_fwd" else q.OP_BWD_INPUT
        need = q.adapter_workspace_bytes(op, self.sets[0]["pw"], M, case.x.dtype, r)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        self.route = "adamw" if kind == "adamw" else q.route(op, self.sets[0]["pw"], M, case.x.dtype)
        self.peak = MFMA_PEAK_TFLOPS
        self.bound = "hbm" if kind == "adamw" or self.flops / self.bytes < self.peak * 1e12 / (
            HBM_PEAK_GBS * 1e9) else "mfma"
        self.steps_done = 0

    def run(self, q, i):
        st = self.sets[i % len(self.sets)]
        if self.kind == "adapter_fwd":
            q.adapter_fwd(st["pw"], st["x"], st["A"], st["B"], self.alpha, out=st["y"], t=st["t"], workspace=self.ws)
        elif self.kind == "adapter_bwd":
            q.adapter_bwd(st["pw"], st["x"], st["d"], st["A"], st["B"], self.alpha, st["t"], d_x=st["dx"],
                          d_A=st["dA"], d_B=st["dB"], workspace=self.ws)
        else:
            # the step count only sets the bias corrections; a fixed one keeps captured replays alike
            q.adamw_step(st["p"], st["g"], st["m"], st["v"], 10, 1e-4, 0.9, 0.999, 1e-8, 0.01)


def torch_dtype(name):
    from synthetic_inputs import DTYPES
    return DTYPES[name]


def build_ops(q, names, rotate):
    from synthetic_inputs import make_linear, make_workload
    specs = []
    for n in names:
        if n == "decode":
            specs.append(("decode", "fwd", make_workload("decode")))
        elif n == "prefill":
            specs.append(("prefill", "fwd", make_workload("prefill")))
        elif n.startswith("qkv_m") and n[5:].isdigit():
            # one QKV row count alone (counter runs)
            specs.append((n, "qkv", make_workload("qkv", M=int(n[5:]))))
        elif n == "qkv":
            for M in QKV_MS:
                specs.append((f"qkv_m{M}", "qkv", make_workload("qkv", M=M)))
            # the decode-shaped triples (one launch of the streaming GEMV), outside the step
            specs.append(("qkv_m1", "qkv", make_workload("qkv", M=1)))
            specs.append(("qkv_m4", "qkv", make_workload("qkv", M=4)))
        elif n == "bwd":
            specs.append(("bwd", "bwd", make_workload("bwd")))
        elif n == "bwd_h":
            # outside the step: the bwd workload with d_out rounded to fp16 (fold route)
            h = copy.copy(make_workload("bwd"))
            h.d_out = h.d_out.to(torch_dtype("f16"))
            specs.append(("bwd_h", "bwd", h))
        elif n == "bwd_gs32":
            # outside the step: the input gradient through the Llama Q projection (N = K = 2048,
            # gs = 32, fp32 d_out)
            specs.append(("bwd_gs32", "bwd", make_linear(512, 2048, 2048, 32, "f32", "f16", seed=0, fwd=False,
                                                         bwd=True, sigma=0.1)))
        elif n == "dq8ca":
            # the prefill workload with its activation rows quantised to int8 per row, outside the step
            specs.append(("dq8ca", "dq8ca", make_workload("prefill")))
        elif n in ("adapter", "adapter_fwd", "adapter_bwd", "adamw"):
            # the adapter step around the frozen MLP up projection (M=512, rank 16), outside the step
            ad = make_workload("adapter")
            for k in ("adapter_fwd", "adapter_bwd", "adamw"):
                if n in ("adapter", k):
                    specs.append((k, k, ad))
        elif n in ("embedding", "emb_t512", "emb_t1"):
            # the row gather from the tied embedding table, outside the step: 512 ids and one id
            emb = make_workload("embedding")
            if n != "emb_t1":
                specs.append(("emb_t512", "embedding", emb))
            if n != "emb_t512":
                one = copy.copy(emb)
                one.M, one.ids = 1, emb.ids[:1].clone()
                specs.append(("emb_t1", "embedding", one))
        else:
            raise SystemExit(f"unknown op {n}")
    def set_bytes(case):
        if case.A is not None:
            return sum(w.N * w.K / 2 + w.scales.numel() * 2 for w in case.weights) + \
                (case.x.numel() + case.d_out.numel()) * case.x.element_size()
        if case.ids is not None:
            return sum(w.N * w.K / 2 + w.scales.numel() * 2 for w in case.weights)
        act = case.x if case.x is not None else case.d_out
        return sum(w.N * w.K / 2 + w.scales.numel() * 2 for w in case.weights) + act.numel() * act.element_size()

    extra = {"qkv_m1", "qkv_m4", "emb_t512", "emb_t1", "bwd_h", "bwd_gs32", "dq8ca", "adapter_fwd", "adapter_bwd",
             "adamw"}
    if rotate <= 0:
        # the step rotates enough sets of every op to exceed the MALL; each op also gets enough
        # copies of its own to exceed it alone, for its per-op timing
        step_bytes = sum(set_bytes(c) for n, _, c in specs if n not in extra) or \
            sum(set_bytes(c) for _, _, c in specs)
        rotate = max(2, int(MALL_BYTES * 1.5 // step_bytes) + 1)
        per_op = [max(rotate, int(MALL_BYTES * 1.5 // set_bytes(c)) + 1) for _, _, c in specs]
    else:
        per_op = [rotate] * len(specs)
    def make(n, k, c, sets):
        if k == "embedding":
            return EmbOp(n, c, q, sets)
        if k in ("adapter_fwd", "adapter_bwd", "adamw"):
            return AdapterOp(n, k, c, q, sets)
        return Op(n, k, c, q, sets)

    ops = [make(n, k, c, sets) for (n, k, c), sets in zip(specs, per_op)]
    for op in ops:
        op.in_step = op.name not in extra
    if not any(op.in_step for op in ops):
        # a run of ops that are normally outside the step (counter runs): they form the step
        for op in ops:
            op.in_step = True
    return ops, rotate


# the sources an op's kernels are built from: the shared headers and the entry points (which
# plan the launch), plus the files holding its kernels
_COMMON_SRC = ("api.hip", "device.h", "internal.h", "layout.h")
_OP_SRC = {"decode": ("gemv.hip",), "qkv_m1": ("gemv.hip", "reduce.hip"), "qkv_m4": ("gemv.hip", "reduce.hip"),
           "prefill": ("gemm_fwd.hip", "reduce.hip"), "qkv_m128": ("gemm_fwd.hip", "reduce.hip"),
           "qkv_m508": ("gemm_fwd.hip", "reduce.hip"), "qkv_m512": ("gemm_fwd.hip", "reduce.hip"),
           "bwd": ("gemm_bwd2.hip", "gemm_bwd.hip", "reduce.hip"), "bwd_h": ("gemm_bwd2.hip", "gemm_bwd.hip", "reduce.hip"),
           "bwd_gs32": ("gemm_bwd2.hip", "gemm_bwd.hip", "reduce.hip"), "emb_t512": ("embedding.hip",),
           "emb_t1": ("embedding.hip",), "dq8ca": ("dq8ca.hip", "reduce.hip"),
           "adapter_fwd": ("adapter.hip", "gemm_fwd.hip", "reduce.hip"),
           "adapter_bwd": ("adapter.hip", "gemm_bwd2.hip", "gemm_bwd.hip", "reduce.hip"), "adamw": ("adapter.hip",)}


def source_hash(op_name=None):
    """Hash of the kernel sources: of every file, or of those an op's kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_group_quantized_q4gsw_amd", "csrc")
    files = sorted(os.listdir(csrc)) if op_name is None else sorted(_COMMON_SRC + _OP_SRC[op_name])
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(op_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on the op's current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(op_name)
    if not ent or ent.get("src_hash") != source_hash(op_name):
        return None
    return ent.get("bytes_per_launch")


# kernels that make up one launch of each op (a GEMM and, with K splits, its reduction)
OP_KERNELS = {"decode": ("gemv_fwd",), "prefill": ("gemm_fwd", "reduce_"),
              "qkv_m128": ("gemm_fwd", "reduce_"), "qkv_m508": ("gemm_fwd", "reduce_"),
              "qkv_m512": ("gemm_fwd", "reduce_"), "bwd": ("gemm_bwd", "reduce_"),
              "bwd_h": ("gemm_bwd", "reduce_"), "bwd_gs32": ("gemm_bwd", "reduce_", "split_planes"),
              "emb_t512": ("embedding_kernel",), "emb_t1": ("embedding_kernel",),
              "dq8ca": ("dq8ca_", "reduce_"),
              "adapter_fwd": ("gemm_fwd", "reduce_", "row_partial", "expand_kernel"),
              "adapter_bwd": ("gemm_bwd", "reduce_", "row_partial", "expand_kernel", "column_"),
              "adamw": ("adamw_kernel",)}


def _counter_means(d, counter):
    """Mean counter value per dispatch, per kernel-name family, from a rocprofv3 --pmc CSV dir."""
    import csv
    import glob
    sums = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            v = float(r["Counter_Value"])
            s = sums.setdefault(name, [0.0, 0])
            s[0] += v
            s[1] += 1
    return {k: v[0] / v[1] for k, v in sums.items()}


def ingest_counters(op_name, op_fetch, op_write, copy_fetch, copy_write, copy_mib):
    """HBM bytes per launch of op_name = (FETCH_SIZE + WRITE_SIZE of its kernels) scaled by what the
    same counters read for a plain copy of copy_mib MiB (bytes moved / counter reading)."""
    cf = _counter_means(copy_fetch, "FETCH_SIZE")
    cw = _counter_means(copy_write, "WRITE_SIZE")
    copy_bytes = float(int(copy_mib) << 20)
    # the calibration run holds only the copy; take its most frequent large-count kernel
    kf = max(cf.values())
    kw = max(cw.values())
    f_fetch = copy_bytes / kf
    f_write = copy_bytes / kw
    of = _counter_means(op_fetch, "FETCH_SIZE")
    ow = _counter_means(op_write, "WRITE_SIZE")
    fams = OP_KERNELS.get(op_name, ())
    fetch = sum(v for k, v in of.items() if any(fm in k for fm in fams))
    write = sum(v for k, v in ow.items() if any(fm in k for fm in fams))
    ent = {"bytes_per_launch": round(fetch * f_fetch + write * f_write), "fetch_bytes": round(fetch * f_fetch),
           "write_bytes": round(write * f_write), "fetch_counter": round(fetch, 1), "write_counter": round(write, 1),
           "copy_mib": copy_mib, "copy_fetch_counter": round(kf, 1), "copy_write_counter": round(kw, 1),
           "scale_fetch": f_fetch, "scale_write": f_write, "kernels": list(fams), "src_hash": source_hash(op_name)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        data = json.load(open(path))
    data[op_name] = ent
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({op_name: ent}))


def copy_calibration(mib, steps):
    import torch
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "steps": steps}))


def stream_floor(steps):
    """Per-launch time of plain streaming reads of the decode workload's weight bytes (codes and
    scales of the [8192, 2048] gs-32 fp16-scale weight) and of 1 GiB, with PyTorch's own kernels:
    a row reduction (sum over rows of 1024 floats), a full sum and a device copy (which also writes
    the bytes).  Each runs over enough rotated copies to exceed the MALL, as a HIP graph between
    HIP events.  The fastest read is an upper bound on what a streaming read of that size costs."""
    import torch
    out = {}
    for label, nbytes in (("decode_weight_bytes", 8192 * 2048 // 2 + (2048 // 32) * 8192 * 2), ("1GiB", 1 << 30)):
        n = nbytes // 4
        sets = max(2, int(MALL_BYTES * 1.5 // nbytes) + 1)
        bufs = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(sets)]
        dst = torch.empty(n, dtype=torch.float32, device="cuda")
        rows = torch.empty(n // 1024, dtype=torch.float32, device="cuda")
        res = torch.empty((), dtype=torch.float32, device="cuda")
        kinds = {"row_sum": lambda b: torch.sum(b.view(-1, 1024), dim=1, out=rows),
                 "full_sum": lambda b: torch.sum(b, dim=0, out=res),
                 "copy": lambda b: dst.copy_(b)}
        launches = sets * max(1, (32 + sets - 1) // sets)
        ent = {"bytes": n * 4, "sets": sets, "launches_per_graph": launches}
        for kname, fn in kinds.items():
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(launches):
                    fn(bufs[i % sets])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            reps = max(3, steps)
            a.record()
            for _ in range(reps):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / (reps * launches)
            ent[kname] = {"us_per_launch": round(us, 3), "read_gbs": round(n * 4 / us / 1e3, 1)}
            del g
        out[label] = ent
        del bufs
    print(json.dumps({"stream_floor": out}), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(ops, rows_per_op):
    """The fp64 oracle (as it stands) on a bounded sample of the step: the first rows of each op,
    with the host's threads (up to 16); then one thread on the first sixteenth of those rows, whose
    outputs must equal the multi-threaded ones bit for bit (the oracle splits outputs, never sums,
    across threads)."""
    import numpy as np
    from oracle import oracle as O
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or min(16, os.cpu_count() or 1)
    used = O.default().threads_used(threads)

    def run(nthreads, frac):
        flops = 0.0
        parts, outs = [], []
        t0 = time.perf_counter()
        for op in ops:
            c = op.case
            rows = max(1, min(op.M, rows_per_op) // frac)
            if op.kind == "bwd":
                d = c.d_out[:rows].contiguous()
                outs.append(O.linear_bwd_input(d, c.w.codes, c.w.scales, c.w.group_size, threads=nthreads)[0])
                flops += 2.0 * rows * c.w.N * c.w.K
            else:
                x = c.x[:rows].contiguous()
                for w in c.weights:
                    outs.append(O.linear_fwd(x, w.codes, w.scales, w.group_size, threads=nthreads)[0])
                    flops += 2.0 * rows * w.N * w.K
            parts.append(f"{op.name}:{rows}/{op.M} rows")
        return flops, time.perf_counter() - t0, parts, outs

    flops, dt, parts, outs = run(threads, 1)
    flops1, dt1, parts1, outs1 = run(1, 16)
    same = all(np.array_equal(a[: b.shape[0]], b) for a, b in zip(outs, outs1))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": "fp64 oracle on the first rows of each op (" + ", ".join(parts) +
                      f"); {flops / 1e9:.2f} GFLOP in {dt:.1f} s",
            "cpu_model": _cpu_model(),
            "single_thread": {"value": flops1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": "the first sixteenth of those rows (" + ", ".join(parts1) +
                                        f"); {flops1 / 1e9:.2f} GFLOP in {dt1:.1f} s",
                              "bitwise_equal_to_threaded": bool(same)}}


def main():
    args = parse()
    if args.ingest_counters:
        ops = [n.strip() for n in args.ops.split(",") if n.strip()]
        if len(ops) != 1:
            raise SystemExit("--ingest-counters takes exactly one op name in --ops")
        ingest_counters(ops[0], *args.ingest_counters, copy_mib=args.copy_mib)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        torch.cuda.set_device(0)
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.stream_floor:
        torch.cuda.set_device(0)
        stream_floor(args.steps)
        return
    import bit_group_quantized_q4gsw_amd as q
    torch.cuda.set_device(0)
    names = [n.strip() for n in args.ops.split(",") if n.strip()]
    ops, rotate = build_ops(q, names, args.rotate)
    torch.cuda.synchronize()

    step_ops = [op for op in ops if op.in_step]
    for i in range(args.warmup):
        for op in ops:
            op.run(q, i)
    torch.cuda.synchronize()

    # per-op timing: eager launches, each bracketed by HIP events on the launch stream (the ops
    # outside the step in a loop of their own)
    ev = {op.name: [] for op in ops}
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)

    def eager(group):
        for i in range(args.steps):
            for op in group:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                op.run(q, args.warmup + i)
                b.record()
                ev[op.name].append((a, b))

    start.record()
    eager(step_ops)
    stop.record()
    torch.cuda.synchronize()
    eager_ms_step = start.elapsed_time(stop) / args.steps
    eager([op for op in ops if not op.in_step])
    torch.cuda.synchronize()

    # whole-step timing: each rotated input set's step captured once as a HIP graph and
    # replayed, so host launch latency does not pace the GPU
    graphs = []
    for s in range(rotate):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for op in step_ops:
                op.run(q, s)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % rotate].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        graphs[i % rotate].replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps

    # per-op timing without host launch latency: each op alone, whole passes over its own rotated
    # input sets (which alone exceed the MALL; at least 32 launches, so the graph launch itself
    # is amortised), captured as a HIP graph and replayed between HIP events
    graph_ms = {}
    for op in ops:
        nset = len(op.sets)
        launches = nset * ((32 + nset - 1) // nset)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(launches):
                op.run(q, s)
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        reps = max(3, (args.steps + launches - 1) // launches)
        start.record()
        for _ in range(reps):
            g.replay()
        stop.record()
        torch.cuda.synchronize()
        graph_ms[op.name] = start.elapsed_time(stop) / (reps * launches)
        del g

    per_op = {}
    total_flops = 0.0
    for op in ops:
        eager_ms = sum(a.elapsed_time(b) for a, b in ev[op.name]) / args.steps
        ms = graph_ms[op.name]
        s = ms / 1e3
        tflops = op.flops / s / 1e12
        gbs = op.bytes / s / 1e9
        wgbs = op.weight_bytes / s / 1e9
        frac = gbs / HBM_PEAK_GBS if op.bound == "hbm" else tflops / op.peak
        per_op[op.name] = {"ms": round(ms, 5), "eager_ms": round(eager_ms, 5), "in_step": op.in_step,
                           "tflops": round(tflops, 2),
                           "weight_gbs": round(wgbs, 1),
                           "alg_gbs": round(gbs, 1), "bound": op.bound, "roofline_frac": round(frac, 4),
                           "route": op.route, "M": op.M, "peak": op.peak if op.bound != "hbm" else HBM_PEAK_GBS,
                           "traffic": traffic_for(op.name)}
        if op.in_step:
            total_flops += op.flops

    dom = max(step_ops, key=lambda o: per_op[o.name]["ms"])
    d = per_op[dom.name]
    src = source_hash()
    if dom.bound == "hbm":
        roof = {"bound": "hbm", "achieved": d["alg_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(d["alg_gbs"] / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": d["tflops"], "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(d["tflops"] / MFMA_PEAK_TFLOPS, 4)}
    roof["traffic"] = traffic_for(dom.name)
    roof["op"] = dom.name
    roof["route"] = dom.route
    roof["per_launch_ms"] = d["ms"]

    line = {
        "metric": METRIC,
        "value": round(total_flops / (ms_step / 1e3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16/f16/f32",
        "data": "synthetic",
        "config": {"workload": "llama-3.2-1b q4gsw step: " + ", ".join(
            f"{o.name} M{o.M} route={o.route}" for o in step_ops), "ops": names, "rotated_sets": rotate,
            "outside_step": [o.name for o in ops if not o.in_step],
            "op_sets": {o.name: len(o.sets) for o in ops},
            "timing": "step: HIP-graph replay of the whole step; per_op ms: HIP-graph replay of the op alone, "
                      ">= 32 launches over the rotated sets (eager_ms: eager launches between HIP events)",
            "eager_ms_per_step": round(eager_ms_step, 5), "wall_s": round(wall, 3), "src_hash": src},
        "per_op": per_op,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(step_ops, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
