"""Thin ctypes binding of libq4gsw.so (include/q4gsw.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory (output and workspace
tensors) and the current HIP stream.  There is no CPU fallback: importing the
package without the built library raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4gsw.so")

F32, F16, BF16 = 0, 1, 2
OP_FWD, OP_BWD_INPUT, OP_QKV, OP_DQ8CA = 0, 1, 2, 3
ROUTES = {
    "none": 0, "generic": 1, "gemv": 2, "gemm_fold": 3, "gemm_group": 4, "gemm_split": 5,
    "bwd_gemv": 6, "bwd_fold": 7, "bwd_split": 8, "qkv_fused": 9, "bwd_bsplit": 10, "dq8ca": 11,
}
FLAG_FOLD_F16 = 1
_TORCH_DTYPE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}


class Q4gswError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


class WeightDesc(ctypes.Structure):
    """Mirror of struct q4gsw_weight."""
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("group_size", ctypes.c_int64),
        ("n_pad", ctypes.c_int64), ("k_pad", ctypes.c_int64), ("g_pad", ctypes.c_int64),
        ("scale_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("data", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
        ("nibble_offset", ctypes.c_uint64), ("scale_offset", ctypes.c_uint64),
    ]


class PlanInfo(ctypes.Structure):
    """q4gsw_plan_info of include/q4gsw.h."""
    _fields_ = [("route", ctypes.c_int32), ("tile_rows", ctypes.c_int32), ("splits", ctypes.c_int32)]


class Options(ctypes.Structure):
    """q4gsw_options of include/q4gsw.h: a per-call route family, block rows and split count."""
    _fields_ = [("route", ctypes.c_int32), ("tile_rows", ctypes.c_int32), ("splits", ctypes.c_int32)]


class AdamwParams(ctypes.Structure):
    """q4gsw_adamw_params of include/q4gsw.h."""
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


# Choices made by forced_route / forced_plan, held per Python thread and handed to each call
# (the library itself keeps no routing state).
_local = threading.local()


def _opts():
    """The current thread's options, or None (library defaults)."""
    o = getattr(_local, "opts", None)
    if o is None or (o.route == 0 and o.tile_rows == 0 and o.splits == 0):
        return None
    return ctypes.byref(o)


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python bit_group_quantized_q4gsw_amd/build.py; "
                              "there is no CPU fallback")
        h = ctypes.CDLL(LIB_PATH)
        i32, i64, u64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
        pw = ctypes.POINTER(WeightDesc)
        po = ctypes.POINTER(Options)
        sigs = {
            "q4gsw_packed_bytes": [i64, i64, i64, i32, ctypes.POINTER(u64)],
            "q4gsw_pack": [vp, vp, i32, i64, i64, i64, vp, u64, vp, pw],
            "q4gsw_unpack": [pw, vp, vp, vp],
            "q4gsw_workspace_bytes": [i32, pw, i64, i32, ctypes.POINTER(u64)],
            "q4gsw_qkv_workspace_bytes": [pw, pw, pw, i64, i32, ctypes.POINTER(u64)],
            "q4gsw_workspace_bytes_ex": [i32, pw, i64, i32, po, ctypes.POINTER(u64)],
            "q4gsw_qkv_workspace_bytes_ex": [pw, pw, pw, i64, i32, po, ctypes.POINTER(u64)],
            "q4gsw_linear_fwd": [pw, vp, i32, i64, vp, vp, u64, vp],
            "q4gsw_linear_bwd_input": [pw, vp, i32, i64, vp, vp, u64, vp],
            "q4gsw_qkv_fused": [pw, pw, pw, vp, i32, i64, vp, vp, vp, vp, u64, vp],
            "q4gsw_linear_fwd_ex": [pw, vp, i32, i64, vp, vp, u64, po, vp],
            "q4gsw_linear_fwd_noalloc": [pw, vp, i32, i64, vp, vp],
            "q4gsw_linear_bwd_input_ex": [pw, vp, i32, i64, vp, vp, u64, po, vp],
            "q4gsw_qkv_fused_ex": [pw, pw, pw, vp, i32, i64, vp, vp, vp, vp, u64, po, vp],
            "q4gsw_route": [i32, pw, i64, i32],
            "q4gsw_plan": [i32, pw, pw, pw, i64, i32, po, ctypes.POINTER(PlanInfo)],
            "q4gsw_embedding": [pw, vp, i64, vp, vp],
            "q4gsw_dq8ca_quantize": [vp, i32, i64, i64, vp, vp, vp, vp],
            "q4gsw_linear_dq8ca": [pw, vp, i32, i64, vp, vp, u64, vp],
            "q4gsw_linear_dq8ca_ex": [pw, vp, i32, i64, vp, vp, u64, po, vp],
            "q4gsw_adapter_workspace_bytes": [i32, pw, i64, i32, i32, ctypes.POINTER(u64)],
            "q4gsw_adapter_fwd": [pw, vp, i32, i64, vp, vp, i32, ctypes.c_float, vp, vp, vp, u64, vp],
            "q4gsw_adapter_bwd": [pw, vp, vp, i32, i64, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, u64, vp],
            "q4gsw_adamw_step": [vp, vp, vp, vp, i64, ctypes.POINTER(AdamwParams), i64, vp],
        }
        for name, args in sigs.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        h.q4gsw_route_name.argtypes = [i32]
        h.q4gsw_route_name.restype = ctypes.c_char_p
        h.q4gsw_status_str.argtypes = [i32]
        h.q4gsw_status_str.restype = ctypes.c_char_p
        h.q4gsw_layout_version.argtypes = []
        h.q4gsw_layout_version.restype = ctypes.c_uint32
        h.q4gsw_build_info.argtypes = []
        h.q4gsw_build_info.restype = ctypes.c_char_p
        _lib = h
    return _lib


def status_str(status: int) -> str:
    return lib().q4gsw_status_str(status).decode()


def route_name(route: int) -> str:
    return lib().q4gsw_route_name(route).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise Q4gswError(status, what)


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return t.contiguous()


def _out(out: Optional[torch.Tensor], shape: Tuple[int, ...], device, name: str) -> torch.Tensor:
    """A caller's output tensor, checked against what the kernels write (contiguous fp32 of
    exactly `shape` on `device`), or a new one."""
    if out is None:
        return torch.empty(*shape, dtype=torch.float32, device=device)
    if (out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != tuple(shape)
            or out.device != device):
        raise ValueError(f"{name} must be a contiguous fp32 tensor of shape {list(shape)} on {device}")
    return out


class PackedWeight:
    """A packed q4gsw weight: the descriptor plus the device buffer it points into."""

    def __init__(self, desc: WeightDesc, buffer: torch.Tensor):
        self.desc = desc
        self.buffer = buffer

    @property
    def N(self) -> int:
        return self.desc.N

    @property
    def K(self) -> int:
        return self.desc.K

    @property
    def group_size(self) -> int:
        return self.desc.group_size

    @property
    def foldable(self) -> bool:
        return bool(self.desc.flags & FLAG_FOLD_F16)

    def ref(self):
        return ctypes.byref(self.desc)


def packed_bytes(N: int, K: int, group_size: int, scale_dtype: torch.dtype) -> int:
    out = ctypes.c_uint64()
    _check(lib().q4gsw_packed_bytes(N, K, group_size, _TORCH_DTYPE[scale_dtype], ctypes.byref(out)),
           "q4gsw_packed_bytes")
    return out.value


def pack(codes: torch.Tensor, scales: torch.Tensor, group_size: int) -> PackedWeight:
    """codes uint8 [N, K] (0..15) and scales [K/group_size, N] (fp16/fp32), both on the GPU."""
    codes = _dev(codes, "codes")
    scales = _dev(scales, "scales")
    if codes.dtype != torch.uint8 or codes.dim() != 2:
        raise ValueError("codes must be uint8 [N, K]")
    N, K = codes.shape
    if scales.dtype not in (torch.float16, torch.float32):
        raise ValueError("scales must be fp16 or fp32")
    if group_size < 1 or K % group_size or tuple(scales.shape) != (K // group_size, N):
        raise ValueError("scales must be [K / group_size, N]")
    nbytes = packed_bytes(N, K, group_size, scales.dtype)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    desc = WeightDesc()
    _check(lib().q4gsw_pack(codes.data_ptr(), scales.data_ptr(), _TORCH_DTYPE[scales.dtype], N, K, group_size,
                            buf.data_ptr(), nbytes, _stream(), ctypes.byref(desc)), "q4gsw_pack")
    return PackedWeight(desc, buf)


def unpack(w: PackedWeight) -> Tuple[torch.Tensor, torch.Tensor]:
    dev = w.buffer.device
    codes = torch.empty(w.N, w.K, dtype=torch.uint8, device=dev)
    sdt = torch.float16 if w.desc.scale_dtype == F16 else torch.float32
    scales = torch.empty(w.K // w.group_size, w.N, dtype=sdt, device=dev)
    _check(lib().q4gsw_unpack(w.ref(), codes.data_ptr(), scales.data_ptr(), _stream()), "q4gsw_unpack")
    return codes, scales


def _workspace(nbytes: int, device) -> Tuple[Optional[torch.Tensor], int, int]:
    if nbytes == 0:
        return None, 0, 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, ws.data_ptr(), nbytes


def workspace_bytes(op: int, w: PackedWeight, M: int, dtype: torch.dtype) -> int:
    out = ctypes.c_uint64()
    _check(lib().q4gsw_workspace_bytes_ex(op, w.ref(), M, _TORCH_DTYPE[dtype], _opts(), ctypes.byref(out)),
           "q4gsw_workspace_bytes")
    return out.value


def _ws_args(need: int, workspace: Optional[torch.Tensor], device):
    """(tensor kept alive, pointer, bytes): the caller's workspace when it is a large enough uint8
    tensor on `device`, else a new one."""
    if workspace is not None and workspace.dtype == torch.uint8 and workspace.is_contiguous() \
            and workspace.device == device and workspace.numel() >= need:
        return workspace, workspace.data_ptr(), workspace.numel()
    return _workspace(need, device)


def linear_fwd(w: PackedWeight, x: torch.Tensor, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M, N] fp32 = x [M, K] . dequant(W)^T."""
    x = _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    y = _out(out, (M, w.N), x.device, "out")
    need = workspace_bytes(OP_FWD, w, M, x.dtype)
    ws, wp, wb = _ws_args(need, workspace, x.device)
    _check(lib().q4gsw_linear_fwd_ex(w.ref(), x.data_ptr(), _TORCH_DTYPE[x.dtype], M, y.data_ptr(), wp, wb,
                                     _opts(), _stream()), "q4gsw_linear_fwd")
    return y


def linear_fwd_noalloc(w: PackedWeight, x: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """y [M, N] fp32 = x [M, K] . dequant(W)^T into the caller's `out`, through the entry point that
    allocates nothing (its split partials live in the library's per-device scratch; calls that
    overlap on one device race on it).  Raises Q4gswError (E_SCRATCH) when the call would need more
    scratch than the library holds."""
    x = _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    if out is None:
        raise ValueError("out is required: this entry point allocates nothing")
    y = _out(out, (M, w.N), x.device, "out")
    _check(lib().q4gsw_linear_fwd_noalloc(w.ref(), x.data_ptr(), _TORCH_DTYPE[x.dtype], M, y.data_ptr(), _stream()),
           "q4gsw_linear_fwd_noalloc")
    return y


def linear_bwd_input(w: PackedWeight, d_out: torch.Tensor, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """d_x [M, K] fp32 = d_out [M, N] . dequant(W), contracting over N."""
    d_out = _dev(d_out, "d_out")
    if d_out.dim() != 2 or d_out.shape[1] != w.N:
        raise ValueError("d_out must be [M, N]")
    M = d_out.shape[0]
    dx = _out(out, (M, w.K), d_out.device, "out")
    need = workspace_bytes(OP_BWD_INPUT, w, M, d_out.dtype)
    ws, wp, wb = _ws_args(need, workspace, d_out.device)
    _check(lib().q4gsw_linear_bwd_input_ex(w.ref(), d_out.data_ptr(), _TORCH_DTYPE[d_out.dtype], M,
                                           dx.data_ptr(), wp, wb, _opts(), _stream()), "q4gsw_linear_bwd_input")
    return dx


def dq8ca_quantize(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Per-row int8 quantisation of x [M, K]: (q int8 [M, K], scale fp32 [M], zero_point int32 [M])."""
    x = _dev(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    q = torch.empty(M, K, dtype=torch.int8, device=x.device)
    scale = torch.empty(M, dtype=torch.float32, device=x.device)
    zp = torch.empty(M, dtype=torch.int32, device=x.device)
    _check(lib().q4gsw_dq8ca_quantize(x.data_ptr(), _TORCH_DTYPE[x.dtype], M, K, q.data_ptr(), scale.data_ptr(),
                                      zp.data_ptr(), _stream()), "q4gsw_dq8ca_quantize")
    return q, scale, zp


def linear_dq8ca(w: PackedWeight, x: torch.Tensor, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M, N] fp32 = the forward of x's rows quantised to int8 per row (linear_dq8ca_q4gsw)."""
    x = _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    y = _out(out, (M, w.N), x.device, "out")
    need = workspace_bytes(OP_DQ8CA, w, M, x.dtype)
    ws, wp, wb = _ws_args(need, workspace, x.device)
    _check(lib().q4gsw_linear_dq8ca_ex(w.ref(), x.data_ptr(), _TORCH_DTYPE[x.dtype], M, y.data_ptr(), wp, wb,
                                       _opts(), _stream()), "q4gsw_linear_dq8ca")
    return y


def adapter_workspace_bytes(op: int, w: PackedWeight, M: int, dtype: torch.dtype, rank: int) -> int:
    out = ctypes.c_uint64()
    _check(lib().q4gsw_adapter_workspace_bytes(op, w.ref(), M, _TORCH_DTYPE[dtype], rank, ctypes.byref(out)),
           "q4gsw_adapter_workspace_bytes")
    return out.value


def _factor(t: torch.Tensor, shape: Tuple[int, int], device, name: str) -> torch.Tensor:
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError(f"{name} must be an fp32 tensor of shape {list(shape)} on {device}")
    return t.contiguous()


def adapter_fwd(w: PackedWeight, x: torch.Tensor, A: torch.Tensor, B: torch.Tensor, alpha: float,
                out: Optional[torch.Tensor] = None, t: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(y [M, N], t [M, r]) = (x . dequant(W)^T + alpha (x A^T) B^T, x A^T) for the low-rank
    adapter A [r, K], B [N, r] (fp32) beside the frozen weight."""
    x = _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != w.K:
        raise ValueError("x must be [M, K]")
    M, r = x.shape[0], A.shape[0]
    A = _factor(A, (r, w.K), x.device, "A")
    B = _factor(B, (w.N, r), x.device, "B")
    y = _out(out, (M, w.N), x.device, "out")
    t = _out(t, (M, r), x.device, "t")
    need = adapter_workspace_bytes(OP_FWD, w, M, x.dtype, r)
    ws, wp, wb = _ws_args(need, workspace, x.device)
    _check(lib().q4gsw_adapter_fwd(w.ref(), x.data_ptr(), _TORCH_DTYPE[x.dtype], M, A.data_ptr(), B.data_ptr(), r,
                                   float(alpha), y.data_ptr(), t.data_ptr(), wp, wb, _stream()), "q4gsw_adapter_fwd")
    return y, t


def adapter_bwd(w: PackedWeight, x: torch.Tensor, d_out: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                alpha: float, t: torch.Tensor, d_x: Optional[torch.Tensor] = None,
                d_A: Optional[torch.Tensor] = None, d_B: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(d_x [M, K], d_A [r, K], d_B [N, r]): the gradients of <d_out, y> for the adapter forward of
    the same x (t is its x A^T)."""
    x = _dev(x, "x")
    d_out = _dev(d_out, "d_out")
    if x.dim() != 2 or x.shape[1] != w.K or d_out.shape != (x.shape[0], w.N) or d_out.dtype != x.dtype:
        raise ValueError("x must be [M, K] and d_out [M, N] of x's dtype")
    M, r = x.shape[0], A.shape[0]
    A = _factor(A, (r, w.K), x.device, "A")
    B = _factor(B, (w.N, r), x.device, "B")
    t = _factor(t, (M, r), x.device, "t")
    dx = _out(d_x, (M, w.K), x.device, "d_x")
    dA = _out(d_A, (r, w.K), x.device, "d_A")
    dB = _out(d_B, (w.N, r), x.device, "d_B")
    need = adapter_workspace_bytes(OP_BWD_INPUT, w, M, x.dtype, r)
    ws, wp, wb = _ws_args(need, workspace, x.device)
    _check(lib().q4gsw_adapter_bwd(w.ref(), x.data_ptr(), d_out.data_ptr(), _TORCH_DTYPE[x.dtype], M, A.data_ptr(),
                                   B.data_ptr(), r, float(alpha), t.data_ptr(), dx.data_ptr(), dA.data_ptr(),
                                   dB.data_ptr(), wp, wb, _stream()), "q4gsw_adapter_bwd")
    return dx, dA, dB


def adamw_step(param: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor,
               step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
               weight_decay: float = 0.01) -> None:
    """One AdamW step in place on contiguous fp32 GPU tensors of one size (param, exp_avg and
    exp_avg_sq are updated)."""
    ts = [param, grad, exp_avg, exp_avg_sq]
    n = param.numel()
    for name, tt in zip(("param", "grad", "exp_avg", "exp_avg_sq"), ts):
        if tt.dtype != torch.float32 or not tt.is_contiguous() or tt.numel() != n or tt.device != param.device \
                or not tt.is_cuda:
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor of {n} elements on {param.device}")
    hp = AdamwParams(lr, beta1, beta2, eps, weight_decay)
    _check(lib().q4gsw_adamw_step(param.data_ptr(), grad.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), n,
                                  ctypes.byref(hp), int(step), _stream()), "q4gsw_adamw_step")


def embedding(w: PackedWeight, ids: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out [*ids.shape, K] fp32: entry ids[i] gives row ids[i] of dequant(W) (zeros outside [0, N))."""
    ids = _dev(ids, "ids")
    if ids.dtype != torch.int64:
        raise ValueError("ids must be int64")
    T = ids.numel()
    o = out if out is not None else torch.empty(*ids.shape, w.K, dtype=torch.float32, device=ids.device)
    if o.dtype != torch.float32 or not o.is_contiguous() or o.numel() != T * w.K or o.device != ids.device:
        raise ValueError("out must be a contiguous fp32 tensor of ids.numel() * K elements on ids' device")
    _check(lib().q4gsw_embedding(w.ref(), ids.data_ptr(), T, o.data_ptr(), _stream()), "q4gsw_embedding")
    return o


def qkv_workspace_bytes(wq: PackedWeight, wk: PackedWeight, wv: PackedWeight, M: int, dtype: torch.dtype) -> int:
    out = ctypes.c_uint64()
    _check(lib().q4gsw_qkv_workspace_bytes_ex(wq.ref(), wk.ref(), wv.ref(), M, _TORCH_DTYPE[dtype], _opts(),
                                              ctypes.byref(out)), "q4gsw_qkv_workspace_bytes")
    return out.value


def qkv_fused(wq: PackedWeight, wk: PackedWeight, wv: PackedWeight, x: torch.Tensor,
              outs: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
              workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(q, k, v) fp32 = x . dequant(Wq)^T, x . dequant(Wk)^T, x . dequant(Wv)^T in one call."""
    x = _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != wq.K:
        raise ValueError("x must be [M, K]")
    M = x.shape[0]
    if outs is None:
        outs = (None, None, None)
    if len(outs) != 3:
        raise ValueError("outs must be three tensors (q, k, v)")
    q, k, v = (_out(o, (M, w.N), x.device, name) for o, w, name in zip(outs, (wq, wk, wv), ("q", "k", "v")))
    need = qkv_workspace_bytes(wq, wk, wv, M, x.dtype)
    ws, wp, wb = _ws_args(need, workspace, x.device)
    _check(lib().q4gsw_qkv_fused_ex(wq.ref(), wk.ref(), wv.ref(), x.data_ptr(), _TORCH_DTYPE[x.dtype], M,
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), wp, wb, _opts(), _stream()),
           "q4gsw_qkv_fused")
    return q, k, v


def route(op: int, w: PackedWeight, M: int, dtype: torch.dtype) -> str:
    """The route a call with these arguments takes (under this thread's forced route, if any).  For
    OP_QKV the route depends on Wq only."""
    o = _opts()
    if o is None:
        return route_name(lib().q4gsw_route(op, w.ref(), M, _TORCH_DTYPE[dtype]))
    info = PlanInfo()
    extra = w.ref() if op == OP_QKV else None
    _check(lib().q4gsw_plan(op, w.ref(), extra, extra, M, _TORCH_DTYPE[dtype], o, ctypes.byref(info)), "q4gsw_plan")
    return route_name(info.route)


def plan(op: int, w: PackedWeight, M: int, dtype: torch.dtype, wk: PackedWeight = None,
         wv: PackedWeight = None) -> dict:
    """How a call runs: route name, MFMA block rows and contraction splits.  For OP_QKV pass wk
    and wv."""
    info = PlanInfo()
    refs = [x.ref() if x is not None else None for x in (wk, wv)]
    _check(lib().q4gsw_plan(op, w.ref(), refs[0], refs[1], M, _TORCH_DTYPE[dtype], _opts(), ctypes.byref(info)),
           "q4gsw_plan")
    return {"route": route_name(info.route), "tile_rows": info.tile_rows, "splits": info.splits}


@contextlib.contextmanager
def _with_options(**fields):
    """Set fields of this thread's per-call options for the calls inside the block."""
    old = getattr(_local, "opts", None)
    new = Options()
    if old is not None:
        ctypes.memmove(ctypes.byref(new), ctypes.byref(old), ctypes.sizeof(Options))
    for k, v in fields.items():
        setattr(new, k, v)
    _local.opts = new
    try:
        yield
    finally:
        _local.opts = old


@contextlib.contextmanager
def forced_plan(tile_rows: int = 0, splits: int = 0):
    """Pin the forward / QKV MFMA block rows (64 or 128) and the contraction splits (the split
    count also governs the 32x32 input-gradient routes) of the calls made by this thread inside the
    block; 0 leaves a choice per shape.  Out-of-range values raise ValueError."""
    if tile_rows not in (0, 64, 128) or not 0 <= splits <= 64:
        raise ValueError("tile_rows must be 0, 64 or 128 and splits 0..64")
    with _with_options(tile_rows=tile_rows, splits=splits):
        yield


@contextlib.contextmanager
def forced_route(name: str):
    """Send the calls made by this thread inside the block onto one route family (tests and
    benchmarks); a call the family cannot serve raises Q4gswError with E_ROUTE."""
    with _with_options(route=ROUTES[name]):
        yield


def build_info() -> str:
    return lib().q4gsw_build_info().decode()
