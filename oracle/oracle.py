"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding.

Inputs are CPU tensors from ``synthetic_inputs`` (activations in f32/f16/bf16,
codes uint8 [N, K], scales f16/f32 [K/group_size, N]).  Their raw bytes are handed
to the C code, which decodes every element to double itself.  Results are numpy
float64 arrays: the output and the normaliser R = sum |activation|*|dequant(W)|.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import build as _build

_DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}


class OracleError(RuntimeError):
    pass


def _ptr(t: torch.Tensor) -> int:
    assert t.device.type == "cpu" and t.is_contiguous()
    return t.data_ptr()


class Oracle:
    """One loaded copy of the oracle library (the default one, or a test build of it)."""

    def __init__(self, path: str):
        handle = ctypes.CDLL(path)
        i64, vp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        for name in ("oracle_linear_fwd", "oracle_linear_bwd_input"):
            fn = getattr(handle, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [vp, ip, i64, vp, vp, ip, i64, i64, i64, vp, vp, ip]
        handle.oracle_dequant.restype = ctypes.c_double
        handle.oracle_dequant.argtypes = [vp, vp, ip, i64, i64, i64, i64, i64]
        handle.oracle_f16_to_f64.restype = ctypes.c_double
        handle.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        handle.oracle_bf16_to_f64.restype = ctypes.c_double
        handle.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        handle.oracle_f32_to_f64.restype = ctypes.c_double
        handle.oracle_f32_to_f64.argtypes = [ctypes.c_uint32]
        handle.oracle_threads.restype = ctypes.c_int
        handle.oracle_threads.argtypes = [ctypes.c_int]
        handle.oracle_embedding.restype = ctypes.c_int
        handle.oracle_embedding.argtypes = [vp, i64, vp, vp, ip, i64, i64, i64, vp]
        handle.oracle_dq8ca_quantize.restype = ctypes.c_int
        handle.oracle_dq8ca_quantize.argtypes = [vp, ip, i64, i64, vp, vp, vp, ip]
        handle.oracle_linear_dq8ca.restype = ctypes.c_int
        handle.oracle_linear_dq8ca.argtypes = [vp, vp, vp, i64, vp, vp, ip, i64, i64, i64, vp, vp, ip]
        dbl = ctypes.c_double
        handle.oracle_lora_fwd.restype = ctypes.c_int
        handle.oracle_lora_fwd.argtypes = [vp, ip, i64, vp, vp, ip, i64, i64, i64, vp, vp, i64, dbl, vp, vp, vp, ip]
        handle.oracle_lora_bwd.restype = ctypes.c_int
        handle.oracle_lora_bwd.argtypes = [vp, vp, ip, i64, vp, vp, ip, i64, i64, i64, vp, vp, i64, dbl,
                                           vp, vp, vp, vp, vp, vp, ip]
        handle.oracle_adamw.restype = ctypes.c_int
        handle.oracle_adamw.argtypes = [vp, vp, vp, vp, i64, dbl, dbl, dbl, dbl, dbl, i64, vp, vp, vp]
        self.lib = handle
        self.path = path

    def _run(self, fn_name: str, act: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
             group_size: int, out_rows: int, out_cols: int, threads: int) -> Tuple[np.ndarray, np.ndarray]:
        act = act.contiguous()
        codes = codes.contiguous()
        scales = scales.contiguous()
        N, K = codes.shape
        out = np.zeros((out_rows, out_cols), dtype=np.float64)
        norm = np.zeros((out_rows, out_cols), dtype=np.float64)
        status = getattr(self.lib, fn_name)(
            _ptr(act), _DTYPE_CODE[act.dtype], act.shape[0], _ptr(codes), _ptr(scales),
            _DTYPE_CODE[scales.dtype], N, K, group_size,
            out.ctypes.data, norm.ctypes.data, threads)
        if status != 0:
            raise OracleError(f"{fn_name} returned {status}")
        return out, norm

    def linear_fwd(self, x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, group_size: int,
                   threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """y = x . dequant(W)^T and its normaliser, both [M, N] float64."""
        N, K = codes.shape
        if x.dim() != 2 or x.shape[1] != K:
            raise OracleError("x must be [M, K]")
        return self._run("oracle_linear_fwd", x, codes, scales, group_size, x.shape[0], N, threads)

    def linear_bwd_input(self, d_out: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                         group_size: int, threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """d_x = d_out . dequant(W) (contracting over N) and its normaliser, both [M, K] float64."""
        N, K = codes.shape
        if d_out.dim() != 2 or d_out.shape[1] != N:
            raise OracleError("d_out must be [M, N]")
        return self._run("oracle_linear_bwd_input", d_out, codes, scales, group_size,
                         d_out.shape[0], K, threads)

    def qkv(self, x: torch.Tensor, weights: Sequence, threads: int = 0) -> List[Tuple[np.ndarray, np.ndarray]]:
        """Three forwards of one activation: [(q, R_q), (k, R_k), (v, R_v)].

        ``weights`` holds three objects with ``codes``, ``scales`` and ``group_size``
        sharing K and group_size (the fused projection triple)."""
        if len(weights) != 3:
            raise OracleError("qkv takes three weights")
        K = weights[0].codes.shape[1]
        gs = weights[0].group_size
        for w in weights:
            if w.codes.shape[1] != K or w.group_size != gs:
                raise OracleError("q, k and v weights must share K and group_size")
        return [self.linear_fwd(x, w.codes, w.scales, w.group_size, threads) for w in weights]

    def embedding(self, ids: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                  group_size: int) -> np.ndarray:
        """Rows ids[t] of dequant(W), [T, K] float64 (rows of zeros for ids outside [0, N))."""
        ids = ids.to(torch.int64).contiguous()
        codes = codes.contiguous()
        scales = scales.contiguous()
        N, K = codes.shape
        out = np.zeros((ids.numel(), K), dtype=np.float64)
        status = self.lib.oracle_embedding(_ptr(ids), ids.numel(), _ptr(codes), _ptr(scales),
                                           _DTYPE_CODE[scales.dtype], N, K, group_size, out.ctypes.data)
        if status != 0:
            raise OracleError(f"oracle_embedding returned {status}")
        return out

    def dq8ca_quantize(self, x: torch.Tensor, threads: int = 0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Per-row int8 quantisation of x [M, K]: (q int8 [M, K], scale float32 [M], zp int32 [M])."""
        x = x.contiguous()
        if x.dim() != 2:
            raise OracleError("x must be [M, K]")
        M, K = x.shape
        q = np.zeros((M, K), dtype=np.int8)
        scale = np.zeros(M, dtype=np.float32)
        zp = np.zeros(M, dtype=np.int32)
        status = self.lib.oracle_dq8ca_quantize(_ptr(x), _DTYPE_CODE[x.dtype], M, K, q.ctypes.data,
                                                scale.ctypes.data, zp.ctypes.data, threads)
        if status != 0:
            raise OracleError(f"oracle_dq8ca_quantize returned {status}")
        return q, scale, zp

    def linear_dq8ca(self, x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, group_size: int,
                     threads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
        """y = (scale * (q - zp)) . dequant(W)^T for the per-row int8 quantisation of x, and its
        normaliser, both [M, N] float64."""
        codes = codes.contiguous()
        scales = scales.contiguous()
        N, K = codes.shape
        if x.dim() != 2 or x.shape[1] != K:
            raise OracleError("x must be [M, K]")
        q, scale, zp = self.dq8ca_quantize(x, threads)
        M = x.shape[0]
        out = np.zeros((M, N), dtype=np.float64)
        norm = np.zeros((M, N), dtype=np.float64)
        status = self.lib.oracle_linear_dq8ca(q.ctypes.data, scale.ctypes.data, zp.ctypes.data, M, _ptr(codes),
                                              _ptr(scales), _DTYPE_CODE[scales.dtype], N, K, group_size,
                                              out.ctypes.data, norm.ctypes.data, threads)
        if status != 0:
            raise OracleError(f"oracle_linear_dq8ca returned {status}")
        return out, norm

    def lora_fwd(self, x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, group_size: int,
                 A: torch.Tensor, B: torch.Tensor, alpha: float, threads: int = 0):
        """The adapter forward: (y [M,N], t = x A^T [M,r], R_y [M,N]) as float64 arrays.
        A is fp32 [r,K], B fp32 [N,r].  codes (and scales) None: the frozen-weight term is left
        out and y, R_y hold the adapter term alone."""
        A = A.to(torch.float32).contiguous()
        B = B.to(torch.float32).contiguous()
        x = x.contiguous()
        if codes is None:
            codes_p, scales_p, sdt = None, None, 0
            N, K = B.shape[0], A.shape[1]
        else:
            codes, scales = codes.contiguous(), scales.contiguous()
            codes_p, scales_p, sdt = _ptr(codes), _ptr(scales), _DTYPE_CODE[scales.dtype]
            N, K = codes.shape
        r = A.shape[0]
        if x.dim() != 2 or x.shape[1] != K or A.shape != (r, K) or B.shape != (N, r):
            raise OracleError("x [M,K], A [r,K], B [N,r]")
        M = x.shape[0]
        y = np.zeros((M, N)); t = np.zeros((M, r)); norm = np.zeros((M, N))
        st = self.lib.oracle_lora_fwd(_ptr(x), _DTYPE_CODE[x.dtype], M, codes_p, scales_p,
                                      sdt, N, K, group_size, _ptr(A), _ptr(B), r,
                                      float(alpha), y.ctypes.data, t.ctypes.data, norm.ctypes.data, threads)
        if st != 0:
            raise OracleError(f"oracle_lora_fwd returned {st}")
        return y, t, norm

    def lora_bwd(self, x: torch.Tensor, d_out: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                 group_size: int, A: torch.Tensor, B: torch.Tensor, alpha: float, threads: int = 0):
        """The adapter backward: dict of float64 arrays dx [M,K], dA [r,K], dB [N,r] and their
        normalisers r_dx, r_dA, r_dB.  x and d_out share one dtype.  codes (and scales) None: the
        frozen-weight term of dx is left out (dA and dB do not depend on it)."""
        x, d_out = x.contiguous(), d_out.contiguous()
        A = A.to(torch.float32).contiguous()
        B = B.to(torch.float32).contiguous()
        if codes is None:
            codes_p, scales_p, sdt = None, None, 0
            N, K = B.shape[0], A.shape[1]
        else:
            codes, scales = codes.contiguous(), scales.contiguous()
            codes_p, scales_p, sdt = _ptr(codes), _ptr(scales), _DTYPE_CODE[scales.dtype]
            N, K = codes.shape
        r = A.shape[0]
        M = x.shape[0]
        if x.dtype != d_out.dtype or x.shape != (M, K) or d_out.shape != (M, N) or A.shape != (r, K) \
                or B.shape != (N, r):
            raise OracleError("x [M,K] and d_out [M,N] of one dtype, A [r,K], B [N,r]")
        out = {k: np.zeros(sh) for k, sh in (("dx", (M, K)), ("dA", (r, K)), ("dB", (N, r)),
                                             ("r_dx", (M, K)), ("r_dA", (r, K)), ("r_dB", (N, r)))}
        st = self.lib.oracle_lora_bwd(_ptr(x), _ptr(d_out), _DTYPE_CODE[x.dtype], M, codes_p, scales_p,
                                      sdt, N, K, group_size, _ptr(A), _ptr(B), r,
                                      float(alpha), out["dx"].ctypes.data, out["dA"].ctypes.data,
                                      out["dB"].ctypes.data, out["r_dx"].ctypes.data, out["r_dA"].ctypes.data,
                                      out["r_dB"].ctypes.data, threads)
        if st != 0:
            raise OracleError(f"oracle_lora_bwd returned {st}")
        return out

    def adamw(self, p: torch.Tensor, g: torch.Tensor, m: torch.Tensor, v: torch.Tensor, lr: float,
              beta1: float, beta2: float, eps: float, weight_decay: float, step: int):
        """One AdamW step on fp32 tensors of one size: (p, m, v) after it, float64 arrays."""
        ts = [t.to(torch.float32).contiguous().reshape(-1) for t in (p, g, m, v)]
        n = ts[0].numel()
        if any(t.numel() != n for t in ts):
            raise OracleError("p, g, m and v must have one size")
        po, mo, vo = np.zeros(n), np.zeros(n), np.zeros(n)
        st = self.lib.oracle_adamw(*[_ptr(t) for t in ts], n, float(lr), float(beta1), float(beta2), float(eps),
                                   float(weight_decay), int(step), po.ctypes.data, mo.ctypes.data, vo.ctypes.data)
        if st != 0:
            raise OracleError(f"oracle_adamw returned {st}")
        return po, mo, vo

    def dequant(self, codes: torch.Tensor, scales: torch.Tensor, group_size: int, n: int, k: int) -> float:
        """One element of dequant(W), as the oracle computes it."""
        codes = codes.contiguous()
        scales = scales.contiguous()
        N, K = codes.shape
        return self.lib.oracle_dequant(_ptr(codes), _ptr(scales), _DTYPE_CODE[scales.dtype], N, K,
                                       group_size, n, k)

    def f16_to_f64(self, bits: int) -> float:
        return self.lib.oracle_f16_to_f64(bits)

    def bf16_to_f64(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_f64(bits)

    def f32_to_f64(self, bits: int) -> float:
        return self.lib.oracle_f32_to_f64(bits)

    def threads_used(self, threads: int = 0) -> int:
        """OpenMP threads a call with ``threads`` would use (0 = the runtime default)."""
        return self.lib.oracle_threads(threads)


_default: Optional[Oracle] = None


def default() -> Oracle:
    """The oracle built from oracle.c (built on first use when missing or stale)."""
    global _default
    if _default is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        _default = Oracle(path)
    return _default


def linear_fwd(x, codes, scales, group_size, threads=0):
    return default().linear_fwd(x, codes, scales, group_size, threads)


def linear_bwd_input(d_out, codes, scales, group_size, threads=0):
    return default().linear_bwd_input(d_out, codes, scales, group_size, threads)


def qkv(x, weights, threads=0):
    return default().qkv(x, weights, threads)


def embedding(ids, codes, scales, group_size):
    return default().embedding(ids, codes, scales, group_size)


def dq8ca_quantize(x, threads=0):
    return default().dq8ca_quantize(x, threads)


def linear_dq8ca(x, codes, scales, group_size, threads=0):
    return default().linear_dq8ca(x, codes, scales, group_size, threads)


def lora_fwd(x, codes, scales, group_size, A, B, alpha, threads=0):
    return default().lora_fwd(x, codes, scales, group_size, A, B, alpha, threads)


def lora_bwd(x, d_out, codes, scales, group_size, A, B, alpha, threads=0):
    return default().lora_bwd(x, d_out, codes, scales, group_size, A, B, alpha, threads)


def adamw(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    return default().adamw(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step)
