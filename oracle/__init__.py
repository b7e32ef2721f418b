"""CPU oracle of the BitLinear forward pass (numpy front end over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  It shares
no code with the GPU library and never imports it.

Each function is a thin ctypes wrapper around one literal definition in
``oracle.c``; see that file for the definitions and the pages they follow.
Arrays are numpy arrays in the layouts of the C functions:

* ``W``  float32 [N][K] weights (out x in), ``packed`` uint8 [N][K/4];
* ``x``  bf16 activations passed as their uint16 bit patterns [M][K];
* codes int8 [M][K], ``d_x`` float32 [M], ``qsum`` int32 [M];
* ``acc`` int32 [M][N], ``y`` float64 [M][N].
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build_oracle()
        _LIB = load(_build.LIB)
    return _LIB


def load(path: str):
    """Load an oracle shared library from ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    p, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    lib.oracle_version.restype = i32
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_set_num_threads.restype = None
    lib.oracle_unpack_weights.argtypes = [p, i64, i64, p]
    lib.oracle_unpack_weights.restype = i64
    lib.oracle_fwht_f32.argtypes = [p, i64]
    lib.oracle_fwht_f32.restype = None
    lib.oracle_pack_weights.argtypes = [p, i64, i64, i32, p, p, p]
    lib.oracle_pack_weights.restype = i32
    for name in ("oracle_quant_act", "oracle_hadamard_quant_act"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, f32, i64, i64, p, p, p]
        fn.restype = i32
    lib.oracle_int_gemm.argtypes = [p, p, i64, i64, i64, p]
    lib.oracle_int_gemm.restype = i32
    lib.oracle_int_gemm_sampled.argtypes = [p, p, i64, i64, i64, p, p, i64, p]
    lib.oracle_int_gemm_sampled.restype = i32
    lib.oracle_dequant.argtypes = [p, p, f32, i64, i64, p]
    lib.oracle_dequant.restype = None
    lib.oracle_transpose_packed.argtypes = [p, i64, i64, p]
    lib.oracle_transpose_packed.restype = i32
    lib.oracle_linear_backward_input.argtypes = [p, p, f32, i64, i64, i64, p]
    lib.oracle_linear_backward_input.restype = i32
    lib.oracle_linear_backward_weight.argtypes = [p, p, p, i64, i64, i64, p]
    lib.oracle_linear_backward_weight.restype = i32
    lib.oracle_rmsnorm_backward.argtypes = [p, p, f32, p, i64, i64, p, p]
    lib.oracle_rmsnorm_backward.restype = i32
    lib.oracle_pack_base3.argtypes = [p, i64, i64, i64, p]
    lib.oracle_pack_base3.restype = i32
    lib.oracle_unpack_base3.argtypes = [p, i64, i64, i64, p]
    lib.oracle_unpack_base3.restype = i64
    lib.oracle_pack_nibbles.argtypes = [p, i64, i64, p]
    lib.oracle_pack_nibbles.restype = i32
    lib.oracle_unpack_nibbles.argtypes = [p, i64, i64, p]
    lib.oracle_unpack_nibbles.restype = i32
    lib.oracle_warmup_lambda.argtypes = [i64, i64]
    lib.oracle_warmup_lambda.restype = ctypes.c_double
    lib.oracle_linear_forward_blend.argtypes = [p, p, f32, i64, i64, p, i64, ctypes.c_double, p]
    lib.oracle_linear_forward_blend.restype = i32
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """The oracle's functions bound to one loaded library (default: ``liboracle.so``)."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else _lib()

    def num_threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Thread count of the oracle's later calls (for one-core timings)."""
        self.lib.oracle_set_num_threads(int(n))

    def unpack_weights(self, packed: np.ndarray, K: int) -> np.ndarray:
        packed = _c(packed, np.uint8)
        N = packed.shape[0]
        q = np.empty((N, K), np.int8)
        bad = self.lib.oracle_unpack_weights(_ptr(packed), N, K, _ptr(q))
        if bad:
            raise ValueError(f"{bad} invalid 2-bit fields (value 3) in packed weights")
        return q

    def fwht_f32(self, v: np.ndarray) -> np.ndarray:
        """Unnormalised Walsh-Hadamard transform of each row of ``v`` (float32)."""
        out = np.array(v, dtype=np.float32, copy=True, order="C")
        rows = out.reshape(-1, out.shape[-1])
        for r in range(rows.shape[0]):
            self.lib.oracle_fwht_f32(_ptr(rows[r]), rows.shape[1])
        return out

    def pack_weights(self, W: np.ndarray, hadamard: bool = False):
        """Return (packed uint8 [N][K/4], d_w, s_w, q int8 [N][K])."""
        W = _c(W, np.float32)
        N, K = W.shape
        packed = np.empty((N, K // 4), np.uint8)
        scale = np.empty(2, np.float32)
        q = np.empty((N, K), np.int8)
        rc = self.lib.oracle_pack_weights(_ptr(W), N, K, int(bool(hadamard)), _ptr(packed),
                                          _ptr(scale), _ptr(q))
        if rc != 0:
            raise ValueError(f"oracle_pack_weights rejected N={N} K={K} hadamard={hadamard}")
        return packed, np.float32(scale[0]), np.float32(scale[1]), q

    def _quant(self, fn, x_bits, gain, eps):
        x_bits = _c(x_bits, np.uint16)
        M, K = x_bits.shape
        g = None if gain is None else _c(gain, np.float32)
        q = np.empty((M, K), np.int8)
        d_x = np.empty(M, np.float32)
        qsum = np.empty(M, np.int32)
        rc = fn(_ptr(x_bits), _ptr(g), ctypes.c_float(eps), M, K, _ptr(q), _ptr(d_x), _ptr(qsum))
        if rc != 0:
            raise ValueError(f"oracle quantisation rejected M={M} K={K}")
        return q, d_x, qsum

    def quant_act(self, x_bits: np.ndarray, gain=None, eps: float = 1e-5):
        """RMSNorm + absmax int8 codes: returns (q int8 [M][K], d_x f32 [M], qsum i32 [M])."""
        return self._quant(self.lib.oracle_quant_act, x_bits, gain, eps)

    def hadamard_quant_act(self, x_bits: np.ndarray, gain=None, eps: float = 1e-5):
        """RMSNorm + Hadamard + absmax int4 codes: returns (q, d_x, qsum)."""
        return self._quant(self.lib.oracle_hadamard_quant_act, x_bits, gain, eps)

    def int_gemm(self, xq: np.ndarray, packed: np.ndarray, K: int) -> np.ndarray:
        xq = _c(xq, np.int8)
        packed = _c(packed, np.uint8)
        M, N = xq.shape[0], packed.shape[0]
        acc = np.empty((M, N), np.int32)
        rc = self.lib.oracle_int_gemm(_ptr(xq), _ptr(packed), M, N, K, _ptr(acc))
        if rc != 0:
            raise ValueError("oracle_int_gemm rejected its arguments")
        return acc

    def int_gemm_sampled(self, xq, packed, K: int, rows, cols) -> np.ndarray:
        xq = _c(xq, np.int8)
        packed = _c(packed, np.uint8)
        rows = _c(rows, np.int64)
        cols = _c(cols, np.int64)
        out = np.empty(rows.shape[0], np.int32)
        rc = self.lib.oracle_int_gemm_sampled(_ptr(xq), _ptr(packed), xq.shape[0], packed.shape[0],
                                              K, _ptr(rows), _ptr(cols), rows.shape[0], _ptr(out))
        if rc != 0:
            raise ValueError("oracle_int_gemm_sampled rejected its arguments")
        return out

    def dequant(self, acc: np.ndarray, d_x: np.ndarray, d_w: float) -> np.ndarray:
        acc = _c(acc, np.int32)
        d_x = _c(d_x, np.float32)
        M, N = acc.shape
        y = np.empty((M, N), np.float64)
        self.lib.oracle_dequant(_ptr(acc), _ptr(d_x), ctypes.c_float(d_w), M, N, _ptr(y))
        return y

    def linear_forward(self, xq, d_x, packed, d_w, K: int):
        """Full contraction + dequantisation: returns (acc int32 [M][N], y float64 [M][N])."""
        acc = self.int_gemm(xq, packed, K)
        return acc, self.dequant(acc, d_x, d_w)

    # --- backward under the straight-through estimator -------------------

    def transpose_packed(self, packed: np.ndarray, K: int) -> np.ndarray:
        """packed uint8 [N][K/4] -> packed_t uint8 [K][N/4] (same layout along rows)."""
        packed = _c(packed, np.uint8)
        N = packed.shape[0]
        out = np.empty((K, N // 4), np.uint8)
        if self.lib.oracle_transpose_packed(_ptr(packed), N, K, _ptr(out)) != 0:
            raise ValueError(f"oracle_transpose_packed rejected N={N} K={K}")
        return out

    def linear_backward_input(self, grad_y_bits, packed, d_w, K: int) -> np.ndarray:
        """grad_n float64 [M][K] = d_w * grad_y (bf16 bits [M][N]) @ q_w."""
        g = _c(grad_y_bits, np.uint16)
        packed = _c(packed, np.uint8)
        M, N = g.shape
        out = np.empty((M, K), np.float64)
        rc = self.lib.oracle_linear_backward_input(_ptr(g), _ptr(packed), ctypes.c_float(d_w),
                                                   M, N, K, _ptr(out))
        if rc != 0:
            raise ValueError("oracle_linear_backward_input rejected its arguments")
        return out

    def linear_backward_weight(self, grad_y_bits, xq, d_x) -> np.ndarray:
        """grad_w float64 [N][K] = sum_m grad_y[m][n] d_x[m] q_x[m][k]."""
        g = _c(grad_y_bits, np.uint16)
        xq = _c(xq, np.int8)
        d_x = _c(d_x, np.float32)
        M, N = g.shape
        K = xq.shape[1]
        out = np.empty((N, K), np.float64)
        rc = self.lib.oracle_linear_backward_weight(_ptr(g), _ptr(xq), _ptr(d_x), M, N, K, _ptr(out))
        if rc != 0:
            raise ValueError("oracle_linear_backward_weight rejected its arguments")
        return out

    def rmsnorm_backward(self, x_bits, grad_n, gain=None, eps: float = 1e-5, with_gain_grad=False):
        """(grad_x float64 [M][K], grad_gain float64 [K] or None) of n = x * gain * r."""
        x_bits = _c(x_bits, np.uint16)
        gn = _c(grad_n, np.float32)
        M, K = x_bits.shape
        g = None if gain is None else _c(gain, np.float32)
        gx = np.empty((M, K), np.float64)
        gg = np.empty(K, np.float64) if with_gain_grad else None
        rc = self.lib.oracle_rmsnorm_backward(_ptr(x_bits), _ptr(g), ctypes.c_float(eps), _ptr(gn),
                                              M, K, _ptr(gx), _ptr(gg))
        if rc != 0:
            raise ValueError("oracle_rmsnorm_backward rejected its arguments")
        return gx, gg


    def pack_base3(self, q: np.ndarray, row_bytes: int) -> np.ndarray:
        """Ternary codes int8 [N][K] -> base-3 packed uint8 [N][row_bytes], five
        weights per byte (byte j = sum_i (q[5j+i] + 1) 3^i)."""
        q = _c(q, np.int8)
        N, K = q.shape
        out = np.empty((N, row_bytes), np.uint8)
        if self.lib.oracle_pack_base3(_ptr(q), N, K, row_bytes, _ptr(out)) != 0:
            raise ValueError(f"oracle_pack_base3 rejected K={K} row_bytes={row_bytes} or a code")
        return out

    def unpack_base3(self, packed3: np.ndarray, K: int):
        """(codes int8 [N][K], count of bytes above 242) of a base-3 packing."""
        packed3 = _c(packed3, np.uint8)
        N, row_bytes = packed3.shape
        q = np.empty((N, K), np.int8)
        bad = self.lib.oracle_unpack_base3(_ptr(packed3), N, K, row_bytes, _ptr(q))
        return q, int(bad)

    def pack_nibbles(self, q: np.ndarray) -> np.ndarray:
        """int4 codes int8 [M][K] -> uint8 [M][K/2]: in each group g of 16 codes,
        byte 8g + j holds code 16g + j (low nibble) and 16g + 8 + j (high
        nibble), two's complement."""
        q = _c(q, np.int8)
        M, K = q.shape
        out = np.empty((M, K // 2), np.uint8)
        if self.lib.oracle_pack_nibbles(_ptr(q), M, K, _ptr(out)) != 0:
            raise ValueError(f"oracle_pack_nibbles rejected K={K} (a multiple of 16) or a code outside [-8, 7]")
        return out

    def unpack_nibbles(self, packed: np.ndarray) -> np.ndarray:
        """uint8 [M][K/2] -> int4 codes int8 [M][K]."""
        packed = _c(packed, np.uint8)
        M, half = packed.shape
        q = np.empty((M, 2 * half), np.int8)
        if self.lib.oracle_unpack_nibbles(_ptr(packed), M, 2 * half, _ptr(q)) != 0:
            raise ValueError("oracle_unpack_nibbles rejected its arguments")
        return q

    def warmup_lambda(self, step: int, total: int) -> float:
        """min(step / total, 1), 0 for step <= 0, 1 for total <= 0."""
        return float(self.lib.oracle_warmup_lambda(int(step), int(total)))

    def linear_forward_blend(self, x_bits, W, lam: float, gain=None, eps: float = 1e-5) -> np.ndarray:
        """float64 y [M][N] of the layer at warm-up blend factor lam (oracle_linear_forward_blend)."""
        x_bits = _c(x_bits, np.uint16)
        W = _c(W, np.float32)
        M, K = x_bits.shape
        N = W.shape[0]
        g = None if gain is None else _c(gain, np.float32)
        y = np.empty((M, N), np.float64)
        rc = self.lib.oracle_linear_forward_blend(_ptr(x_bits), _ptr(g), ctypes.c_float(eps), M, K, _ptr(W), N,
                                                  ctypes.c_double(lam), _ptr(y))
        if rc != 0:
            raise ValueError(f"oracle_linear_forward_blend rejected M={M} N={N} K={K}")
        return y


_DEFAULT = None


def default() -> Oracle:
    """The oracle bound to ``oracle/liboracle.so`` (built on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT

