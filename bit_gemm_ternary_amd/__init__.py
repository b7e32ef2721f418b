"""bit_gemm_ternary_amd: BitNet b1.58 BitLinear forward on MI355X (gfx950).

Thin Python binding over the C ABI of ``libbitnet_hip.so`` (declared in
``include/bitnet.h``).  The functions below only check and marshal arguments
(torch device tensors in, torch device tensors out, the current torch stream
passed through); every step of the computation runs in the library's HIP
kernels.  There is no CPU fallback: if the library is missing the calls raise.

    packed, w_scale = pack_weights(W)                 # once per layer
    xq, x_scale, x_qsum = quant_act(x)                # bf16 [M][K] -> int8 codes
    y = linear_forward(xq, x_scale, x_qsum, packed, w_scale)
    y = bitlinear(x, packed, w_scale)                 # both steps
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "BitnetError", "lib", "library_path", "pack_weights", "pack_weights_workspace_bytes",
    "base3_row_bytes", "pack_base3", "linear_forward_base3",
    "quant_act", "hadamard_quant_act", "linear_forward", "bitlinear", "bitlinear_forward",
    "BitLinear",
    "STATUS", "set_kernel_events",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbitnet_hip.so")
_LIB = None

STATUS = {
    0: "BITNET_OK", 1: "BITNET_ERR_NULL", 2: "BITNET_ERR_SHAPE", 3: "BITNET_ERR_UNSUPPORTED",
    4: "BITNET_ERR_ALIGN", 5: "BITNET_ERR_WORKSPACE", 6: "BITNET_ERR_HIP", 7: "BITNET_ERR_VALUE",
}


class BitnetError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load ``libbitnet_hip.so`` (built by ``bit_gemm_ternary_amd.build``) and declare its ABI."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m bit_gemm_ternary_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(_LIB_PATH)
    p, i64, f32, i32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                            ctypes.c_size_t)
    L.bitnet_pack_weights_workspace_bytes.argtypes = [i64, i64, i32]
    L.bitnet_pack_weights_workspace_bytes.restype = sz
    L.bitnet_pack_weights.argtypes = [p, i64, i64, i32, p, p, p, sz, p]
    L.bitnet_pack_weights.restype = i32
    for name in ("bitnet_quant_act", "bitnet_hadamard_quant_act"):
        fn = getattr(L, name)
        fn.argtypes = [p, p, f32, i64, i64, p, p, p, p]
        fn.restype = i32
    L.bitnet_linear_forward.argtypes = [p, p, p, p, p, i64, i64, i64, p, p, p]
    L.bitnet_linear_forward.restype = i32
    L.bitnet_hadamard_quant_act_f6.argtypes = [p, p, f32, i64, i64, p, p, p, p]
    L.bitnet_hadamard_quant_act_f6.restype = i32
    L.bitnet_linear_forward_f6.argtypes = [p, p, p, p, p, i64, i64, i64, p, p, p]
    L.bitnet_linear_forward_f6.restype = i32
    L.bitnet_bitlinear_forward.argtypes = [p, p, f32, p, p, i64, i64, i64, p, p, p, p, p, p]
    L.bitnet_bitlinear_forward.restype = i32
    L.bitnet_bitlinear_forward_grouped.argtypes = [p, p, f32, p, p, p, i32, i64, i64, p, p, p, p,
                                                   p, p]
    L.bitnet_bitlinear_forward_grouped.restype = i32
    L.bitnet_transpose_packed.argtypes = [p, i64, i64, p, p]
    L.bitnet_transpose_packed.restype = i32
    L.bitnet_linear_backward_input.argtypes = [p, p, p, i64, i64, i64, p, p]
    L.bitnet_linear_backward_input.restype = i32
    L.bitnet_linear_backward_weight_workspace_bytes.argtypes = [i64, i64, i64]
    L.bitnet_linear_backward_weight_workspace_bytes.restype = sz
    L.bitnet_linear_backward_weight.argtypes = [p, p, p, i64, i64, i64, p, p, sz, p]
    L.bitnet_linear_backward_weight.restype = i32
    L.bitnet_rmsnorm_backward_workspace_bytes.argtypes = [i64, i64]
    L.bitnet_rmsnorm_backward_workspace_bytes.restype = sz
    L.bitnet_rmsnorm_backward.argtypes = [p, p, f32, p, i64, i64, p, p, p, sz, p]
    L.bitnet_rmsnorm_backward.restype = i32
    L.bitnet_status_string.argtypes = [i32]
    L.bitnet_status_string.restype = ctypes.c_char_p
    L.bitnet_last_error.argtypes = []
    L.bitnet_last_error.restype = ctypes.c_char_p
    L.bitnet_version.argtypes = []
    L.bitnet_version.restype = i32
    L.bitnet_set_kernel_events.argtypes = [p, p]
    L.bitnet_set_kernel_events.restype = i32
    L.bitnet_base3_row_bytes.argtypes = [i64]
    L.bitnet_base3_row_bytes.restype = sz
    L.bitnet_pack_base3.argtypes = [p, i64, i64, p, p]
    L.bitnet_pack_base3.restype = i32
    L.bitnet_linear_forward_base3.argtypes = [p, p, p, p, p, i64, i64, i64, p, p, p]
    L.bitnet_linear_forward_base3.restype = i32
    _LIB = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise BitnetError(status, lib().bitnet_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def set_kernel_events(start_event, stop_event) -> None:
    """Arm two raw hipEvent_t handles (ints) to time the next kernel a call on this thread launches."""
    lib().bitnet_set_kernel_events(ctypes.c_void_p(start_event), ctypes.c_void_p(stop_event))


def pack_weights_workspace_bytes(N: int, K: int, hadamard: bool = False) -> int:
    return int(lib().bitnet_pack_weights_workspace_bytes(N, K, int(bool(hadamard))))


def pack_weights(W, hadamard: bool = False, out=None, workspace=None):
    """float32 [N][K] device weights -> (packed uint8 [N][K/4], w_scale float32 [2] = (d_w, s_w)).

    ``out`` may hold preallocated (packed, w_scale), ``workspace`` a uint8 device
    buffer of at least pack_weights_workspace_bytes(N, K, hadamard) bytes.
    """
    torch = _torch()
    _require(W, "W", torch.float32, 2)
    N, K = W.shape
    if out is None:
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
        w_scale = torch.empty(2, dtype=torch.float32, device=W.device)
    else:
        packed, w_scale = out
        _require(packed, "packed", torch.uint8, 2)
        _require(w_scale, "w_scale", torch.float32, 1)
        if tuple(packed.shape) != (N, K // 4) or w_scale.shape[0] < 2:
            raise ValueError(f"out must be (uint8 [{N}][{K // 4}], float32 [2])")
    if workspace is None:
        ws_bytes = pack_weights_workspace_bytes(N, K, hadamard)
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=W.device)
    else:
        _require(workspace, "workspace", torch.uint8, 1)
    _check(lib().bitnet_pack_weights(_ptr(W), N, K, int(bool(hadamard)), _ptr(packed),
                                     _ptr(w_scale), _ptr(workspace), workspace.numel(),
                                     _stream(W.device)))
    return packed, w_scale


def pack_weights_grouped(Ws, hadamard: bool = False):
    """Pack several float32 [N_g][K] matrices that share an input (q|k|v, gate|up)
    into one stacked buffer for bitlinear_forward_grouped.

    Returns (packed uint8 [sum N_g][K/4], w_scales float32 [G][2], group_rows list).
    Each group keeps its own absmean scale, exactly as pack_weights gives it.
    """
    torch = _torch()
    if not 1 <= len(Ws) <= 8:
        raise ValueError("between 1 and 8 weight matrices")
    K = Ws[0].shape[1]
    rows = [int(W.shape[0]) for W in Ws]
    dev = Ws[0].device
    packed = torch.empty((sum(rows), K // 4), dtype=torch.uint8, device=dev)
    w_scales = torch.empty((len(Ws), 2), dtype=torch.float32, device=dev)
    r0 = 0
    for g, W in enumerate(Ws):
        _require(W, "W", torch.float32, 2)
        if W.shape[1] != K:
            raise ValueError("all grouped matrices need the same K")
        N = rows[g]
        ws_bytes = pack_weights_workspace_bytes(N, K, hadamard)
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        _check(lib().bitnet_pack_weights(_ptr(W), N, K, int(bool(hadamard)), _ptr(packed[r0:r0 + N]),
                                         _ptr(w_scales[g]), _ptr(workspace), workspace.numel(),
                                         _stream(dev)))
        r0 += N
    return packed, w_scales, rows


def bitlinear_forward_grouped(x, packed, w_scales, group_rows, gain=None, eps: float = 1e-5,
                              out=None, codes=None, acc_out=None):
    """Grouped fused BitLinear forward (bitnet_bitlinear_forward_grouped): x is
    quantised once and contracted with every group of the stacked ``packed``;
    y float32 [M][sum(group_rows)].  Arguments otherwise as bitlinear_forward."""
    torch = _torch()
    _require(x, "x", torch.bfloat16, 2)
    _require(packed, "packed", torch.uint8, 2)
    _require(w_scales, "w_scales", torch.float32, 2)
    M, K = x.shape
    rows = [int(r) for r in group_rows]
    N = sum(rows)
    if packed.shape[0] != N or packed.shape[1] * 4 != K:
        raise ValueError(f"packed is {list(packed.shape)}, expected [{N}][{K // 4}]")
    if tuple(w_scales.shape) != (len(rows), 2):
        raise ValueError(f"w_scales must be [{len(rows)}][2]")
    if gain is not None:
        _require(gain, "gain", torch.float32, 1)
    if codes is None:
        codes = (torch.empty((M, K), dtype=torch.int8, device=x.device),
                 torch.empty(M, dtype=torch.float32, device=x.device),
                 torch.empty(M, dtype=torch.int32, device=x.device))
    xq, x_scale, x_qsum = codes
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _require(out, "out", torch.float32, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}][{N}]")
    if acc_out is not None:
        _require(acc_out, "acc_out", torch.int32, 2)
        if tuple(acc_out.shape) != (M, N):
            raise ValueError(f"acc_out must be [{M}][{N}]")
    rows_c = (ctypes.c_int64 * len(rows))(*rows)
    _check(lib().bitnet_bitlinear_forward_grouped(
        _ptr(x), _ptr(gain), ctypes.c_float(eps), _ptr(packed), _ptr(w_scales),
        ctypes.cast(rows_c, ctypes.c_void_p), len(rows),
        M, K, _ptr(xq), _ptr(x_scale), _ptr(x_qsum), _ptr(out), _ptr(acc_out), _stream(x.device)))
    return (out, acc_out) if acc_out is not None else out


def _quant(name, x, gain, eps, out):
    torch = _torch()
    _require(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if gain is not None:
        _require(gain, "gain", torch.float32, 1)
        if gain.shape[0] != K:
            raise ValueError(f"gain has {gain.shape[0]} entries, x has K={K}")
    if out is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        x_scale = torch.empty(M, dtype=torch.float32, device=x.device)
        x_qsum = torch.empty(M, dtype=torch.int32, device=x.device)
    else:
        xq, x_scale, x_qsum = out
        _require(xq, "xq", torch.int8, 2)
        _require(x_scale, "x_scale", torch.float32, 1)
        _require(x_qsum, "x_qsum", torch.int32, 1)
        if tuple(xq.shape) != (M, K) or x_scale.shape[0] != M or x_qsum.shape[0] != M:
            raise ValueError("out tensors do not match x")
    _check(getattr(lib(), name)(_ptr(x), _ptr(gain), ctypes.c_float(eps), M, K, _ptr(xq),
                                _ptr(x_scale), _ptr(x_qsum), _stream(x.device)))
    return xq, x_scale, x_qsum


def quant_act(x, gain=None, eps: float = 1e-5, out=None):
    """bf16 [M][K] -> (int8 codes [M][K], d_x float32 [M], code sums int32 [M]).

    ``out`` may hold preallocated (codes, d_x, sums) tensors to write into.
    """
    return _quant("bitnet_quant_act", x, gain, eps, out)


def hadamard_quant_act(x, gain=None, eps: float = 1e-5, out=None):
    """H-BitLinear: bf16 [M][K] (K = 2^p) -> (int4 codes as int8 [M][K], d_x, code sums)."""
    return _quant("bitnet_hadamard_quant_act", x, gain, eps, out)


def hadamard_quant_act_f6(x, gain=None, eps: float = 1e-5, out=None):
    """bf16 [M][K] -> (xq6 uint8 [M][K/4*3] 6-bit E3M2 codes, x_scale float32 [M],
    x_qsum int32 [M]) (bitnet_hadamard_quant_act_f6)."""
    torch = _torch()
    _require(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if gain is not None:
        _require(gain, "gain", torch.float32, 1)
    if out is None:
        out = (torch.empty((M, K // 4 * 3), dtype=torch.uint8, device=x.device),
               torch.empty(M, dtype=torch.float32, device=x.device),
               torch.empty(M, dtype=torch.int32, device=x.device))
    xq6, x_scale, x_qsum = out
    _require(xq6, "xq6", torch.uint8, 2)
    if tuple(xq6.shape) != (M, K // 4 * 3):
        raise ValueError(f"xq6 must be [{M}][{K // 4 * 3}]")
    _check(lib().bitnet_hadamard_quant_act_f6(_ptr(x), _ptr(gain), ctypes.c_float(eps), M, K,
                                              _ptr(xq6), _ptr(x_scale), _ptr(x_qsum),
                                              _stream(x.device)))
    return xq6, x_scale, x_qsum


def linear_forward_f6(xq6, x_scale, x_qsum, packed, w_scale, return_acc: bool = False, out=None,
                      acc_out=None):
    """FP4 x FP6 contraction + dequantisation (bitnet_linear_forward_f6); returns y
    float32 [M][N], or (y, acc int32 [M][N]) when return_acc."""
    torch = _torch()
    _require(xq6, "xq6", torch.uint8, 2)
    _require(packed, "packed", torch.uint8, 2)
    _require(w_scale, "w_scale", torch.float32, 1)
    M = xq6.shape[0]
    K = xq6.shape[1] // 3 * 4
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError(f"packed is [{N}][{packed.shape[1]}], expected [{N}][{K // 4}]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=xq6.device)
    if return_acc and acc_out is None:
        acc_out = torch.empty((M, N), dtype=torch.int32, device=xq6.device)
    _check(lib().bitnet_linear_forward_f6(_ptr(xq6), _ptr(x_scale), _ptr(x_qsum), _ptr(packed),
                                          _ptr(w_scale), M, N, K, _ptr(out), _ptr(acc_out),
                                          _stream(xq6.device)))
    return (out, acc_out) if acc_out is not None else out


def linear_forward(xq, x_scale, x_qsum, packed, w_scale, return_acc: bool = False, out=None,
                   acc_out=None):
    """Ternary contraction + dequant: y float32 [M][N] (and int32 accumulators if asked).

    ``out`` / ``acc_out`` may be preallocated [M][N] float32 / int32 tensors.
    """
    torch = _torch()
    _require(xq, "xq", torch.int8, 2)
    _require(x_scale, "x_scale", torch.float32, 1)
    _require(x_qsum, "x_qsum", torch.int32, 1)
    _require(packed, "packed", torch.uint8, 2)
    _require(w_scale, "w_scale", torch.float32, 1)
    M, K = xq.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError(f"packed is [{N}][{packed.shape[1]}], expected [{N}][{K // 4}] for K={K}")
    if x_scale.shape[0] != M or x_qsum.shape[0] != M or w_scale.shape[0] < 1:
        raise ValueError("x_scale / x_qsum must have M entries and w_scale at least one")
    if out is None:
        y = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    else:
        _require(out, "out", torch.float32, 2)
        if tuple(out.shape) != (M, N):
            raise ValueError(f"out must be [{M}][{N}]")
        y = out
    acc = acc_out
    if acc is not None:
        _require(acc, "acc_out", torch.int32, 2)
        if tuple(acc.shape) != (M, N):
            raise ValueError(f"acc_out must be [{M}][{N}]")
    elif return_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    _check(lib().bitnet_linear_forward(_ptr(xq), _ptr(x_scale), _ptr(x_qsum), _ptr(packed),
                                       _ptr(w_scale), M, N, K, _ptr(y), _ptr(acc),
                                       _stream(xq.device)))
    return (y, acc) if (return_acc or acc_out is not None) else y


def bitlinear_forward(x, packed, w_scale, gain=None, eps: float = 1e-5, out=None, codes=None,
                      acc_out=None):
    """Fused int8 BitLinear forward (bitnet_bitlinear_forward): bf16 [M][K] -> y float32 [M][N].

    ``codes`` may hold preallocated (xq, x_scale, x_qsum) for the intermediate
    codes (they are written); ``out`` / ``acc_out`` preallocated outputs.
    Returns y, or (y, acc) when ``acc_out`` is given.
    """
    torch = _torch()
    _require(x, "x", torch.bfloat16, 2)
    _require(packed, "packed", torch.uint8, 2)
    _require(w_scale, "w_scale", torch.float32, 1)
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError(f"packed is [{N}][{packed.shape[1]}], expected [{N}][{K // 4}] for K={K}")
    if gain is not None:
        _require(gain, "gain", torch.float32, 1)
    if codes is None:
        codes = (torch.empty((M, K), dtype=torch.int8, device=x.device),
                 torch.empty(M, dtype=torch.float32, device=x.device),
                 torch.empty(M, dtype=torch.int32, device=x.device))
    xq, x_scale, x_qsum = codes
    _require(xq, "xq", torch.int8, 2)
    _require(x_scale, "x_scale", torch.float32, 1)
    _require(x_qsum, "x_qsum", torch.int32, 1)
    if tuple(xq.shape) != (M, K) or x_scale.shape[0] != M or x_qsum.shape[0] != M:
        raise ValueError("codes tensors do not match x")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _require(out, "out", torch.float32, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}][{N}]")
    if acc_out is not None:
        _require(acc_out, "acc_out", torch.int32, 2)
        if tuple(acc_out.shape) != (M, N):
            raise ValueError(f"acc_out must be [{M}][{N}]")
    _check(lib().bitnet_bitlinear_forward(_ptr(x), _ptr(gain), ctypes.c_float(eps), _ptr(packed),
                                          _ptr(w_scale), M, N, K, _ptr(xq), _ptr(x_scale),
                                          _ptr(x_qsum), _ptr(out), _ptr(acc_out),
                                          _stream(x.device)))
    return (out, acc_out) if acc_out is not None else out


# --- backward under the straight-through estimator ------------------------

def base3_row_bytes(K: int) -> int:
    """Bytes per row of the base-3 packing (five weights per byte, rows padded to 16)."""
    return int(lib().bitnet_base3_row_bytes(K))


def pack_base3(packed, K: int, out=None):
    """2-bit packed uint8 [N][K/4] -> base-3 packed uint8 [N][base3_row_bytes(K)] (bitnet_pack_base3)."""
    torch = _torch()
    _require(packed, "packed", torch.uint8, 2)
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError(f"packed is [{N}][{packed.shape[1]}], expected [{N}][{K // 4}]")
    rb = base3_row_bytes(K)
    if out is None:
        out = torch.empty((N, rb), dtype=torch.uint8, device=packed.device)
    _check(lib().bitnet_pack_base3(_ptr(packed), N, K, _ptr(out), _stream(packed.device)))
    return out


def linear_forward_base3(xq, x_scale, x_qsum, packed3, w_scale, return_acc: bool = False, out=None):
    """One token on base-3 packed weights (bitnet_linear_forward_base3): y float32 [1][N]."""
    torch = _torch()
    _require(xq, "xq", torch.int8, 2)
    _require(x_scale, "x_scale", torch.float32, 1)
    _require(x_qsum, "x_qsum", torch.int32, 1)
    _require(packed3, "packed3", torch.uint8, 2)
    _require(w_scale, "w_scale", torch.float32, 1)
    M, K = xq.shape
    N = packed3.shape[0]
    if packed3.shape[1] != base3_row_bytes(K):
        raise ValueError(f"packed3 is [{N}][{packed3.shape[1]}], expected [{N}][{base3_row_bytes(K)}] for K={K}")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=xq.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device) if return_acc else None
    _check(lib().bitnet_linear_forward_base3(_ptr(xq), _ptr(x_scale), _ptr(x_qsum), _ptr(packed3),
                                             _ptr(w_scale), M, N, K, _ptr(y), _ptr(acc),
                                             _stream(xq.device)))
    return (y, acc) if return_acc else y


def transpose_packed(packed, K: int, out=None):
    """packed uint8 [N][K/4] -> packed_t uint8 [K][N/4] (bitnet_transpose_packed)."""
    torch = _torch()
    _require(packed, "packed", torch.uint8, 2)
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError(f"packed is [{N}][{packed.shape[1]}], expected [{N}][{K // 4}]")
    if out is None:
        out = torch.empty((K, N // 4), dtype=torch.uint8, device=packed.device)
    _check(lib().bitnet_transpose_packed(_ptr(packed), N, K, _ptr(out), _stream(packed.device)))
    return out


def linear_backward_input(grad_y, packed_t, w_scale, out=None):
    """grad_n float32 [M][K] = d_w * grad_y (bf16 [M][N]) @ q_w, from packed_t [K][N/4]."""
    torch = _torch()
    _require(grad_y, "grad_y", torch.bfloat16, 2)
    _require(packed_t, "packed_t", torch.uint8, 2)
    _require(w_scale, "w_scale", torch.float32, 1)
    M, N = grad_y.shape
    K = packed_t.shape[0]
    if packed_t.shape[1] * 4 != N:
        raise ValueError(f"packed_t is [{K}][{packed_t.shape[1]}], expected [{K}][{N // 4}]")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=grad_y.device)
    _check(lib().bitnet_linear_backward_input(_ptr(grad_y), _ptr(packed_t), _ptr(w_scale), M, N, K,
                                              _ptr(out), _stream(grad_y.device)))
    return out


def linear_backward_weight(grad_y, xq, x_scale, out=None, workspace=None):
    """grad_w float32 [N][K] = sum_m grad_y[m][n] d_x[m] q_x[m][k] (bitnet_linear_backward_weight)."""
    torch = _torch()
    _require(grad_y, "grad_y", torch.bfloat16, 2)
    _require(xq, "xq", torch.int8, 2)
    _require(x_scale, "x_scale", torch.float32, 1)
    M, N = grad_y.shape
    K = xq.shape[1]
    if xq.shape[0] != M or x_scale.shape[0] != M:
        raise ValueError("xq and x_scale must have M rows")
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=grad_y.device)
    need = int(lib().bitnet_linear_backward_weight_workspace_bytes(M, N, K))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=grad_y.device)
    _check(lib().bitnet_linear_backward_weight(_ptr(grad_y), _ptr(xq), _ptr(x_scale), M, N, K,
                                               _ptr(out), _ptr(workspace), workspace.numel(),
                                               _stream(grad_y.device)))
    return out


def rmsnorm_backward(x, grad_n, gain=None, eps: float = 1e-5, with_gain_grad: bool = False):
    """(grad_x float32 [M][K], grad_gain float32 [K] or None) of n = x * gain * r."""
    torch = _torch()
    _require(x, "x", torch.bfloat16, 2)
    _require(grad_n, "grad_n", torch.float32, 2)
    M, K = x.shape
    if tuple(grad_n.shape) != (M, K):
        raise ValueError("grad_n must have the shape of x")
    if gain is not None:
        _require(gain, "gain", torch.float32, 1)
    grad_x = torch.empty((M, K), dtype=torch.float32, device=x.device)
    grad_gain = torch.empty(K, dtype=torch.float32, device=x.device) if with_gain_grad else None
    ws, ws_bytes = None, 0
    if with_gain_grad:
        ws_bytes = int(lib().bitnet_rmsnorm_backward_workspace_bytes(M, K))
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=x.device)
    _check(lib().bitnet_rmsnorm_backward(_ptr(x), _ptr(gain), ctypes.c_float(eps), _ptr(grad_n), M, K,
                                         _ptr(grad_x), _ptr(grad_gain), _ptr(ws), ws_bytes,
                                         _stream(x.device)))
    return grad_x, grad_gain


def bitlinear(x, packed, w_scale, hadamard: bool = False, gain=None, eps: float = 1e-5):
    """One BitLinear forward: quantise bf16 activations, contract, dequantise."""
    if not hadamard:
        return bitlinear_forward(x, packed, w_scale, gain, eps)
    xq, x_scale, x_qsum = hadamard_quant_act(x, gain, eps)
    return linear_forward(xq, x_scale, x_qsum, packed, w_scale)


class BitLinear:
    """A bias-free linear layer with ternary weights, packed once at construction."""

    def __init__(self, weight, hadamard: bool = False, gain=None, eps: float = 1e-5):
        self.out_features, self.in_features = weight.shape
        self.hadamard = bool(hadamard)
        self.gain = gain
        self.eps = float(eps)
        self.packed, self.w_scale = pack_weights(weight, hadamard=self.hadamard)

    def __call__(self, x):
        return bitlinear(x, self.packed, self.w_scale, self.hadamard, self.gain, self.eps)
