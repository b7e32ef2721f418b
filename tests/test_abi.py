"""The C-ABI library loads, exports every symbol include/bitnet.h declares, and
rejects bad arguments on the host before any HIP call (CPU only: nothing here
launches work or touches device memory; the pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import bit_gemm_ternary_amd as bt
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "bitnet.h")

A16 = 0x10000      # 16-byte-aligned stand-in addresses, never dereferenced
A4 = 0x10004
BAD = 0x10001


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitnet_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return bt.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"bitnet_pack_weights", "bitnet_quant_act", "bitnet_hadamard_quant_act",
            "bitnet_linear_forward"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_header_enum_matches_binding():
    text = open(HEADER).read()
    enum = dict((name, int(v)) for name, v in re.findall(r"(BITNET_[A-Z_]+)\s*=\s*(\d+)", text))
    assert {v: k for k, v in enum.items()} == bt.STATUS


def test_version_and_status_strings(L):
    assert L.bitnet_version() == 1
    for s in range(8):
        assert L.bitnet_status_string(s)
    assert L.bitnet_status_string(99) == b"unknown status"


def _quant(L, name, x=A16, gain=None, eps=1e-5, M=4, K=256, xq=A16, sx=A4, qs=A4):
    return getattr(L, name)(ctypes.c_void_p(x), None if gain is None else ctypes.c_void_p(gain),
                            ctypes.c_float(eps), M, K, ctypes.c_void_p(xq), ctypes.c_void_p(sx),
                            ctypes.c_void_p(qs), None)


@pytest.mark.parametrize("name", ["bitnet_quant_act", "bitnet_hadamard_quant_act"])
def test_quant_argument_errors(L, name):
    assert _quant(L, name, M=-1) == 2
    for K in (0, 32, 100, 65600):
        assert _quant(L, name, K=K) == 2
    assert _quant(L, name, eps=-1.0) == 7
    assert _quant(L, name, eps=float("nan")) == 7
    assert _quant(L, name, x=0) == 1
    assert _quant(L, name, qs=0) == 1
    assert _quant(L, name, x=BAD) == 4
    assert _quant(L, name, xq=A4) == 4
    assert _quant(L, name, gain=A4) == 4
    assert _quant(L, name, M=0, x=0) == 0     # empty batch: no-op, nothing dereferenced
    assert b"must" in L.bitnet_last_error() or b"out of range" in L.bitnet_last_error()


def test_hadamard_needs_power_of_two(L):
    assert _quant(L, "bitnet_hadamard_quant_act", K=192) == 3
    assert _quant(L, "bitnet_hadamard_quant_act", K=128) == 3
    assert _quant(L, "bitnet_hadamard_quant_act", K=65536) == 3
    assert b"power of two" in L.bitnet_last_error()


def _pack(L, W=A16, N=8, K=256, had=0, packed=A16, ws=A4, work=A16, work_bytes=1 << 20):
    return L.bitnet_pack_weights(ctypes.c_void_p(W), N, K, had, ctypes.c_void_p(packed),
                                 ctypes.c_void_p(ws), ctypes.c_void_p(work), work_bytes, None)


def test_pack_argument_errors(L):
    assert _pack(L, N=0) == 2
    assert _pack(L, K=100) == 2
    assert _pack(L, had=2) == 7
    assert _pack(L, had=1, K=192) == 3
    assert _pack(L, W=0) == 1
    assert _pack(L, work=0) == 1
    assert _pack(L, W=BAD) == 4
    assert _pack(L, work_bytes=8) == 5
    assert b"needed" in L.bitnet_last_error()


def test_pack_workspace_size(L):
    assert L.bitnet_pack_weights_workspace_bytes(100, 256, 0) == 1024      # 800 B of sums, padded
    assert L.bitnet_pack_weights_workspace_bytes(100, 256, 1) == 1024 + 100 * 256 * 4
    assert L.bitnet_pack_weights_workspace_bytes(0, 256, 0) == 0


def _fwd(L, xq=A16, sx=A4, qs=A4, P=A16, ws=A4, M=2, N=8, K=256, y=A4, acc=None):
    return L.bitnet_linear_forward(ctypes.c_void_p(xq), ctypes.c_void_p(sx), ctypes.c_void_p(qs),
                                   ctypes.c_void_p(P), ctypes.c_void_p(ws), M, N, K,
                                   ctypes.c_void_p(y), None if acc is None else ctypes.c_void_p(acc),
                                   None)


def test_forward_argument_errors(L):
    assert _fwd(L, M=-1) == 2
    assert _fwd(L, N=-5) == 2
    assert _fwd(L, K=96) == 2
    assert _fwd(L, y=0) == 1
    assert _fwd(L, P=0) == 1
    assert _fwd(L, xq=A4) == 4
    assert _fwd(L, P=BAD) == 4
    assert _fwd(L, y=BAD) == 4
    assert _fwd(L, acc=BAD) == 4
    assert _fwd(L, M=0, xq=0, y=0) == 0       # empty: no-op
    assert _fwd(L, N=0, xq=0, y=0) == 0


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        bt.quant_act(torch.zeros((2, 64), dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        bt.quant_act(torch.zeros((2, 64), dtype=torch.float32))


def _fused(L, x=A16, gain=None, eps=1e-5, P=A16, ws=A4, M=1, N=8, K=256, xq=A16, sx=A4, qs=A4,
           y=A4, acc=None):
    return L.bitnet_bitlinear_forward(
        ctypes.c_void_p(x), None if gain is None else ctypes.c_void_p(gain), ctypes.c_float(eps),
        ctypes.c_void_p(P), ctypes.c_void_p(ws), M, N, K, ctypes.c_void_p(xq), ctypes.c_void_p(sx),
        ctypes.c_void_p(qs), ctypes.c_void_p(y), None if acc is None else ctypes.c_void_p(acc), None)


def test_fused_forward_argument_errors(L):
    assert _fused(L, M=-1) == 2
    assert _fused(L, N=-1) == 2
    assert _fused(L, K=100) == 2
    assert _fused(L, eps=-1.0) == 7
    assert _fused(L, x=0) == 1
    assert _fused(L, P=0) == 1
    assert _fused(L, y=0) == 1
    assert _fused(L, x=BAD) == 4
    assert _fused(L, P=A4) == 4
    assert _fused(L, acc=BAD) == 4
    assert _fused(L, M=0, x=0, P=0, y=0) == 0


def _hfused(L, x=A16, gain=None, eps=1e-5, P=A16, ws=A4, M=1, N=8, K=1024, xq4=A16, sx=A4, qs=A4,
            y=A4, acc=None):
    return L.bitnet_hadamard_bitlinear_forward(
        ctypes.c_void_p(x), None if gain is None else ctypes.c_void_p(gain), ctypes.c_float(eps),
        ctypes.c_void_p(P), ctypes.c_void_p(ws), M, N, K, ctypes.c_void_p(xq4), ctypes.c_void_p(sx),
        ctypes.c_void_p(qs), ctypes.c_void_p(y), None if acc is None else ctypes.c_void_p(acc), None)


def test_hadamard_fused_forward_argument_errors(L):
    assert _hfused(L, M=-1) == 2
    assert _hfused(L, N=-1) == 2
    assert _hfused(L, K=100) == 2          # not a multiple of 64
    assert _hfused(L, K=384) == 3          # not a power of two
    assert _hfused(L, K=128) == 3          # below 256
    assert _hfused(L, K=65536) == 3        # above 32768
    assert _hfused(L, eps=-1.0) == 7
    assert _hfused(L, x=0) == 1
    assert _hfused(L, xq4=0) == 1
    assert _hfused(L, P=0) == 1
    assert _hfused(L, ws=0) == 1
    assert _hfused(L, y=0) == 1
    assert _hfused(L, x=BAD) == 4
    assert _hfused(L, xq4=A4) == 4
    assert _hfused(L, sx=BAD) == 4
    assert _hfused(L, P=A4) == 4
    assert _hfused(L, y=BAD) == 4
    assert _hfused(L, acc=BAD) == 4
    assert _hfused(L, M=0, x=0, xq4=0, P=0, y=0) == 0


def test_shard_argument_errors(L):
    p = ctypes.c_void_p
    A8 = 0x10008
    st = lambda x=A16, gain=None, M=2, K=256, amax=A4, ss=A8: L.bitnet_token_stats(
        p(x), None if gain is None else p(gain), M, K, p(amax), p(ss), None)
    assert st(M=-1) == 2
    assert st(K=100) == 2
    assert st(x=0) == 1
    assert st(ss=0) == 1
    assert st(x=A4) == 4
    assert st(gain=A4) == 4
    assert st(ss=A4) == 4                  # float64 output needs 8-byte alignment
    assert st(M=0, x=0) == 0

    def qs(x=A16, M=2, K=256, Kt=1024, amax=A4, ss=A8, xq=A16, sx=A4, q=A4, eps=1e-5):
        return L.bitnet_quant_act_with_stats(p(x), None, ctypes.c_float(eps), M, K, Kt, p(amax), p(ss),
                                             p(xq), p(sx), p(q), None)
    assert qs(Kt=128) == 2                 # K_total below K
    assert qs(Kt=(1 << 24) + 1) == 2
    assert qs(K=100) == 2
    assert qs(eps=-1.0) == 7
    assert qs(amax=0) == 1
    assert qs(xq=0) == 1
    assert qs(ss=A4) == 4
    assert qs(xq=A4) == 4
    assert qs(M=0, x=0, amax=0) == 0

    dq = lambda acc=A4, sx=A4, ws=A4, M=2, N=8, y=A4: L.bitnet_dequant(p(acc), p(sx), p(ws), M, N, p(y), None)
    assert dq(M=-1) == 2
    assert dq(N=-1) == 2
    assert dq(acc=0) == 1
    assert dq(y=0) == 1
    assert dq(acc=BAD) == 4
    assert dq(y=BAD) == 4
    assert dq(M=0, acc=0) == 0
    assert dq(N=0, y=0) == 0


def test_kernel_events_hook_is_exported(L):
    assert L.bitnet_set_kernel_events(None, None) == 0


def _grouped(L, rows=(8, 4), x=A16, gain=None, eps=1e-5, P=A16, ws=A4, M=1, K=256, xq=A16, sx=A4,
             qs=A4, y=A4, acc=None, groups=None, null_rows=False):
    rows_c = (ctypes.c_int64 * max(len(rows), 1))(*rows)
    return L.bitnet_bitlinear_forward_grouped(
        ctypes.c_void_p(x), None if gain is None else ctypes.c_void_p(gain), ctypes.c_float(eps),
        ctypes.c_void_p(P), ctypes.c_void_p(ws),
        None if null_rows else ctypes.cast(rows_c, ctypes.c_void_p),
        len(rows) if groups is None else groups, M, K, ctypes.c_void_p(xq), ctypes.c_void_p(sx),
        ctypes.c_void_p(qs), ctypes.c_void_p(y), None if acc is None else ctypes.c_void_p(acc), None)


def test_grouped_forward_argument_errors(L):
    assert _grouped(L, M=-1) == 2
    assert _grouped(L, K=100) == 2
    assert _grouped(L, eps=-1.0) == 7
    assert _grouped(L, groups=0) == 2
    assert _grouped(L, rows=tuple([4] * 9)) == 2           # more than 8 groups
    assert _grouped(L, rows=(8, 0, 4)) == 2                # an empty group
    assert _grouped(L, rows=(2 ** 31 - 1, 1)) == 2         # total rows past 2^31 - 1
    assert _grouped(L, null_rows=True) == 1
    assert _grouped(L, x=0) == 1
    assert _grouped(L, P=0) == 1
    assert _grouped(L, ws=0) == 1
    assert _grouped(L, y=0) == 1
    assert _grouped(L, x=BAD) == 4
    assert _grouped(L, P=A4) == 4
    assert _grouped(L, ws=BAD) == 4
    assert _grouped(L, acc=BAD) == 4
    assert _grouped(L, M=0, x=0, P=0, y=0) == 0


def test_f6_argument_errors(L):
    q = lambda **kw: _quant(L, "bitnet_hadamard_quant_act_f6", **kw)
    assert q(K=384) == 3          # not a power of two
    assert q(M=-1) == 2
    assert q(x=0) == 1
    assert q(xq=BAD) == 4

    def fwd(xq=A16, sx=A4, qs=A4, P=A16, ws=A4, M=4, N=8, K=256, y=A4, acc=None):
        return L.bitnet_linear_forward_f6(ctypes.c_void_p(xq), ctypes.c_void_p(sx),
                                          ctypes.c_void_p(qs), ctypes.c_void_p(P),
                                          ctypes.c_void_p(ws), M, N, K, ctypes.c_void_p(y),
                                          None if acc is None else ctypes.c_void_p(acc), None)
    assert fwd(K=100) == 2
    assert fwd(M=-1) == 2
    assert fwd(xq=0) == 1
    assert fwd(xq=A4) == 4
    assert fwd(acc=BAD) == 4
    assert fwd(M=0, xq=0) == 0


def test_i4_argument_errors(L):
    q = lambda **kw: _quant(L, "bitnet_hadamard_quant_act_i4", **kw)
    assert q(K=384) == 3          # not a power of two
    assert q(K=128) == 3          # below 256
    assert q(M=-1) == 2
    assert q(x=0) == 1
    assert q(xq=BAD) == 4

    def fwd(xq=A16, sx=A4, qs=A4, P=A16, ws=A4, M=4, N=8, K=256, y=A4, acc=None):
        return L.bitnet_linear_forward_i4(ctypes.c_void_p(xq), ctypes.c_void_p(sx),
                                          ctypes.c_void_p(qs), ctypes.c_void_p(P),
                                          ctypes.c_void_p(ws), M, N, K, ctypes.c_void_p(y),
                                          None if acc is None else ctypes.c_void_p(acc), None)
    assert fwd(K=100) == 2
    assert fwd(M=-1) == 2
    assert fwd(N=-1) == 2
    assert fwd(xq=0) == 1
    assert fwd(y=0) == 1
    assert fwd(xq=A4) == 4
    assert fwd(P=A4) == 4
    assert fwd(acc=BAD) == 4
    assert fwd(M=0, xq=0) == 0
    assert fwd(N=0, P=0) == 0


def test_backward_argument_errors(L):
    p = ctypes.c_void_p
    # transpose: N and K multiples of 64, pointers 16-byte aligned
    assert L.bitnet_transpose_packed(p(A16), 100, 256, p(A16), None) == 2
    assert L.bitnet_transpose_packed(p(A16), 128, 96, p(A16), None) == 2
    assert L.bitnet_transpose_packed(None, 128, 256, p(A16), None) == 1
    assert L.bitnet_transpose_packed(p(A16), 128, 256, p(A4), None) == 4
    # grad_n
    bi = lambda gy=A16, pt=A16, ws=A4, M=8, N=128, K=256, out=A4: L.bitnet_linear_backward_input(
        p(gy), p(pt), p(ws), M, N, K, p(out), None)
    assert bi(M=-1) == 2
    assert bi(N=96) == 2
    assert bi(K=32) == 2
    assert bi(gy=0) == 1
    assert bi(out=0) == 1
    assert bi(gy=A4) == 4
    assert bi(pt=BAD) == 4
    assert bi(M=0, gy=0, pt=0) == 0   # empty batch: nothing enqueued
    # grad_w: workspace size and alignment
    need = L.bitnet_linear_backward_weight_workspace_bytes(8, 128, 256)
    assert need == (2 * 128 + 256) * 64 * 2
    assert L.bitnet_linear_backward_weight_workspace_bytes(0, 128, 256) == 0
    assert L.bitnet_linear_backward_weight_workspace_bytes(8, 100, 256) == 0
    assert L.bitnet_linear_backward_weight_workspace_bytes(2 ** 21, 128, 256) > 0
    assert L.bitnet_linear_backward_weight_workspace_bytes(2 ** 21 + 1, 128, 256) == 0
    bw = lambda gy=A16, xq=A16, sx=A4, M=8, N=128, K=256, out=A4, ws=A16, wsb=need: \
        L.bitnet_linear_backward_weight(p(gy), p(xq), p(sx), M, N, K, p(out), p(ws), wsb, None)
    assert bw(N=64 + 32) == 2
    assert bw(M=2 ** 21 + 1) == 2
    assert bw(out=0) == 1
    assert bw(gy=0) == 1
    assert bw(xq=A4) == 4
    assert bw(ws=0) == 5
    assert bw(wsb=need - 1) == 5
    assert bw(ws=A4) == 4
    # RMSNorm backward: the workspace is needed only with a gain gradient
    rb = lambda x=A16, g=None, eps=1e-5, gn=A4, M=8, K=256, gx=A4, gg=None, ws=None, wsb=0: \
        L.bitnet_rmsnorm_backward(p(x), None if g is None else p(g), ctypes.c_float(eps), p(gn), M, K,
                                  p(gx), None if gg is None else p(gg), None if ws is None else p(ws),
                                  wsb, None)
    assert rb(K=100) == 2
    assert rb(eps=-1.0) == 7
    assert rb(x=0) == 1
    assert rb(gx=BAD) == 4
    assert rb(gg=A4) == 5
    assert rb(gg=A4, ws=A4, wsb=L.bitnet_rmsnorm_backward_workspace_bytes(8, 256)) == 4
    assert L.bitnet_rmsnorm_backward_workspace_bytes(8, 256) == 32 * 8 + 1 * 256 * 8


def test_base3_argument_errors(L):
    p = ctypes.c_void_p
    # row bytes: ceil(K / 5) rounded up to 16; 0 for an invalid K
    assert L.bitnet_base3_row_bytes(64) == 16
    assert L.bitnet_base3_row_bytes(4096) == 832
    assert L.bitnet_base3_row_bytes(11008) == 2208
    assert L.bitnet_base3_row_bytes(100) == 0
    assert L.bitnet_base3_row_bytes(0) == 0
    # repack: K rules of the packing, pointers 16-byte aligned
    assert L.bitnet_pack_base3(p(A16), 8, 96, p(A16), None) == 2
    assert L.bitnet_pack_base3(p(A16), -1, 256, p(A16), None) == 2
    assert L.bitnet_pack_base3(None, 8, 256, p(A16), None) == 1
    assert L.bitnet_pack_base3(p(A16), 8, 256, p(A4), None) == 4
    assert L.bitnet_pack_base3(None, 0, 256, None, None) == 0          # nothing to pack
    # one-token contraction
    f = lambda xq=A16, sx=A4, qs=A4, p3=A16, ws=A4, M=1, N=8, K=256, y=A4, acc=None: \
        L.bitnet_linear_forward_base3(p(xq), p(sx), p(qs), p(p3), p(ws), M, N, K, p(y),
                                      None if acc is None else p(acc), None)
    assert f(M=2) == 3                       # one token only
    assert f(K=20544) == 3                   # above 20480
    assert f(K=100) == 2
    assert f(N=-1) == 2
    assert f(xq=0) == 1
    assert f(p3=A4) == 4
    assert f(y=BAD) == 4
    assert f(M=0, xq=0, p3=0) == 0           # empty batch: nothing enqueued


def test_stream_read_argument_errors(L):
    f = L.bitnet_stream_read
    v = ctypes.c_void_p
    assert f(v(A16), 0, v(A4), None) == 2
    assert f(v(A16), 24, v(A4), None) == 2
    assert f(v(A16), 8, v(A4), None) == 2
    assert f(None, 1024, v(A4), None) == 1
    assert f(v(A16), 1024, None, None) == 1
    assert f(v(A4), 1024, v(A4), None) == 4
    assert f(v(A16), 1024, v(BAD), None) == 4


def test_pack_noalloc_argument_errors(L):
    f = L.bitnet_pack_weights_noalloc
    v = ctypes.c_void_p
    assert f(v(A16), 0, 256, 0, v(A16), v(A4), None) == 2
    assert f(v(A16), 8, 100, 0, v(A16), v(A4), None) == 2
    assert f(v(A16), 8, 256, 2, v(A16), v(A4), None) == 7
    assert f(v(A16), 8, 192, 1, v(A16), v(A4), None) == 3
    assert f(None, 8, 256, 0, v(A16), v(A4), None) == 1
    assert f(v(A16), 8, 256, 0, v(A16), None, None) == 1
    assert f(v(A4), 8, 256, 0, v(A16), v(A4), None) == 4
    assert f(v(A16), 8, 256, 0, v(A16), v(BAD), None) == 4
    # Beyond the static scratch: refused before any HIP call.
    cap = bt.NOALLOC_SCRATCH_BYTES
    rows = cap // 8 + 1
    assert L.bitnet_pack_weights_workspace_bytes(rows, 256, 0) > cap
    assert f(v(A16), rows, 256, 0, v(A16), v(A4), None) == 5
    assert b"scratch" in L.bitnet_last_error()
    assert L.bitnet_pack_weights_workspace_bytes(512, 4096, 1) > cap
    assert f(v(A16), 512, 4096, 1, v(A16), v(A4), None) == 5


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define BITNET_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == bt.NOALLOC_SCRATCH_BYTES


def test_blend_argument_errors(L):
    f = L.bitnet_linear_forward_blend
    v = ctypes.c_void_p
    ws = L.bitnet_linear_forward_blend_workspace_bytes(4, 256)
    assert ws >= 4 * 256 * 5
    ok = dict(x=v(A16), gain=None, eps=1e-5, W=v(A16), packed=v(A16), w=v(A4), lam=0.5, M=4, N=8, K=256,
              y=v(A4), ws=v(A16), wsb=ws)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["gain"], ctypes.c_float(a["eps"]), a["W"], a["packed"], a["w"],
                 ctypes.c_float(a["lam"]), a["M"], a["N"], a["K"], a["y"], a["ws"], a["wsb"], None)

    assert call(lam=-0.1) == 7
    assert call(lam=1.5) == 7
    assert call(lam=float("nan")) == 7
    assert call(K=100) == 2
    assert call(M=-1) == 2
    assert call(eps=-1.0) == 7
    assert call(W=None) == 1
    assert call(ws=None) == 1
    assert call(x=v(A4)) == 4
    assert call(gain=v(A4)) == 4
    assert call(wsb=ws - 1) == 5
    assert call(M=0, x=None, W=None) == 0
