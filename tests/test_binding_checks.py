"""The Python binding rejects caller-supplied tensors of the wrong shape, dtype
or device before anything reaches the C ABI (CPU only).  The C ABI takes raw
pointers and sizes, so these checks are the only guard against a buffer that
is too small for what a kernel writes or reads.

Tensors here are CPU tensors that report a GPU device (a torch.Tensor subclass
overriding ``device``): every call must raise ValueError during its argument
checks, before any allocation, stream query or library call, which on this
machine would fail differently."""
import pytest
import torch

import bit_gemm_ternary_amd as bt


class _OnGpu0(torch.Tensor):
    @property
    def device(self):
        return torch.device("cuda", 0)


class _OnGpu1(torch.Tensor):
    @property
    def device(self):
        return torch.device("cuda", 1)


def D(shape, dtype, cls=_OnGpu0):
    return torch.Tensor._make_subclass(cls, torch.zeros(shape, dtype=dtype))


u8, i8, i32, f32, bf16 = torch.uint8, torch.int8, torch.int32, torch.float32, torch.bfloat16
M, K, N = 4, 256, 512


def codes(m=M, k=K):
    return (D((m, k), i8), D((m,), f32), D((m,), i32))


def raises(fn, match=None):
    with pytest.raises(ValueError, match=match):
        fn()


def test_bitlinear_forward():
    x, p, w = D((M, K), bf16), D((N, K // 4), u8), D((2,), f32)
    out = D((M, N), f32)
    raises(lambda: bt.bitlinear_forward(x, p, w, gain=D((K - 1,), f32), codes=codes(), out=out), "gain")
    raises(lambda: bt.bitlinear_forward(x, p, w, codes=codes(k=K - 64), out=out), "xq")
    raises(lambda: bt.bitlinear_forward(x, p, w, codes=(D((M, K), i8), D((M - 1,), f32), D((M,), i32)),
                                        out=out), "x_scale")
    raises(lambda: bt.bitlinear_forward(x, p, w, codes=(D((M, K), i8), D((M,), f32), D((1,), i32)),
                                        out=out), "x_qsum")
    raises(lambda: bt.bitlinear_forward(x, p, w, codes=codes(), out=D((M, N - 1), f32)), "out")
    raises(lambda: bt.bitlinear_forward(x, p, w, codes=codes(), out=out, acc_out=D((M, 1), i32)), "acc_out")
    raises(lambda: bt.bitlinear_forward(x, D((N, K // 4 + 1), u8), w, codes=codes(), out=out), "packed")
    raises(lambda: bt.bitlinear_forward(x, p, D((0,), f32), codes=codes(), out=out), "w_scale")
    raises(lambda: bt.bitlinear_forward(x, D((N, K // 4), u8, _OnGpu1), w, codes=codes(), out=out), "packed")


def test_bitlinear_forward_grouped():
    x = D((M, K), bf16)
    rows = [256, 128, 128]
    p, ws = D((N, K // 4), u8), D((3, 2), f32)
    out = D((M, N), f32)
    raises(lambda: bt.bitlinear_forward_grouped(x, p, ws, rows, codes=codes(k=K // 2), out=out), "xq")
    raises(lambda: bt.bitlinear_forward_grouped(x, p, ws, rows, codes=(D((M, K), i8), D((M,), f32),
                                                                       D((M + 1,), i32)), out=out), "x_qsum")
    raises(lambda: bt.bitlinear_forward_grouped(x, p, ws, rows, gain=D((2 * K,), f32), codes=codes(),
                                                out=out), "gain")
    raises(lambda: bt.bitlinear_forward_grouped(x, p, D((2, 2), f32), rows, codes=codes(), out=out), "w_scales")
    raises(lambda: bt.bitlinear_forward_grouped(x, p, ws, [256, 128, 129], codes=codes(), out=out), "packed")
    raises(lambda: bt.bitlinear_forward_grouped(x, p, ws, rows, codes=codes(), out=D((M, N + 4), f32)), "out")
    raises(lambda: bt.bitlinear_forward_grouped(x, p, ws, [0, 256, 256], codes=codes(), out=out))
    raises(lambda: bt.bitlinear_forward_grouped(x, p, ws, rows, codes=codes(), out=out,
                                                acc_out=D((M, N - 1), i32)), "acc_out")


def test_quant_calls():
    x = D((M, K), bf16)
    raises(lambda: bt.quant_act(x, gain=D((K + 1,), f32), out=codes()), "gain")
    raises(lambda: bt.quant_act(x, out=codes(m=M + 1)), "xq")
    raises(lambda: bt.hadamard_quant_act(x, out=(D((M, K), i8), D((M,), f32), D((M, 1), i32))), "x_qsum")
    f6 = (D((M, K // 4 * 3), u8), D((M,), f32), D((M,), i32))
    raises(lambda: bt.hadamard_quant_act_f6(x, gain=D((K // 2,), f32), out=f6), "gain")
    raises(lambda: bt.hadamard_quant_act_f6(x, out=(D((M, K // 4 * 3), u8), D((M - 1,), f32), D((M,), i32))),
           "x_scale")
    raises(lambda: bt.hadamard_quant_act_f6(x, out=(D((M, K), u8), D((M,), f32), D((M,), i32))), "xq6")


def test_linear_forward_and_f6():
    xq, xs, qs = codes()
    p, w = D((N, K // 4), u8), D((2,), f32)
    raises(lambda: bt.linear_forward(xq, xs, qs, p, w, out=D((M, N + 1), f32)), "out")
    raises(lambda: bt.linear_forward(xq, xs, qs, p, w, out=D((M, N), f32), acc_out=D((N, M), i32)), "acc_out")
    raises(lambda: bt.linear_forward(xq, D((M + 1,), f32), qs, p, w), "x_scale")
    xq6 = D((M, K // 4 * 3), u8)
    out = D((M, N), f32)
    raises(lambda: bt.linear_forward_f6(xq6, D((M - 1,), f32), qs, p, w, out=out), "x_scale")
    with pytest.raises(TypeError, match="x_qsum"):
        bt.linear_forward_f6(xq6, xs, D((M,), f32), p, w, out=out)
    raises(lambda: bt.linear_forward_f6(xq6, xs, qs, p, D((0,), f32), out=out), "w_scale")
    raises(lambda: bt.linear_forward_f6(xq6, xs, qs, p, w, out=D((M, N // 2), f32)), "out")
    raises(lambda: bt.linear_forward_f6(xq6, xs, qs, p, w, out=out, acc_out=D((M, N // 2), i32)), "acc_out")
    raises(lambda: bt.linear_forward_f6(xq6, xs, qs, D((N, K // 8), u8), w, out=out), "packed")


def test_i4_calls():
    x = D((M, K), bf16)
    i4 = (D((M, K // 2), u8), D((M,), f32), D((M,), i32))
    raises(lambda: bt.hadamard_quant_act_i4(x, gain=D((K // 2,), f32), out=i4), "gain")
    raises(lambda: bt.hadamard_quant_act_i4(x, out=(D((M, K), u8), D((M,), f32), D((M,), i32))), "xq4")
    raises(lambda: bt.hadamard_quant_act_i4(x, out=(D((M, K // 2), u8), D((M + 1,), f32), D((M,), i32))),
           "x_scale")
    xq4, xs, qs = i4
    p, w = D((N, K // 4), u8), D((2,), f32)
    out = D((M, N), f32)
    raises(lambda: bt.linear_forward_i4(xq4, xs, qs, D((N, K // 2), u8), w, out=out), "packed")
    raises(lambda: bt.linear_forward_i4(xq4, D((M - 1,), f32), qs, p, w, out=out), "x_scale")
    raises(lambda: bt.linear_forward_i4(xq4, xs, qs, p, w, out=D((M, N - 1), f32)), "out")
    raises(lambda: bt.linear_forward_i4(xq4, xs, qs, p, w, out=out, acc_out=D((M, N + 4), i32)), "acc_out")
    with pytest.raises(TypeError, match="xq4"):
        bt.linear_forward_i4(D((M, K // 2), i8), xs, qs, p, w, out=out)


def test_hadamard_bitlinear_forward_calls():
    k = 1024
    x, p, w = D((1, k), bf16), D((N, k // 4), u8), D((2,), f32)
    i4 = (D((1, k // 2), u8), D((1,), f32), D((1,), i32))
    out = D((1, N), f32)
    f = bt.hadamard_bitlinear_forward
    raises(lambda: f(x, p, w, gain=D((k // 2,), f32), codes=i4, out=out), "gain")
    raises(lambda: f(x, p, w, codes=(D((1, k), u8), D((1,), f32), D((1,), i32)), out=out), "xq4")
    raises(lambda: f(x, p, w, codes=(D((1, k // 2), u8), D((2,), f32), D((1,), i32)), out=out), "x_scale")
    raises(lambda: f(x, p, w, codes=(D((1, k // 2), u8), D((1,), f32), D((3,), i32)), out=out), "x_qsum")
    raises(lambda: f(x, p, w, codes=i4, out=D((1, N + 1), f32)), "out")
    raises(lambda: f(x, p, w, codes=i4, out=out, acc_out=D((2, N), i32)), "acc_out")
    raises(lambda: f(x, D((N, k // 2), u8), w, codes=i4, out=out), "packed")
    raises(lambda: f(x, p, D((0,), f32), codes=i4, out=out), "w_scale")
    raises(lambda: f(x, D((N, k // 4), u8, _OnGpu1), w, codes=i4, out=out), "packed")
    with pytest.raises(TypeError, match="xq4"):
        f(x, p, w, codes=(D((1, k // 2), i8), D((1,), f32), D((1,), i32)), out=out)


def test_shard_calls():
    x = D((M, K), bf16)
    raises(lambda: bt.token_stats(x, gain=D((K + 8,), f32)), "gain")
    raises(lambda: bt.token_stats(x, out=(D((M + 1,), f32), D((M,), torch.float64))), "amax")
    with pytest.raises(TypeError, match="sumsq"):
        bt.token_stats(x, out=(D((M,), f32), D((M,), f32)))
    amax, ss = D((M,), f32), D((M,), torch.float64)
    raises(lambda: bt.quant_act_with_stats(x, D((M - 1,), f32), ss, 4 * K, out=codes()), "amax")
    with pytest.raises(TypeError, match="sumsq"):
        bt.quant_act_with_stats(x, amax, D((M,), f32), 4 * K, out=codes())
    raises(lambda: bt.quant_act_with_stats(x, amax, ss, 4 * K, out=codes(k=K - 64)), "xq")
    raises(lambda: bt.quant_act_with_stats(x, amax, ss, 4 * K, gain=D((K // 2,), f32), out=codes()), "gain")
    acc = D((M, N), i32)
    raises(lambda: bt.dequant(acc, D((M + 1,), f32), D((2,), f32), out=D((M, N), f32)), "x_scale")
    raises(lambda: bt.dequant(acc, D((M,), f32), D((0,), f32), out=D((M, N), f32)), "w_scale")
    raises(lambda: bt.dequant(acc, D((M,), f32), D((2,), f32), out=D((M, N - 4), f32)), "out")
    with pytest.raises(TypeError, match="acc"):
        bt.dequant(D((M, N), f32), D((M,), f32), D((2,), f32))


def test_base3_calls():
    p = D((N, K // 4), u8)
    rb = bt.base3_row_bytes(K)
    raises(lambda: bt.pack_base3(p, K, out=D((N, rb - 16), u8)), "out")
    raises(lambda: bt.pack_base3(p, K, out=D((N - 1, rb), u8)), "out")
    xq, xs, qs = codes(m=1)
    raises(lambda: bt.linear_forward_base3(xq, xs, qs, D((N, rb), u8), D((2,), f32), out=D((1, N - 1), f32)),
           "out")
    raises(lambda: bt.linear_forward_base3(xq, xs, qs, D((N, rb + 16), u8), D((2,), f32)), "packed3")


def test_backward_calls():
    p = D((N, K // 4), u8)
    raises(lambda: bt.transpose_packed(p, K, out=D((K, N // 4 - 1), u8)), "out")
    gy, pt, w = D((M, N), bf16), D((K, N // 4), u8), D((2,), f32)
    raises(lambda: bt.linear_backward_input(gy, pt, w, out=D((M, K + 64), f32)), "out")
    raises(lambda: bt.linear_backward_input(gy, pt, D((0,), f32), out=D((M, K), f32)), "w_scale")
    xq = D((M, K), i8)
    raises(lambda: bt.linear_backward_weight(gy, xq, D((M, 1), f32), out=D((N, K), f32)), "x_scale")
    raises(lambda: bt.linear_backward_weight(gy, xq, D((M,), f32), out=D((N, K - 64), f32)), "out")
    raises(lambda: bt.linear_backward_weight(gy, D((M + 1, K), i8), D((M,), f32)), "xq")
    x = D((M, K), bf16)
    raises(lambda: bt.rmsnorm_backward(x, D((M, K), f32), gain=D((K - 64,), f32)), "gain")
    raises(lambda: bt.rmsnorm_backward(x, D((M, K + 64), f32)), "grad_n")


def test_pack_weights():
    W = D((N, K), f32)
    raises(lambda: bt.pack_weights(W, out=(D((N, K // 4 - 1), u8), D((2,), f32))), "packed")
    raises(lambda: bt.pack_weights(W, out=(D((N, K // 4), u8), D((1,), f32))), "w_scale")
    raises(lambda: bt.pack_weights(W, out=(D((N, K // 4), u8), D((2,), f32)),
                                   workspace=D((16,), u8, _OnGpu1)), "workspace")


def test_stream_read():
    raises(lambda: bt.stream_read(D((1024,), u8), D((0,), i32)), "sink")
    raises(lambda: bt.stream_read(D((1024,), u8), D((1,), i32, _OnGpu1)), "sink")
