"""bitnet_pack_weights_noalloc (library-owned static scratch, no allocation)
against bitnet_pack_weights (caller workspace) through the C ABI: packed bytes
and both scales bit-identical, on two calls in a row with the second one
smaller (the scratch keeps the first call's contents), with and without the
Hadamard pre-rotation, plus the oracle on the same inputs."""
import ctypes

import numpy as np
import pytest

import bit_gemm_ternary_amd as bt
from bit_gemm_ternary_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    bt.lib()
    return torch.device("cuda:0")


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _with_workspace(L, W, hadamard, dev):
    N, K = W.shape
    packed = torch.full((N, K // 4), 0xEE, dtype=torch.uint8, device=dev)
    w_scale = torch.full((2,), -1.0, dtype=torch.float32, device=dev)
    need = L.bitnet_pack_weights_workspace_bytes(N, K, hadamard)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    st = L.bitnet_pack_weights(_p(W), N, K, hadamard, _p(packed), _p(w_scale), _p(ws), ws.numel(),
                               _stream(dev))
    assert st == 0, L.bitnet_last_error()
    return packed, w_scale


def _noalloc(L, W, hadamard, dev):
    N, K = W.shape
    packed = torch.full((N, K // 4), 0xEE, dtype=torch.uint8, device=dev)
    w_scale = torch.full((2,), -1.0, dtype=torch.float32, device=dev)
    st = L.bitnet_pack_weights_noalloc(_p(W), N, K, hadamard, _p(packed), _p(w_scale), _stream(dev))
    assert st == 0, L.bitnet_last_error()
    return packed, w_scale


# (N, K, hadamard) of the first, larger call and of the second, smaller one.
SEQUENCES = [
    ((4096, 4096, 0), (300, 1024, 0)),        # decode projection, then a ragged small matrix
    ((131072, 256, 0), (33, 64, 0)),          # 1 MiB of row sums, then a tiny matrix
    ((64, 4096, 1), (5, 256, 1)),             # rotated rows in the scratch (1 MiB + sums)
    ((250, 4096, 1), (64, 2048, 1)),          # near the scratch's size with the rotation
]


@pytest.mark.parametrize("first,second", SEQUENCES)
def test_noalloc_matches_workspace_entry_point(dev, orc, first, second):
    L = bt.lib()
    for seed, (N, K, had) in enumerate((first, second)):
        print(f"noalloc case N={N} K={K} hadamard={had}", flush=True)
        assert L.bitnet_pack_weights_workspace_bytes(N, K, had) <= bt.NOALLOC_SCRATCH_BYTES
        Wh = synth.weights(N, K, seed=9100 + seed)
        W = torch.from_numpy(Wh).to(dev)
        want_p, want_s = _with_workspace(L, W, had, dev)
        got_p, got_s = _noalloc(L, W, had, dev)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got_p.cpu().numpy(), want_p.cpu().numpy())
        np.testing.assert_array_equal(got_s.cpu().numpy(), want_s.cpu().numpy())
        if N * K <= 1 << 22:
            ref_p, ref_dw, ref_sw, _ = orc.pack_weights(Wh, hadamard=bool(had))
            np.testing.assert_array_equal(got_p.cpu().numpy(), ref_p)
            assert got_s.cpu().numpy().tolist() == [np.float32(ref_dw), np.float32(ref_sw)]


def test_noalloc_refuses_more_than_its_scratch(dev):
    L = bt.lib()
    N, K = 512, 4096
    assert L.bitnet_pack_weights_workspace_bytes(N, K, 1) > bt.NOALLOC_SCRATCH_BYTES
    W = torch.zeros((N, K), dtype=torch.float32, device=dev)
    packed = torch.full((N, K // 4), 7, dtype=torch.uint8, device=dev)
    w_scale = torch.full((2,), 3.0, dtype=torch.float32, device=dev)
    st = L.bitnet_pack_weights_noalloc(_p(W), N, K, 1, _p(packed), _p(w_scale), _stream(dev))
    assert st == 5
    torch.cuda.synchronize()
    assert (packed.cpu().numpy() == 7).all() and (w_scale.cpu().numpy() == 3.0).all()


def test_noalloc_python_binding(dev):
    W = torch.from_numpy(synth.weights(777, 512, seed=9200)).to(dev)
    out = (torch.empty((777, 128), dtype=torch.uint8, device=dev),
           torch.empty(2, dtype=torch.float32, device=dev))
    got_p, got_s = bt.pack_weights_noalloc(W, out)
    want_p, want_s = bt.pack_weights(W)
    torch.cuda.synchronize()
    assert torch.equal(got_p, want_p) and torch.equal(got_s, want_s)
