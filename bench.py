#!/usr/bin/env python3
"""BitLinear forward benchmark on one MI355X.

Headline (one JSON line on stdout): decode GEMV weight GB/s.  A step is one
W1.58A8 decode forward (M = 1) through the three Llama-7B-shaped projections
(K, N) = (4096, 4096), (4096, 11008), (11008, 4096): per projection, RMSNorm +
int8 quantisation of the bf16 token fused into the ternary GEMV with its
dequantisation epilogue (bitnet_bitlinear_forward, one kernel).  Inputs are
resident in HBM; the packed weights rotate over enough distinct copies
(> 1 GiB) that the 256 MB Infinity Cache cannot serve them, so every step
streams its weights from HBM.  The --steps timed steps are captured into ONE
HIP graph, replayed once untimed, and the timed region is a single replay of
it after a cache flush (a plain 1 GiB read of another buffer), so the
region measures the GPU, not Python or per-launch host overhead, whatever
--steps is.

  value            packed weight bytes per step / step time (GB/s); config also
                   gives it as a fraction of a plain 2 GiB read (bitnet_stream_read)
                   and the warm number (one weight copy, Infinity-Cache resident)
  roofline         the fused decode kernel alone: algorithmic bytes (packed
                   weights, bf16 activations, codes and outputs) per launch /
                   launch duration, each projection launched back to back in one
                   HIP graph over its own >= 1 GiB weight rotation, timed by HIP
                   events on the graph's stream (median over five regions;
                   per_launch also gives the median eager duration of one launch
                   on an idle GPU, from events stamped by the kernel's own dispatch)
  decode_sizes     context: the same fused decode kernel (M = 1) on larger
                   projections (8192 x 8192 up to 16384 x 53248), launched back to
                   back like roofline.per_launch: per-launch time and GB/s once the
                   launch's fixed cost is spread over 17-218 MB of packed weights
  base3            context: the one-token contraction on base-3 packed weights (five
                   per byte, 1.6 bits) against the 2-bit packing, codes precomputed
  prefill          W1.58A8 prefill M=2048, K=4096, N=14336: int8 TOPS of the
                   matrix-core GEMM against the dense int8 peak, and against that
                   peak scaled to the engine clock measured during the kernel
                   (committed counter summary)
  hadamard         H-BitLinear M=512: FWHT + int4 quantisation GB/s and GEMM TOPS,
                   for int8 codes (int8 matrix core) and for 6-bit E3M2 codes (FP4 x
                   FP6 matrix core, against the 10.1 PFLOP/s fp6 peak), packed 4-bit
                   codes; one token through the layer as two kernels and as the
                   single fused launch
  block            the seven BitLinear projections of a Llama-3-8B block at
                   M = 1, 16 and 256 tokens: time per block, packed weight GB/s,
                   int TOPS
  shard            one device's share of that block split eight ways (M = 1):
                   q|k|v and gate|up by output features, o and down by input
                   features (statistics, quantisation with the whole token's
                   statistics, int32 partial sums, dequantisation); time per
                   share and per kernel, collectives not run
  backward         STE backward of the prefill layer: grad_n and grad_w on the bf16
                   matrix cores, RMSNorm backward, packed-weight transpose
  blend            the warm-up blend of the prefill layer (lambda = 0.5): the
                   float32 contraction of blended operands, TFLOP/s against the
                   fp32 matrix-core peak
  pack             offline weight preparation (absmean scale, ternarise, pack;
                   with the Hadamard pre-rotation for the H-BitLinear weight):
                   time per matrix and GB/s of its two passes over W
  cpu_baseline     the CPU oracle on this host running the same decode step, on
                   all cores and on one core

roofline.traffic is the HBM bytes per launch of the fused decode kernel that
rocprofv3's FETCH_SIZE and WRITE_SIZE counters read, scaled by what the same
counters read for a plain device copy of known size (--copy-calibration); it is
read from the committed counter summary and reported as null when the kernel
source has changed since those counters were taken.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix-core peak, 5.0 POP/s
PEAK_CLOCK_GHZ = 2.4        # the engine clock that peak is quoted at
FP6_PEAK_TOPS = 10100.0     # MI355X dense fp6 / fp4 matrix-core peak, 10.1 PFLOP/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak, 2.5 PFLOP/s
FP32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix-core peak
ROTATE_BYTES = 1 << 30      # > 4 x the 256 MB Infinity Cache
METRIC = "BitLinear decode GEMV weight GB/s (%HBM peak); prefill int8 TOPS (%MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-iters", type=int, default=30)
    ap.add_argument("--pack-iters", type=int, default=10, help="timed calls per matrix of the pack leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall time budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the prefill / H-BitLinear legs")
    ap.add_argument("--eager", action="store_true", help="launch steps eagerly instead of from graphs")
    ap.add_argument("--block-steps", type=int, default=200, help="timed steps per token count of the block leg")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of COPY_BYTES, ten times (HBM counter calibration)")
    ap.add_argument("--legs", default="decode,decode_sizes,base3,prefill,hadamard,block,shard,backward,blend,pack",
                    help="comma-separated legs to run (the headline needs decode)")
    ap.add_argument("--cpu-one-core-seconds", type=float, default=5.0,
                    help="wall time budget of the one-core CPU-oracle sample")
    return ap.parse_args()


COPY_BYTES = 256 << 20
READ_REF_BYTES = 2 << 30
CSRC = os.path.join(ROOT, "bit_gemm_ternary_amd", "csrc")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode1_kernel.decode_M1.hbm_traffic.md")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("gemv.hip", "common.hpp", "xreduce.hpp")]
GEMM_SUMMARY = os.path.join(ROOT, "profiles", "gemm_kernel.prefill_M2048_K4096_N14336.counters.md")
GEMM_SOURCES = [os.path.join(CSRC, f) for f in ("gemm_mfma.hip", "common.hpp")]


def kernel_source_digest(paths=None) -> str:
    import hashlib

    h = hashlib.sha256()
    for path in paths or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def summary_data(path, sources):
    """The bench-data line of a committed counter summary, or None if there is
    none or the kernel source has changed since the counters were taken."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("bench-data: "):
                    data = json.loads(line[len("bench-data: "):])
                    break
            else:
                return None
    except OSError:
        return None
    if data.get("source_sha256") != kernel_source_digest(sources):
        return None
    return data


def measured_traffic():
    """HBM bytes per step of the fused decode kernels (committed counter summary)."""
    return summary_data(TRAFFIC_SUMMARY, KERNEL_SOURCES)


def hbm_read_reference(torch, bt):
    """GB/s of a plain read of READ_REF_BYTES (2 GiB) of device memory
    (bitnet_stream_read: every byte once, 16-byte loads over the whole chip):
    the median of five reads after three untimed ones."""
    buf = torch.ones(READ_REF_BYTES // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        bt.stream_read(buf, sink)
    ms = []
    for _ in range(5):
        ms.append(time_region(lambda: bt.stream_read(buf, sink), 1, torch)[0])
    gbs = READ_REF_BYTES / (float(np.median(ms)) * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return round(gbs, 1)


def hbm_copy_reference(torch):
    """GB/s of a plain 1 GiB device copy (torch copy_, read + write bytes counted)."""
    src = torch.ones(READ_REF_BYTES // 8, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    n = 10
    ms, _ = time_region(lambda: [dst.copy_(src) for _ in range(n)], n, torch)
    gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def copy_calibration(torch):
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 10}), flush=True)


FLUSH_BYTES = 1 << 30        # device-copy traffic that evicts the Infinity Cache and the L2s


class CacheFlush:
    """One plain read (bitnet_stream_read) of a 1 GiB buffer no step touches.
    Enqueued just before a timed region it evicts the 256 MB Infinity Cache and
    every XCD's L2 without leaving dirty lines behind, and it keeps the GPU busy
    while the host submits the graph that follows, so the region's first event
    is not stamped ahead of that submission."""

    def __init__(self, torch, dev, nbytes=FLUSH_BYTES):
        import bit_gemm_ternary_amd as bt

        self.bt = bt
        self.buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
        self.sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def __call__(self):
        self.bt.stream_read(self.buf, self.sink)


def capture_steps(step, n, copies, torch):
    """One HIP graph of n steps, step s on rotation copy s % copies."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for s in range(n):
                step(s % copies)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def time_region(launch, n, torch, prelude=None):
    """(ms per step, wall seconds) of launch(), which enqueues n steps, timed by
    two events on the current stream between two synchronisations.  prelude()
    (a cache flush, or an untimed replay of the same graph) is enqueued after the
    first synchronisation and before the start event: the GPU runs it while the
    host submits the timed work, and the start event is stamped once it ends."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if prelude is not None:
        prelude()
    start.record()
    launch()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n, time.perf_counter() - t0


def b2b_us(fn, n, copies, torch, dev, eager=False):
    """Average duration (us) of fn(r), r = 0, 1, ... on rotation copy r % copies,
    launched n times back to back in one HIP graph after a cache flush; median
    of three such regions (each region also carries the graph launch's fixed
    cost, 12-19 us, spread over the n launches)."""
    t = StepTimer(fn, n, copies, torch, cache_flush(torch, dev), eager=eager)
    us = t.median_ms(3) * 1e3
    t.close()
    return us


class StepTimer:
    """Times exactly n steps (step s on rotation copy s % copies) as ONE graph
    launch: the steps are captured once into a single HIP graph, which is
    replayed once untimed (its first replay uploads it), and every timed region
    is one replay of it after a cache flush.  eager: the steps are launched one
    by one instead (no graph), after the same flush."""

    def __init__(self, step, n, copies, torch, flush, eager=False):
        self.step, self.n, self.copies, self.torch, self.flush = step, n, copies, torch, flush
        self.graph = None
        if not eager:
            self.graph = capture_steps(step, n, copies, torch)
            self.graph.replay()
            torch.cuda.synchronize()

    def launch(self):
        if self.graph is not None:
            self.graph.replay()
        else:
            for s in range(self.n):
                self.step(s % self.copies)

    def time(self):
        """(ms per step, wall seconds) of one timed region over the n steps, cold caches."""
        return time_region(self.launch, self.n, self.torch, self.flush)

    def time_warm(self):
        """ms per step with warm caches: the region follows an untimed run of the
        same steps instead of a flush."""
        return time_region(self.launch, self.n, self.torch, self.launch)[0]

    def median_ms(self, regions=5):
        """Median over `regions` cold timed regions of the ms per step."""
        return float(np.median([self.time()[0] for _ in range(regions)]))

    def close(self):
        self.graph = None


_FLUSH = None


def cache_flush(torch, dev):
    """The process's CacheFlush (allocated once)."""
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = CacheFlush(torch, dev)
    return _FLUSH


def per_launch_count(steps):
    """Launches per timed region of the back-to-back per-launch figures."""
    return max(200, min(3 * steps, 3000))


def timed(run, steps, torch):
    """(ms per call, wall seconds) of run(steps), an eager loop of library calls,
    between two synchronisations (legs whose single calls take tens of us or more)."""
    return time_region(lambda: run(steps), steps, torch)


class HipEvents:
    """hipEvent_t handles from the process's HIP runtime (the one torch and the library share)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self) -> int:
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.events.append(ev.value)
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ctypes.c_void_p(ev))
        self.events = []


class DecodeLayer:
    """Device buffers of one M=1 projection with R rotating copies of its packed weights."""

    def __init__(self, layer, copies, dev, bt, torch, packed=None):
        self.layer = layer
        M, K, N = layer.M, layer.K, layer.N
        if packed is None:
            packed = packed_copies(layer, copies, dev, bt, torch)
        self.packed, self.w_scale = packed
        x = layer.activations()
        self.x = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.codes = (torch.empty((M, K), dtype=torch.int8, device=dev),
                      torch.empty(M, dtype=torch.float32, device=dev),
                      torch.empty(M, dtype=torch.int32, device=dev))
        self.y = torch.empty((M, N), dtype=torch.float32, device=dev)
        self.weight_bytes = N * K // 4
        # Fused kernel algorithmic bytes: packed weights + bf16 token + w_scale in;
        # codes, scale, sum and float32 outputs out.
        self.kernel_bytes = self.weight_bytes + 2 * M * K + 8 + M * K + 8 * M + 4 * M * N

    def forward(self, bt, r):
        bt.bitlinear_forward(self.x, self.packed[r], self.w_scale, None, 1e-5, out=self.y,
                             codes=self.codes)


def packed_copies(layer, copies, dev, bt, torch):
    """(copies of the layer's packed weights, w_scale)."""
    W = torch.from_numpy(layer.weights()).to(dev)
    packed, w_scale = bt.pack_weights(W)
    del W
    return [packed] + [packed.clone() for _ in range(copies - 1)], w_scale


def decode_bench(args, dev, bt, torch, synth):
    layers_spec = synth.workload("decode")
    step_bytes = sum(l.N * l.K // 4 for l in layers_spec)
    copies = max(1, math.ceil(ROTATE_BYTES / step_bytes))
    layers = [DecodeLayer(l, copies, dev, bt, torch) for l in layers_spec]
    torch.cuda.synchronize()
    log(f"decode: {len(layers)} projections, {step_bytes / 1e6:.2f} MB packed per step, "
        f"{copies} rotating copies ({copies * step_bytes / 2**30:.2f} GiB)")

    def step(r):
        for L in layers:
            L.forward(bt, r)

    # Warm-up (also loads the kernels).
    for s in range(args.warmup):
        step(s % copies)
    torch.cuda.synchronize()

    # The timed region: exactly args.steps steps, one replay of one graph that
    # holds them all, after a cache flush (every step streams its weights from
    # HBM: consecutive steps use distinct copies, and a copy comes back only
    # after the other 40, over 1 GiB later).
    flush = cache_flush(torch, dev)
    timer = StepTimer(step, args.steps, copies, torch, flush, eager=args.eager)
    ms_per_step, wall_s = timer.time()
    timer.close()
    # Warm reference: the same steps on one weight copy, which then stays
    # resident in the 256 MB Infinity Cache (and partly in L2).
    warm = StepTimer(lambda r: step(0), min(args.steps, 500), 1, torch, flush, eager=args.eager)
    warm_ms = warm.time_warm()
    warm.close()

    # Per-kernel durations: the same steps again, launched eagerly with the
    # kernel-timing hook armed before every launch, so each event pair is
    # stamped by that kernel's own dispatch on the stream it runs on.
    hev = HipEvents()
    n_instr = min(args.steps, 1000)
    pairs = [[(hev.create(), hev.create()) for _ in layers] for _ in range(n_instr)]
    torch.cuda.synchronize()
    for s in range(n_instr):
        r = s % copies
        for i, L in enumerate(layers):
            bt.set_kernel_events(*pairs[s][i])
            L.forward(bt, r)
    torch.cuda.synchronize()
    isolated_us = [float(np.median([hev.elapsed_ms(*pairs[s][i]) for s in range(n_instr)])) * 1e3
                   for i in range(len(layers))]
    hev.close()

    # Average launch duration in a stream of launches: each projection alone,
    # back to back in one HIP graph over its own rotation of >= 1 GiB of weight
    # copies, between two HIP events on the stream the graph runs on; the
    # median over five such regions, each after a cache flush.  (The eager,
    # kernel-stamped durations above also count each launch's ramp-up on an
    # idle GPU.)
    per_layer_us = []
    launches = per_launch_count(args.steps)
    for L in layers:
        extra = max(0, math.ceil(ROTATE_BYTES / L.weight_bytes) - len(L.packed))
        own = L.packed + [L.packed[0].clone() for _ in range(extra)]

        def one(r, L=L, own=own):
            bt.bitlinear_forward(L.x, own[r], L.w_scale, None, 1e-5, out=L.y, codes=L.codes)

        t = StepTimer(one, launches, len(own), torch, flush, eager=args.eager)
        per_layer_us.append(t.median_ms() * 1e3)
        t.close()
        del t, own, one
        torch.cuda.empty_cache()
    kernel_bytes = sum(L.kernel_bytes for L in layers)
    kernel_us = sum(per_layer_us)
    per_layer = [{"K": L.layer.K, "N": L.layer.N, "packed_bytes": L.weight_bytes,
                  "kernel_bytes": L.kernel_bytes, "avg_us": round(us, 3),
                  "GB_s": round(L.kernel_bytes / us / 1e3, 1),
                  "isolated_us": round(iso, 3)}
                 for L, us, iso in zip(layers, per_layer_us, isolated_us)]
    return {
        "step_bytes": step_bytes, "copies": copies, "ms_per_step": ms_per_step,
        "wall_s": wall_s, "value": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "kernel_bytes": kernel_bytes, "kernel_us": kernel_us, "per_layer": per_layer,
        "instrumented_steps": n_instr, "layers": layers,
        "warm_value": step_bytes / (warm_ms * 1e-3) / 1e9,
    }


# (K, N) of the larger decode projections: Llama-70B-sized o / gate|up / down
# and a 405B-sized gate|up.
DECODE_SIZES = [(8192, 8192), (8192, 28672), (28672, 8192), (16384, 53248)]


def decode_sizes_bench(args, dev, bt, torch, synth):
    """The fused decode kernel (M = 1) on larger projections: average launch
    duration back to back from HIP graphs over >= 1 GiB of rotating weight
    copies, as for the headline's per-launch figures.  Seeded N(0, 0.02)
    weights and N(0, 1) tokens drawn on the device."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(5151)
    rows = []
    for K, N in DECODE_SIZES:
        W = torch.randn((N, K), generator=gen, device=dev) * 0.02
        packed, w_scale = bt.pack_weights(W)
        del W
        nbytes = N * K // 4
        copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
        own = [packed] + [packed.clone() for _ in range(copies - 1)]
        x = torch.randn((1, K), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        codes = (torch.empty((1, K), dtype=torch.int8, device=dev),
                 torch.empty(1, dtype=torch.float32, device=dev),
                 torch.empty(1, dtype=torch.int32, device=dev))

        def one(r, own=own, x=x, y=y, codes=codes, w_scale=w_scale):
            bt.bitlinear_forward(x, own[r], w_scale, None, 1e-5, out=y, codes=codes)

        for r in range(copies):
            one(r)
        torch.cuda.synchronize()
        t = StepTimer(one, per_launch_count(args.steps), copies, torch, cache_flush(torch, dev),
                      eager=args.eager)
        us = t.median_ms() * 1e3
        t.close()
        kernel_bytes = nbytes + 2 * K + 8 + K + 8 + 4 * N
        rows.append({"K": K, "N": N, "packed_MB": round(nbytes / 1e6, 1), "copies": copies,
                     "avg_us": round(us, 2), "GB_s": round(kernel_bytes / us / 1e3, 1),
                     "frac_hbm": round(kernel_bytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        del t, own, packed, x, y, codes, one
        torch.cuda.empty_cache()
    return {"what": "fused decode kernel, M = 1, larger projections (context for the headline, "
                    "which runs the 7B shapes)", "by_shape": rows}


def base3_bench(args, dev, bt, torch, synth):
    """Base-3 packing (five weights per byte) against the 2-bit packing on the
    same one-token contraction (codes precomputed, no fused quantisation in
    either): per-launch time back to back over >= 1 GiB of rotating copies."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(6161)
    rows = []
    for K, N in [(4096, 4096), (4096, 11008), (11008, 4096), (8192, 28672), (16384, 53248)]:
        W = torch.randn((N, K), generator=gen, device=dev) * 0.02
        packed, w_scale = bt.pack_weights(W)
        del W
        p3 = bt.pack_base3(packed, K)
        x = torch.randn((1, K), generator=gen, device=dev).to(torch.bfloat16)
        q, dx, qs = bt.quant_act(x)
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        row = {"K": K, "N": N}
        for name, base, fwd in (
                ("two_bit", packed, lambda w: bt.linear_forward(q, dx, qs, w, w_scale, out=y)),
                ("base3", p3, lambda w: bt.linear_forward_base3(q, dx, qs, w, w_scale, out=y))):
            nbytes = base.numel()
            copies = max(2, math.ceil(ROTATE_BYTES / nbytes))
            own = [base] + [base.clone() for _ in range(copies - 1)]

            def one(r, own=own, fwd=fwd):
                fwd(own[r])

            for r in range(copies):
                one(r)
            torch.cuda.synchronize()
            t = StepTimer(one, per_launch_count(args.steps), copies, torch, cache_flush(torch, dev),
                          eager=args.eager)
            us = t.median_ms() * 1e3
            t.close()
            row[name] = {"packed_MB": round(nbytes / 1e6, 2), "avg_us": round(us, 2),
                         "GB_s": round(nbytes / us / 1e3, 1), "Gweights_s": round(N * K / us / 1e3, 1)}
            del t, own, one
            torch.cuda.empty_cache()
        row["base3_speedup"] = round(row["two_bit"]["avg_us"] / row["base3"]["avg_us"], 3)
        rows.append(row)
        del packed, p3, x, q, dx, qs, y
        torch.cuda.empty_cache()
    return {"what": "one-token contraction, codes precomputed: 2-bit packing (bitnet_linear_forward) "
                    "against base-3 packing (bitnet_linear_forward_base3), 1.6 instead of 2 bits per weight",
            "by_shape": rows}


def time_launches(fn, iters, bt):
    """Median kernel duration (us) of fn() over `iters` launches, from event pairs
    stamped by each launch's own dispatch (the library's kernel-timing hook)."""
    import torch

    hev = HipEvents()
    pairs = [(hev.create(), hev.create()) for _ in range(iters)]
    for a, b in pairs:
        bt.set_kernel_events(a, b)
        fn()
    torch.cuda.synchronize()
    us = float(np.median([hev.elapsed_ms(a, b) for a, b in pairs])) * 1e3
    hev.close()
    return us


def prefill_bench(args, dev, bt, torch, synth):
    layer = synth.workload("prefill")[0]
    M, K, N = layer.M, layer.K, layer.N
    packed, w_scale = bt.pack_weights(torch.from_numpy(layer.weights()).to(dev))
    x = torch.from_numpy(layer.activations().view(np.int16)).to(dev).view(torch.bfloat16)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    qs = torch.empty(M, dtype=torch.int32, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    quant = lambda: bt.quant_act(x, None, 1e-5, out=(xq, xs, qs))
    gemm = lambda: bt.linear_forward(xq, xs, qs, packed, w_scale, out=y)
    for _ in range(5):
        quant()
        gemm()
    torch.cuda.synchronize()
    quant_us = time_launches(quant, args.prefill_iters, bt)
    gemm_us = time_launches(gemm, args.prefill_iters, bt)
    tops = 2.0 * M * N * K / (gemm_us * 1e-6) / 1e12
    # Context only: the vendor int8 GEMM (hipBLASLt, through torch._int_mm) on
    # the same shape with the weights stored unpacked, one int8 code each
    # (ternary values drawn at random), int32 output and no dequantisation.
    lib_us = None
    try:
        gen = torch.Generator(device="cpu").manual_seed(11)
        wq = torch.randint(-1, 2, (N, K), generator=gen, dtype=torch.int8).to(dev)
        ref = lambda: torch._int_mm(xq, wq.t())
        for _ in range(3):
            ref()
        lib_ms, _ = timed(lambda n: [ref() for _ in range(n)], args.prefill_iters, torch)
        lib_us = lib_ms * 1e3
        del wq
    except (RuntimeError, AttributeError) as ex:  # not every torch build exposes it
        log(f"prefill: no library int8 GEMM reference ({ex})")
    quant_bytes = M * K * 2 + M * K + 8 * M
    counters = summary_data(GEMM_SUMMARY, GEMM_SOURCES)
    # Engine clock of this run: the kernel's cycles per CU (counter summary)
    # over its measured duration.
    clock = None if counters is None else round(counters["cu_cycles_per_launch"] / (gemm_us * 1e3), 3)
    return {
        "workload": f"W1.58A8 prefill M={M} K={K} N={N} (FFN up)",
        "gemm_us": round(gemm_us, 2), "TOPS": round(tops, 1),
        "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": round(tops / INT8_PEAK_TOPS, 4),
                     "traffic": None if counters is None else counters["hbm_bytes_per_launch"],
                     "clock_ghz_measured": clock,
                     "frac_at_measured_clock": None if clock is None else
                     round(tops / (INT8_PEAK_TOPS * clock / PEAK_CLOCK_GHZ), 4)},
        "quant_us": round(quant_us, 2), "quant_GB_s": round(quant_bytes / quant_us / 1e3, 1),
        "step_ms": round((gemm_us + quant_us) / 1e3, 4),
        "library_int8_gemm_reference": None if lib_us is None else {
            "what": "hipBLASLt int8 GEMM via torch._int_mm, unpacked int8 ternary weights, "
                    "int32 output, no dequantisation (context, not this path)",
            "us": round(lib_us, 2), "TOPS": round(2.0 * M * N * K / (lib_us * 1e-6) / 1e12, 1)},
    }


def hadamard_bench(args, dev, bt, torch, synth):
    out = []
    for layer in synth.workload("hadamard"):
        M, K, N = layer.M, layer.K, layer.N
        packed, w_scale = bt.pack_weights(torch.from_numpy(layer.weights()).to(dev), hadamard=True)
        x = torch.from_numpy(layer.activations().view(np.int16)).to(dev).view(torch.bfloat16)
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        xs = torch.empty(M, dtype=torch.float32, device=dev)
        qs = torch.empty(M, dtype=torch.int32, device=dev)
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        xq6 = torch.empty((M, K // 4 * 3), dtype=torch.uint8, device=dev)
        xq4 = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        hq = lambda: bt.hadamard_quant_act(x, None, 1e-5, out=(xq, xs, qs))
        gemm = lambda: bt.linear_forward(xq, xs, qs, packed, w_scale, out=y)
        hq6 = lambda: bt.hadamard_quant_act_f6(x, None, 1e-5, out=(xq6, xs, qs))
        gemm6 = lambda: bt.linear_forward_f6(xq6, xs, qs, packed, w_scale, out=y)
        hq4 = lambda: bt.hadamard_quant_act_i4(x, None, 1e-5, out=(xq4, xs, qs))
        gemm4 = lambda: bt.linear_forward_i4(xq4, xs, qs, packed, w_scale, out=y)
        # one token of the same layer: the GEMVs on int8 and on packed 4-bit codes
        y1 = torch.empty((1, N), dtype=torch.float32, device=dev)
        gemv = lambda: bt.linear_forward(xq[:1], xs[:1], qs[:1], packed, w_scale, out=y1)
        gemv4 = lambda: bt.linear_forward_i4(xq4[:1], xs[:1], qs[:1], packed, w_scale, out=y1)
        # one token through the whole layer: the quantisation kernel then the
        # GEMV, against the single fused launch, back to back over rotating
        # weight copies
        rot = [packed] + [packed.clone() for _ in range(max(0, math.ceil(ROTATE_BYTES / (N * K // 4)) - 1))]
        c1 = (xq4[:1], xs[:1], qs[:1])

        def layer_two(r):
            bt.hadamard_quant_act_i4(x[:1], None, 1e-5, out=c1)
            bt.linear_forward_i4(*c1, rot[r], w_scale, out=y1)

        def layer_fused(r):
            bt.hadamard_bitlinear_forward(x[:1], rot[r], w_scale, codes=c1, out=y1)
        for _ in range(5):
            hq()
            gemm()
            hq6()
            gemm6()
            hq4()
            gemm4()
            gemv()
            gemv4()
            layer_two(0)
            layer_fused(0)
        torch.cuda.synchronize()
        hq_us = time_launches(hq, args.prefill_iters, bt)
        gemm_us = time_launches(gemm, args.prefill_iters, bt)
        hq6_us = time_launches(hq6, args.prefill_iters, bt)
        gemm6_us = time_launches(gemm6, args.prefill_iters, bt)
        hq4_us = time_launches(hq4, args.prefill_iters, bt)
        gemm4_us = time_launches(gemm4, args.prefill_iters, bt)
        gemv_us = time_launches(gemv, args.prefill_iters, bt)
        gemv4_us = time_launches(gemv4, args.prefill_iters, bt)
        two_us = b2b_us(layer_two, 400, len(rot), torch, dev, eager=args.eager)
        fused_us = b2b_us(layer_fused, 400, len(rot), torch, dev, eager=args.eager)
        del rot
        hq_bytes = M * K * 2 + M * K + 8 * M
        hq6_bytes = M * K * 2 + M * K // 4 * 3 + 8 * M
        hq4_bytes = M * K * 2 + M * K // 2 + 8 * M
        gemv_bytes = N * K // 4 + K + 4 * N
        ops = 2.0 * M * N * K
        out.append({"M": M, "K": K, "N": N,
                    "fwht_int4_us": round(hq_us, 2),
                    "fwht_int4_GB_s": round(hq_bytes / hq_us / 1e3, 1),
                    "fwht_int4_frac_hbm": round(hq_bytes / hq_us / 1e3 / HBM_PEAK_GBS, 4),
                    "gemm_us": round(gemm_us, 2),
                    "gemm_TOPS": round(ops / (gemm_us * 1e-6) / 1e12, 1),
                    "f6": {"fwht_e3m2_us": round(hq6_us, 2),
                           "fwht_e3m2_GB_s": round(hq6_bytes / hq6_us / 1e3, 1),
                           "gemm_fp4xfp6_us": round(gemm6_us, 2),
                           "gemm_fp4xfp6_TOPS": round(ops / (gemm6_us * 1e-6) / 1e12, 1),
                           "gemm_fp4xfp6_frac_fp6_peak": round(ops / (gemm6_us * 1e-6) / 1e12 / FP6_PEAK_TOPS, 4)},
                    "i4": {"fwht_nibble_us": round(hq4_us, 2),
                           "fwht_nibble_GB_s": round(hq4_bytes / hq4_us / 1e3, 1),
                           "fwht_nibble_frac_hbm": round(hq4_bytes / hq4_us / 1e3 / HBM_PEAK_GBS, 4),
                           "gemm_nibble_us": round(gemm4_us, 2),
                           "gemm_nibble_TOPS": round(ops / (gemm4_us * 1e-6) / 1e12, 1),
                           "gemv_m1_int8_us": round(gemv_us, 2),
                           "gemv_m1_nibble_us": round(gemv4_us, 2),
                           "gemv_m1_nibble_GB_s": round((gemv_bytes - K // 2) / gemv4_us / 1e3, 1),
                           "layer_m1_two_kernels_us": round(two_us, 2),
                           "layer_m1_fused_us": round(fused_us, 2),
                           "layer_m1_fused_GB_s": round((N * K // 4 + 2 * K + K // 2 + 4 * N) / fused_us / 1e3, 1),
                           "layer_m1_timing": "per layer, back to back in one graph over >= 1 GiB of weight "
                                              "copies"}})
    return out


def backward_bench(args, dev, bt, torch, synth):
    """STE backward of the prefill layer (M 2048 tokens, K 4096 -> N 14336)."""
    layer = synth.workload("prefill")[0]
    M, K, N = layer.M, layer.K, layer.N
    packed, w_scale = bt.pack_weights(torch.from_numpy(layer.weights()).to(dev))
    packed_t = bt.transpose_packed(packed, K)
    x = torch.from_numpy(layer.activations().view(np.int16)).to(dev).view(torch.bfloat16)
    xq, xs, _ = bt.quant_act(x, None, 1e-5)
    rng = np.random.default_rng(7001)
    gy = torch.from_numpy(synth.bf16_bits(rng.standard_normal((M, N)).astype(np.float32) * 1e-2)
                          .view(np.int16)).to(dev).view(torch.bfloat16)
    gn = torch.empty((M, K), dtype=torch.float32, device=dev)
    gw = torch.empty((N, K), dtype=torch.float32, device=dev)
    ws = torch.empty(bt.lib().bitnet_linear_backward_weight_workspace_bytes(M, N, K), dtype=torch.uint8,
                     device=dev)
    pt = torch.empty_like(packed_t)
    tr = lambda: bt.transpose_packed(packed, K, out=pt)
    bin_ = lambda: bt.linear_backward_input(gy, packed_t, w_scale, out=gn)
    bw = lambda: bt.linear_backward_weight(gy, xq, xs, out=gw, workspace=ws)
    rb = lambda: bt.rmsnorm_backward(x, gn, None, 1e-5)
    for _ in range(3):
        tr(); bin_(); bw(); rb()
    torch.cuda.synchronize()
    iters = max(5, args.prefill_iters // 2)
    tr_us = time_launches(tr, iters, bt)
    in_us = time_launches(bin_, iters, bt)
    rb_us = time_launches(rb, iters, bt)
    w_ms, _ = timed(lambda n: [bw() for _ in range(n)], iters, torch)  # three kernels per call
    flops = 2.0 * M * N * K
    w_us = w_ms * 1e3
    rb_bytes = M * K * (2 + 4 + 4) + 8 * M
    # Context only: the vendor bf16 GEMM (hipBLASLt through torch.matmul) on the
    # two contraction shapes, with the ternary weights and the activation codes
    # stored unpacked as bf16 and one bf16 pass for dL/dW.
    lib = None
    try:
        gen = torch.Generator(device="cpu").manual_seed(13)
        wb = torch.randint(-1, 2, (N, K), generator=gen).to(torch.bfloat16).to(dev)
        xb = xq.to(torch.bfloat16)
        gyt = gy.t().contiguous()
        ref_n = lambda: torch.matmul(gy, wb)
        ref_w = lambda: torch.matmul(gyt, xb)
        for _ in range(2):
            ref_n(); ref_w()
        n_ms, _ = timed(lambda n: [ref_n() for _ in range(n)], iters, torch)
        w2_ms, _ = timed(lambda n: [ref_w() for _ in range(n)], iters, torch)
        lib = {"what": "hipBLASLt bf16 GEMM via torch.matmul, unpacked bf16 operands, one bf16 pass "
                       "(context, not this path)",
               "grad_n_us": round(n_ms * 1e3, 2), "grad_w_us": round(w2_ms * 1e3, 2)}
        del wb, xb, gyt
    except RuntimeError as ex:
        log(f"backward: no library bf16 GEMM reference ({ex})")
    return {
        "workload": f"STE backward of the prefill layer: grad_y bf16 [{M}][{N}], ternary W [{N}][{K}], "
                    "int8 codes of x; grad_n, grad_w, RMSNorm backward",
        "grad_n_us": round(in_us, 2),
        "grad_n_TFLOPs": round(flops / (in_us * 1e-6) / 1e12, 1),
        "grad_n_frac_bf16_peak": round(flops / (in_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "grad_w_us": round(w_us, 2),
        "grad_w_TFLOPs": round(flops / (w_us * 1e-6) / 1e12, 1),
        "grad_w_note": "three kernels per call (operand transposes + GEMM); the GEMM runs the hi and "
                       "lo halves, 2x the algorithmic 2 M N K flops counted here",
        "rmsnorm_bwd_us": round(rb_us, 2),
        "rmsnorm_bwd_GB_s": round(rb_bytes / rb_us / 1e3, 1),
        "transpose_packed_us": round(tr_us, 2),
        "library_bf16_gemm_reference": lib,
    }


def blend_bench(args, dev, bt, torch, synth):
    """The warm-up blend (lambda = 0.5) of the prefill layer (M 2048, K 4096,
    N 14336): quantisation, blended activations and the float32 contraction
    with the weights blended in its stage loads, one call."""
    layer = synth.workload("prefill")[0]
    M, K, N = layer.M, layer.K, layer.N
    W = torch.from_numpy(layer.weights()).to(dev)
    packed, w_scale = bt.pack_weights(W)
    x = torch.from_numpy(layer.activations().view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(bt.lib().bitnet_linear_forward_blend_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    call = lambda: bt.linear_forward_blend(x, W, packed, w_scale, 0.5, out=y, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ms, _ = timed(lambda n: [call() for _ in range(n)], max(3, args.prefill_iters // 3), torch)
    flops = 2.0 * M * N * K
    tf = flops / (ms * 1e-3) / 1e12
    del W, packed, x, y, ws
    return {"workload": f"warm-up blend lambda=0.5, M={M} K={K} N={N}", "us": round(ms * 1e3, 1),
            "TFLOPs": round(tf, 1), "frac_fp32_peak": round(tf / FP32_PEAK_TFLOPS, 4)}


def pack_bench(args, dev, bt, torch, synth):
    """Offline weight preparation (absmean scale, ternarise, pack; and the
    Hadamard pre-rotation) of the prefill and H-BitLinear weight matrices."""
    out = []
    cases = [(synth.workload("prefill")[0], False), (synth.workload("hadamard")[1], True)]
    for layer, had in cases:
        N, K = layer.N, layer.K
        W = torch.from_numpy(layer.weights()).to(dev)
        packed = torch.empty((N, K // 4), dtype=torch.uint8, device=dev)
        w_scale = torch.empty(2, dtype=torch.float32, device=dev)
        ws = torch.empty(max(bt.pack_weights_workspace_bytes(N, K, had), 16), dtype=torch.uint8,
                         device=dev)
        call = lambda: bt.pack_weights(W, had, out=(packed, w_scale), workspace=ws)
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        ms, _ = timed(lambda n: [call() for _ in range(n)], args.pack_iters, torch)
        # The scale needs every weight before the first code: two passes over W
        # (plus, with the rotation, one write and two reads of the rotated copy).
        passes = 2 if not had else 4
        bytes_ = passes * 4 * N * K + N * K // 4
        out.append({"N": N, "K": K, "hadamard": had, "us": round(ms * 1e3, 1),
                    "algorithmic_bytes": bytes_,
                    "GB_s": round(bytes_ / (ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(bytes_ / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        del W, ws
    return out


class GroupedLayer:
    """Projections sharing one input (q|k|v or gate|up) stacked row-wise, run
    with one bitnet_bitlinear_forward_grouped call per step."""

    def __init__(self, members, copies, dev, torch):
        # members: [(DecodeLayer, ...)] sharing the first member's input
        first = members[0]
        self.x = first.x
        self.codes = first.codes
        self.rows = [m.layer.N for m in members]
        self.packed = [torch.cat([m.packed[r] for m in members]) for r in range(copies)]
        self.w_scales = torch.stack([m.w_scale for m in members])
        M = first.layer.M
        self.y = torch.empty((M, sum(self.rows)), dtype=torch.float32, device=dev)

    def forward(self, bt, r):
        bt.bitlinear_forward_grouped(self.x, self.packed[r], self.w_scales, self.rows, None, 1e-5,
                                     out=self.y, codes=self.codes)


def block_bench(args, dev, bt, torch, synth):
    """The seven projections of a Llama-3-8B block, each RMSNorm + quantisation +
    contraction + dequantisation, at M = 1, 16 and 256 tokens; weights rotate
    over > 1 GiB of copies as in the decode leg.  Timed twice: seven separate
    bitnet_bitlinear_forward calls, and four calls with q|k|v and gate|up
    grouped (bitnet_bitlinear_forward_grouped: one quantisation and one launch
    per shared input)."""
    spec = synth.workload("block", M=1)
    block_bytes = sum(l.N * l.K // 4 for l in spec)
    copies = max(1, math.ceil(ROTATE_BYTES / block_bytes))
    packed = [packed_copies(l, copies, dev, bt, torch) for l in spec]
    names = [l.name for l in spec]
    out = []
    for M in (1, 16, 256):
        layers = [DecodeLayer(l, copies, dev, bt, torch, packed=p)
                  for l, p in zip(synth.workload("block", M=M), packed)]
        by = dict(zip(names, layers))
        grouped = [GroupedLayer([by["q"], by["k"], by["v"]], copies, dev, torch), by["o"],
                   GroupedLayer([by["gate"], by["up"]], copies, dev, torch), by["down"]]
        ops = 2.0 * M * sum(l.N * l.K for l in spec)
        row = {"M": M}
        for label, units in (("separate", layers), ("grouped", grouped)):
            def step(r, units=units):
                for U in units:
                    U.forward(bt, r)

            for s in range(min(args.warmup, 2 * copies)):
                step(s % copies)
            torch.cuda.synchronize()
            t = StepTimer(step, args.block_steps, copies, torch, cache_flush(torch, dev),
                          eager=args.eager)
            ms = t.median_ms(3)
            t.close()
            del t
            row[label] = {"launch_units": len(units), "us_per_block": round(ms * 1e3, 2),
                          "packed_GB_s": round(block_bytes / (ms * 1e-3) / 1e9, 1),
                          "TOPS": round(ops / (ms * 1e-3) / 1e12, 2)}
        out.append(row)
        del layers, grouped, by
        torch.cuda.empty_cache()
    return {"workload": "Llama-3-8B block: q 4096x4096, k/v 4096x1024, o 4096x4096, gate/up "
                        "4096x14336, down 14336x4096; bf16 N(0,1) tokens, RMSNorm + int8 quant "
                        "before each projection (grouped: q|k|v and gate|up share one quantisation)",
            "packed_bytes_per_block": block_bytes, "weight_rotation_copies": copies,
            "by_tokens": out}


# Row-parallel projections of the eight-way split block: the whole token's K.
SHARD_K_TOTAL = {"o/8": 4096, "down/8": 14336}


def shard_bench(args, dev, bt, torch, synth):
    """One device's share of a Llama-3-8B block split eight ways, M = 1: q|k|v
    and gate|up by output features (the fused decode call on N / 8 rows), o and
    down by input features (a K / 8 slice: token statistics, quantisation with
    the whole token's statistics, the contraction to int32 partial sums, the
    dequantisation).  The collectives between those calls (a maximum and a sum
    of the statistics, a sum of the partials) are not run: one device's
    kernels only, on its own statistics.  Weights rotate over > 1 GiB of copies
    as in the decode leg."""
    spec = synth.workload("shard")
    share_bytes = sum(l.N * l.K // 4 for l in spec)
    copies = max(1, math.ceil(ROTATE_BYTES / share_bytes))
    layers = [DecodeLayer(l, copies, dev, bt, torch) for l in spec]
    for L in layers:
        if L.layer.name in SHARD_K_TOTAL:
            L.stats = (torch.empty(1, dtype=torch.float32, device=dev),
                       torch.empty(1, dtype=torch.float64, device=dev))
            L.acc = torch.empty((1, L.layer.N), dtype=torch.int32, device=dev)

    def stats(L):
        bt.token_stats(L.x, out=L.stats)

    def quant(L):
        bt.quant_act_with_stats(L.x, L.stats[0], L.stats[1], SHARD_K_TOTAL[L.layer.name], out=L.codes)

    def contract(L, r):
        bt.linear_forward(*L.codes, L.packed[r], L.w_scale, out=L.y, acc_out=L.acc)

    def dequant(L):
        bt.dequant(L.acc, L.codes[1], L.w_scale, out=L.y)

    def step(r):
        for L in layers:
            if L.layer.name in SHARD_K_TOTAL:
                stats(L)
                quant(L)
                contract(L, r)
                dequant(L)
            else:
                L.forward(bt, r)

    for s in range(min(args.warmup, 2 * copies)):
        step(s % copies)
    torch.cuda.synchronize()
    t = StepTimer(step, args.block_steps, copies, torch, cache_flush(torch, dev), eager=args.eager)
    ms = t.median_ms(3)
    t.close()
    del t
    rows = []
    n = 400
    for L in layers:
        if L.layer.name in SHARD_K_TOTAL:
            us = {"token_stats": b2b_us(lambda r, L=L: stats(L), n, 1, torch, dev, args.eager),
                  "quant_act_with_stats": b2b_us(lambda r, L=L: quant(L), n, 1, torch, dev, args.eager),
                  "contraction": b2b_us(lambda r, L=L: contract(L, r), n, copies, torch, dev, args.eager),
                  "dequant": b2b_us(lambda r, L=L: dequant(L), n, 1, torch, dev, args.eager)}
            split = "input features (K slice)"
        else:
            us = {"fused_decode": b2b_us(lambda r, L=L: L.forward(bt, r), n, copies, torch, dev, args.eager)}
            split = "output features (N rows)"
        rows.append({"name": L.layer.name, "K": L.layer.K, "N": L.layer.N, "split_by": split,
                     "packed_bytes": L.weight_bytes, "kernel_us": {k: round(v, 2) for k, v in us.items()}})
    del layers
    torch.cuda.empty_cache()
    return {"workload": "one device's share of the Llama-3-8B block split eight ways, M = 1: q|k|v 4096->768 "
                        "and gate|up 4096->3584 by output features; o 512->4096 and down 1792->4096 by input "
                        "features (K slices of 4096 and 14336)",
            "per_device_packed_bytes": share_bytes, "weight_rotation_copies": copies,
            "us_per_block": round(ms * 1e3, 2), "packed_GB_s": round(share_bytes / (ms * 1e-3) / 1e9, 1),
            "collectives": "not run (between the calls of the K-sliced projections)",
            "kernel_us_note": "average per launch, 400 launches of one kernel back to back in one graph "
                              "(the contraction and fused decode over the rotating weight copies)",
            "layers": rows}


def cpu_baseline(args, synth):
    import oracle

    orc = oracle.default()
    layers = []
    for l in synth.workload("decode"):
        packed, d_w, _, _ = orc.pack_weights(l.weights())
        layers.append((l, packed, d_w, l.activations()))
    step_bytes = sum(l.N * l.K // 4 for l, *_ in layers)

    def step():
        for l, packed, d_w, x in layers:
            xq, d_x, _ = orc.quant_act(x)
            orc.linear_forward(xq, d_x, packed, d_w, l.K)

    step()
    n, t0 = 0, time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    all_cores = orc.num_threads()
    out = {"value": round(step_bytes * n / el / 1e9, 4), "unit": "GB/s", "cores": all_cores,
           "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n} decode steps (int8 quant + int32 contraction + dequant of the three "
                     f"M=1 projections) in {el:.1f} s on {os.cpu_count()} host CPUs"}
    # The same steps on one core.
    orc.set_num_threads(1)
    try:
        n1, t0 = 0, time.perf_counter()
        while True:
            step()
            n1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= args.cpu_one_core_seconds:
                break
    finally:
        orc.set_num_threads(all_cores)
    out["one_core"] = {"value": round(step_bytes * n1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                       "sample": f"{n1} decode steps in {el1:.1f} s"}
    return out


def main():
    args = parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this BitLinear build has no multi-GPU path "
              "(the workload would shard by tokens or output features; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_gemm_ternary_amd as bt
    from bit_gemm_ternary_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bt.lib()

    legs = set(args.legs.split(","))
    secondary = {}
    if "decode" not in legs:
        # Secondary legs only (used for per-kernel counter runs); no headline line.
        for name, fn in (("decode_sizes", decode_sizes_bench), ("base3", base3_bench),
                         ("prefill", prefill_bench), ("hadamard", hadamard_bench),
                         ("block", block_bench), ("shard", shard_bench), ("backward", backward_bench),
                         ("blend", blend_bench), ("pack", pack_bench)):
            if name in legs:
                secondary[name] = fn(args, dev, bt, torch, synth)
                torch.cuda.empty_cache()
        print(json.dumps(secondary), flush=True)
        return

    dec = decode_bench(args, dev, bt, torch, synth)
    log(f"decode: {dec['ms_per_step'] * 1e3:.2f} us/step, {dec['value']:.1f} GB/s; "
        f"GEMV kernels {dec['per_layer']}")
    del dec["layers"]
    torch.cuda.empty_cache()
    read_ref = hbm_read_reference(torch, bt)
    copy_ref = hbm_copy_reference(torch)

    if not args.no_secondary:
        for name, fn in (("decode_sizes", decode_sizes_bench), ("base3", base3_bench),
                         ("prefill", prefill_bench), ("hadamard", hadamard_bench),
                         ("block", block_bench), ("shard", shard_bench), ("backward", backward_bench),
                         ("blend", blend_bench), ("pack", pack_bench)):
            if name in legs:
                secondary[name] = fn(args, dev, bt, torch, synth)
                log(f"{name}: {secondary[name]}")
                torch.cuda.empty_cache()

    cpu = None if args.no_cpu_baseline else cpu_baseline(args, synth)

    achieved = dec["kernel_bytes"] / dec["kernel_us"] / 1e3
    traffic = measured_traffic()
    line = {
        "metric": METRIC,
        "value": round(dec["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "decode GEMV W1.58A8, M=1, (K,N) in (4096,4096), (4096,11008), (11008,4096); "
                        "bf16 N(0,1) tokens with 1% outlier channels x20; N(0,0.02) weights, absmean "
                        "ternary, 2 bits/weight",
            "step": "per projection: RMSNorm + int8 quant fused into the ternary GEMV + dequant "
                    "(3 kernels per step)",
            "packed_bytes_per_step": dec["step_bytes"],
            "weight_rotation_copies": dec["copies"],
            "launch": "eager" if args.eager else "one hip graph of the timed steps, one replay after a cache flush",
            "frac_hbm_peak": round(dec["value"] / HBM_PEAK_GBS, 4),
            "hbm_read_reference_GB_s": read_ref,
            "frac_of_read_reference": round(dec["value"] / read_ref, 4),
            "hbm_copy_reference_GB_s": copy_ref,
            "warm_value_GB_s": round(dec["warm_value"], 1),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "frac_of_read_reference": round(achieved / read_ref, 4),
            "traffic": None if traffic is None else traffic["hbm_bytes_per_step"],
            "traffic_per_launch": None if traffic is None else traffic["hbm_bytes_per_launch"],
            "kernel": "decode1_kernel, fused (3 launches per step)",
            "bytes_per_step": dec["kernel_bytes"],
            "us_per_step": round(dec["kernel_us"], 3),
            "per_launch": dec["per_layer"],
        },
        "cpu_baseline": cpu,
    }
    line.update(secondary)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
