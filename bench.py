"""Benchmark of the paged KV-cache data plane on one MI355X.

A step is one pass of the hot path over one batch of synthetic input:
  * headline (decode): Qwen3-8B-shaped single-layer decode, 64 sequences with context
    lengths uniform in [512, 4096], block_size 256: store the 64 new tokens' K/V through
    slot_mapping, then paged decode attention over the pool.  Inputs are already in HBM;
    three copies of the pool at different addresses are rotated so consecutive steps do
    not hit the 256 MB last-level cache with the previous step's K/V.
  * prefill legs (reported beside it): 8 x 2048-token causal varlen prefill (store all
    16384 tokens, then attend through the block tables) and the prefix-cached chunked
    prefill (16 sequences, shared 1024-token prefix, 512-token chunks).
  * long-context legs (reported beside it): decode layer by layer over all 36 layers'
    pools for 4 x 40960 (C5a) and 256 log-uniform lengths in [128, 32768] (C5b).

value = algorithmic bytes of the decode step (store + decode) / measured step time, the
step replayed from HIP graphs as a serving engine runs decode (a graph of three steps,
one per rotated pool copy, plus single-step graphs for the remainder, so exactly `steps`
steps are timed; ms_per_step is the event time per step).  eager_step gives the same
step launched call by call.
roofline = the decode call (stream-K kernel + its fixup kernel) timed with HIP events on
the stream it runs on: algorithmic decode bytes / average duration vs 8 TB/s.  The average
duration is that of `steps` decode calls launched back to back (over the same 3 rotated pool
copies) between one event pair; per_call_event_us keeps the mean of the per-call event pairs
of the eager steps, which add a few microseconds of event overhead to each ~100-us call.
traffic = HBM bytes per decode call measured by rocprofv3 counters (FETCH_SIZE and
WRITE_SIZE, calibrated on a plain copy of known size), read from
profiles/decode_c2_counters.json when it was taken on the current decode sources.
cpu_baseline = the float64 CPU oracle (store_ref + decode_ref) on the same C2 batch, with the
host's CPU model; each long-context leg carries its own cpu_baseline: decode_ref over the
full layer 0 (C5a: 4 sequences, C5b: all 256), per layer and x36 "extrapolated".
engine_clock = the GPU engine clock the driver reports (pp_dpm_sclk), sampled every 2 ms
while the decode graph steps are timed and while each prefill leg settles and is timed.
prefill[i].roofline = the leg's algorithmic TFLOP/s against the dense bf16 MFMA peak, with
MFMA busy, VALU-MFMA co-execution and the bytes read from beyond L2 (FETCH_SIZE, calibrated,
MALL hits included: an upper bound on HBM reads) from
profiles/prefill_c3_c4_counters.json when it was taken on the current prefill sources.
decode_call / prefill_call / store_call = mean, median and minimum of the per-call event times;
the prefill legs' headline times (the prefill and the store before it) are the median calls.
back_to_back_us is the mean of `steps` prefill calls launched back to back between one event
pair: longer than the per-call median, because the sustained MFMA load with no store between
two calls runs at a lower engine clock.  The store is also reported back to back
(store_batched_*).
Prefill legs are timed in steady state: after the warm-up calls, 10 calls are timed at once
(cold_prefill_call), the matrix cores are then kept busy for settle_s = 1.5 seconds (the
first sustained MFMA work of a process runs slower while the engine clock settles: the
first leg measured 370 us per C3 call after 0.25 s of it and 331 us after 1.5 s), and only
then are the `steps` reported calls timed.
peaks = the spec peaks beside CUs x max engine clock x 4096 flop/clock (bf16 MFMA) from the
device properties.
qk_norm_rope_store = the fused q/k RMSNorm + rotary + KV store over C3's 16384 prompt
tokens and C2's 64 decode tokens: algorithmic bytes / mean event time vs 8 TB/s.  The
short HBM legs (this one, add_rms_norm and the prefill legs' store) also report batched_*:
`steps` back-to-back calls between one event pair, per call.  An event pair around each
call adds a few microseconds of launch and event overhead, a large share of a 20-us
kernel; the batched figure keeps only the gaps between consecutive kernels.
add_rms_norm = the fused residual add + RMSNorm over the same token counts' 4096-wide
hidden rows (the norm in front of each block's projections), same figures.
block_manager = host wall time of the C++ block manager (through the binding): admitting
the long-context batch's 256 prompts and building one decode step's and one 8 x 2048
prefill's index arrays.
prefill also holds the varlen leg: C3's prompts through the prefill over contiguous K/V
(views of a packed qkv, the branch without a prefix cache), timed like the paged legs.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu] [--no-prefill] [--no-c5]
Prints ONE JSON line on stdout; progress goes to stderr.

Counter collection (two rocprofv3 passes, then a summary written to profiles/):
  rocprofv3 --pmc FETCH_SIZE -d DIR_F -o pass --output-format csv -- python bench.py --counter-pass
  rocprofv3 --pmc WRITE_SIZE -d DIR_W -o pass --output-format csv -- python bench.py --counter-pass
  python bench.py --summarize-counters DIR_F/pass_counter_collection.csv \
                                       DIR_W/pass_counter_collection.csv
--counter-pass runs a plain elementwise copy (torch.neg over COPY_BYTES of bf16: reads
and writes COPY_BYTES) three times, then the decode leg only.

Prefill counters (three rocprofv3 passes, groups in PREFILL_COUNTER_GROUPS, then a summary
written to profiles/prefill_c3_c4_counters.md):
  rocprofv3 --pmc <group i> -d DIR<i> -o pass --output-format csv -- python bench.py --prefill-counter-pass
  python bench.py --summarize-prefill-counters DIR0/... DIR1/... DIR2/pass_counter_collection.csv
--prefill-counter-pass runs the same calibration copy, then PREFILL_CALLS prefill calls of
C3 and of C4 (after storing their tokens).
"""

from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
COUNTERS = os.path.join(ROOT, "profiles", "decode_c2_counters.json")
PREFILL_COUNTERS = os.path.join(ROOT, "profiles", "prefill_c3_c4_counters.md")
PREFILL_COUNTERS_JSON = os.path.join(ROOT, "profiles", "prefill_c3_c4_counters.json")
SCLK_FILES = ("/sys/class/drm/card0/device/pp_dpm_sclk", "/sys/class/drm/card1/device/pp_dpm_sclk")
PREFILL_SOURCES = ["prefill.hip", "common.hpp", "launch.hpp"]
PREFILL_CALLS = 12              # prefill calls per leg in the prefill counter pass (2 warm-up)
COPY_BYTES = 1 << 30            # calibration copy: 1 GiB read + 1 GiB written per launch
DECODE_KERNELS = ("decode_streamk_kernel", "decode_fixup_kernel")
DECODE_SOURCES = ["decode.hip", "common.hpp", "launch.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stats_us(ms_list):
    """Mean, median and minimum of per-call event times (ms) in microseconds."""
    xs = sorted(ms_list)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"mean_us": round(1e3 * sum(xs) / n, 2), "median_us": round(1e3 * med, 2),
            "min_us": round(1e3 * xs[0], 2)}


def device_peaks(props):
    """Spec peaks beside the peaks implied by the device's own properties.

    The bf16 MFMA rate of a CDNA4 CU is 4096 flop per clock (4 SIMDs x 1024), so the
    device-derived peak is CUs x max engine clock x 4096.  The clock comes from the HIP
    runtime (hipDeviceAttributeClockRate, kHz).
    """
    clock_khz = getattr(props, "clock_rate", None)
    if not clock_khz:
        try:
            import ctypes
            hip = ctypes.CDLL("libamdhip64.so")
            v = ctypes.c_int(0)
            if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:   # ClockRate
                clock_khz = v.value
        except OSError:
            clock_khz = None
    cus = props.multi_processor_count
    out = {"hbm_spec_gbs": HBM_PEAK_GBS, "mfma_bf16_spec_tflops": MFMA_BF16_PEAK_TFLOPS,
           "cus": cus, "max_clock_mhz": round(clock_khz / 1e3, 1) if clock_khz else None,
           "mfma_bf16_from_props_tflops":
               round(cus * clock_khz * 1e3 * 4096 / 1e12, 1) if clock_khz else None}
    return out


def kernel_source_sha(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "paged_kv_cache_258_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Samples the GPU engine clock the driver reports (the current level of
    pp_dpm_sclk, marked '*') every few milliseconds in a background thread, while the
    timed calls run.  Gives the median / min / max MHz of the samples, or None where the
    file is not readable."""

    def __init__(self, period_s=0.002):
        import threading
        self.path = next((f for f in SCLK_FILES if os.access(f, os.R_OK)), None)
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def parse(text):
        for line in text.splitlines():
            if line.rstrip().endswith("*"):
                num = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                return int(num) if num else None
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                with open(self.path) as f:
                    mhz = self.parse(f.read())
                if mhz:
                    self.samples.append(mhz)
            except OSError:
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"median_mhz": xs[len(xs) // 2], "min_mhz": xs[0], "max_mhz": xs[-1],
                "samples": len(xs), "source": "pp_dpm_sclk, sampled every 2 ms"}


def prefill_counter_record(kernel_sha):
    """Per-leg counter figures of the committed prefill summary, if it was taken on the
    current prefill sources; otherwise None."""
    try:
        with open(PREFILL_COUNTERS_JSON) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    return c if c.get("source_sha") == kernel_sha else None


def prefill_roofline(leg, tflops, flop, median_us, counters):
    """The roofline object of one prefill leg: achieved algorithmic TFLOP/s of the median
    call against the dense bf16 MFMA peak, with MFMA-busy and the bytes read from beyond L2 from the
    counter summary when it matches the sources."""
    rec = (counters or {}).get("legs", {}).get(leg, {})
    return {"bound": "mfma", "kernel": "prefill_bf16_kernel", "achieved": round(tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": rec.get("fetch_bytes_per_call"), "mfma_busy": rec.get("mfma_busy"),
            "valu_mfma_coexec": rec.get("coexec_of_mfma_busy"),
            "counter_clock_mhz": rec.get("clock_mhz"),
            "algorithmic_flop_per_launch": int(flop), "avg_launch_us": round(median_us, 2),
            "kernel_source_sha": kernel_source_sha(PREFILL_SOURCES)}


def i32(a, dev):
    import numpy as np
    import torch
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=dev)


def bench_decode(dev, steps, warmup, graph=True):
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import accounting as acc
    from paged_kv_cache_258_amd import workloads as wl

    case = wl.c2_decode(dev)
    sh = case.shape
    lens_d = i32(case.context_lens, dev)
    table_d = i32(case.block_table, dev)
    slots_d = i32(case.slot_mapping, dev)
    sets = [(case.k_cache, case.v_cache)] + [(case.k_cache.clone(), case.v_cache.clone())
                                            for _ in range(2)]
    out = torch.empty_like(case.q)
    need = nkv.nkv_paged_attn_decode_workspace_size(len(case.context_lens), sh.num_q_heads,
                                                    sh.num_kv_heads, sh.head_dim,
                                                    case.block_table.shape[1], sh.block_size)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def step(i, ev=None):
        kc, vc = sets[i % 3]
        if ev is not None:
            ev[0].record()
        nkv.nkv_store_kvcache(case.k, case.v, kc, vc, slots_d)
        if ev is not None:
            ev[1].record()
        nkv.nkv_paged_attn_decode(case.q, kc, vc, lens_d, table_d, sh.scale, out=out, workspace=ws)
        if ev is not None:
            ev[2].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(i, evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / steps
    store_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    dec_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    dec_stats = stats_us([e[1].elapsed_time(e[2]) for e in evs])
    store_stats = stats_us([e[0].elapsed_time(e[1]) for e in evs])
    dec_bytes = acc.decode_bytes(case.context_lens, sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                                 sh.block_size, sh.elem_bytes)
    st_bytes = acc.store_bytes(case.slot_mapping, sh.num_kv_heads, sh.head_dim, sh.elem_bytes)
    # The decode call alone, `steps` calls back to back over the rotated pool copies between
    # one event pair: its average launch duration without the per-call event pairs, which
    # add a few microseconds each.
    rot = itertools.count()

    def decode_only():
        kc, vc = sets[next(rot) % 3]
        nkv.nkv_paged_attn_decode(case.q, kc, vc, lens_d, table_d, sh.scale, out=out, workspace=ws)

    dec_batched_ms = batched_us(decode_only, steps) * 1e-3
    log(f"[decode C2] step {ms_step*1e3:.1f} us (store {store_ms*1e3:.1f} us, decode "
        f"{dec_ms*1e3:.1f} us) -> decode {dec_bytes/dec_ms/1e6:.0f} GB/s, wall {wall:.3f}s; "
        f"decode calls back to back {dec_batched_ms*1e3:.1f} us -> {dec_bytes/dec_batched_ms/1e6:.0f} GB/s")

    # The same steps replayed from HIP graphs, captured after a warm-up call on a side
    # stream.  The calls allocate, memset and synchronise nothing.
    if not graph:
        return dict(case=case, ms_step=ms_step, store_ms=store_ms, dec_ms=dec_ms, dec_bytes=dec_bytes,
                    st_bytes=st_bytes, workspace_bytes=need, dec_stats=dec_stats, store_stats=store_stats,
                    dec_batched_ms=dec_batched_ms)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # one graph of three steps (one per rotated pool copy) for the bulk of the steps, and
    # one single-step graph per copy for the remainder
    three = torch.cuda.CUDAGraph()
    with torch.cuda.graph(three):
        for i in range(3):
            step(i)
    single = [torch.cuda.CUDAGraph() for _ in range(3)]
    for i, g in enumerate(single):
        with torch.cuda.graph(g):
            step(i)
    for _ in range(max(1, warmup // 3)):
        three.replay()
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0.record()
        for _ in range(steps // 3):
            three.replay()
        for i in range(steps % 3):
            single[i].replay()
        t1.record()
        torch.cuda.synchronize()
    graph_ms_step = t0.elapsed_time(t1) / steps
    log(f"[decode C2, graph replay] step {graph_ms_step*1e3:.1f} us over {steps} steps")
    return dict(case=case, ms_step=ms_step, store_ms=store_ms, dec_ms=dec_ms, dec_bytes=dec_bytes,
                st_bytes=st_bytes, workspace_bytes=need, dec_stats=dec_stats, store_stats=store_stats,
                dec_batched_ms=dec_batched_ms, graph_ms_step=graph_ms_step, engine_clock=clk.summary())


def prefill_inputs(dev, which):
    """C3 or C4 inputs on the device: the case, its pools (C4's shared prefix already
    stored), the index arrays as int32 device tensors and the output buffer."""
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import workloads as wl

    prefix = None
    if which == "C3":
        case = wl.c3_prefill(dev)
    else:
        prefix, case = wl.c4_prefix_chunk(dev)
    kc, vc = case.k_cache, case.v_cache
    if prefix is not None:
        pk, pv, ps = prefix
        nkv.nkv_store_kvcache(pk, pv, kc, vc, i32(ps, dev))
    cu_q, cu_k = i32(case.cu_seqlens_q, dev), i32(case.cu_seqlens_k, dev)
    table, slots = i32(case.block_table, dev), i32(case.slot_mapping, dev)
    return case, kc, vc, cu_q, cu_k, table, slots, torch.empty_like(case.q)


def batched_us(call, n):
    """Mean time per call of n back-to-back calls between one event pair: the launch and
    event overheads that a per-call event pair adds to a kernel of tens of microseconds are
    left out; the gaps between consecutive kernels stay in."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        call()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def bench_prefill(dev, which, steps, warmup, settle_s=1.5):
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import accounting as acc

    case, kc, vc, cu_q, cu_k, table, slots, out = prefill_inputs(dev, which)
    sh = case.shape

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        nkv.nkv_store_kvcache(case.k, case.v, kc, vc, slots)
        if ev is not None:
            ev[1].record()
        nkv.nkv_paged_attn_prefill(case.q, kc, vc, cu_q, cu_k, table, case.max_seqlen_q,
                                   case.max_seqlen_k, sh.scale, out=out)
        if ev is not None:
            ev[2].record()

    def timed(n):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for i in range(n):
            step(evs[i])
        torch.cuda.synchronize()
        return evs

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # The first tens of milliseconds of back-to-back MFMA work run slower than the rest
    # (the engine clock settles under the sustained load): time a few calls right away
    # ("cold"), keep the matrix cores busy for settle_s, then time the steady state.
    cold = stats_us([e[1].elapsed_time(e[2]) for e in timed(10)])
    with ClockSampler() as clk:          # over the settling and the timed calls
        t_end = time.perf_counter() + settle_s
        while time.perf_counter() < t_end:
            for _ in range(20):
                step()
            torch.cuda.synchronize()
        evs = timed(steps)
    st_stats = stats_us([e[0].elapsed_time(e[1]) for e in evs])
    pf_stats = stats_us([e[1].elapsed_time(e[2]) for e in evs])
    st_batched = batched_us(lambda: nkv.nkv_store_kvcache(case.k, case.v, kc, vc, slots), steps)
    # `steps` prefill calls back to back as well: reported beside the per-call median, which
    # stays the leg's time (back to back, the sustained MFMA load runs at a lower engine
    # clock than the steps with a store between two calls, and takes longer)
    pf_batched = batched_us(lambda: nkv.nkv_paged_attn_prefill(case.q, kc, vc, cu_q, cu_k, table,
                                                                 case.max_seqlen_q, case.max_seqlen_k,
                                                                 sh.scale, out=out), steps)
    # The median call: a rare stall of tens of milliseconds inside one timed interval (seen
    # on some boxes, in either leg and in the store before it) would otherwise dominate the
    # mean of 50 sub-ms calls; the means stay in prefill_call and store_call.
    pf_ms = pf_stats["median_us"] * 1e-3
    store_ms = st_stats["median_us"] * 1e-3
    flops = acc.prefill_flops(case.cu_seqlens_q, case.cu_seqlens_k, sh.num_q_heads, sh.head_dim)
    st_bytes = acc.store_bytes(case.slot_mapping, sh.num_kv_heads, sh.head_dim, sh.elem_bytes)
    tflops = flops / pf_ms / 1e9
    log(f"[prefill {which}] store {store_ms*1e3:.1f} us ({st_bytes/store_ms/1e6:.0f} GB/s; back to back "
        f"{st_batched:.1f} us -> {st_bytes/st_batched/1e3:.0f} GB/s), prefill {pf_ms*1e3:.1f} us "
        f"({pf_batched:.1f} us back to back) -> {tflops:.1f} TFLOP/s")
    return {"workload": which, "prefill_us": round(pf_ms * 1e3, 2),
            "tflops": round(tflops, 2), "frac_of_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "back_to_back_us": round(pf_batched, 2),
            "flop": flops, "prefill_call": pf_stats, "cold_prefill_call": cold,
            "settle_s": settle_s, "store_us": round(store_ms * 1e3, 2), "store_call": st_stats,
            "store_gbs": round(st_bytes / store_ms / 1e6, 1),
            "store_batched_us": round(st_batched, 2),
            "store_batched_gbs": round(st_bytes / st_batched / 1e3, 1),
            "store_batched_frac_of_hbm_peak": round(st_bytes / st_batched / 1e3 / HBM_PEAK_GBS, 4),
            "engine_clock": clk.summary(),
            "roofline": prefill_roofline(which, tflops, flops, pf_ms * 1e3,
                                         prefill_counter_record(kernel_source_sha(PREFILL_SOURCES)))}


def bench_varlen_prefill(dev, steps, warmup, settle_s=1.5):
    """C3's 8 x 2048-token prompts through the prefill over contiguous K/V (the branch
    without a prefix cache): q, k and v are views of one packed N(0,1) projection output
    [16384, (32 + 2*8) * 128] bf16.  Timed like the paged legs (cold calls, settle, median)."""
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import accounting as acc
    from paged_kv_cache_258_amd import workloads as wl

    sh = wl.QWEN3_8B
    lens = [2048] * 8
    t = sum(lens)
    hq, hkv, d = sh.num_q_heads, sh.num_kv_heads, sh.head_dim
    gen = torch.Generator(device=dev).manual_seed(wl.SEED_BASE + 79)
    qkv = wl.randn((t, (hq + 2 * hkv) * d), gen, dev, "bf16")
    q = qkv[:, :hq * d].view(t, hq, d)
    k = qkv[:, hq * d:(hq + hkv) * d].view(t, hkv, d)
    v = qkv[:, (hq + hkv) * d:].view(t, hkv, d)
    cu = wl.cu_seqlens(lens)
    cu_d = i32(cu, dev)
    out = torch.empty((t, hq, d), dtype=torch.bfloat16, device=dev)

    def call():
        nkv.nkv_attn_varlen_prefill(q, k, v, cu_d, cu_d, 2048, 2048, sh.scale, out=out)

    def timed(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        return stats_us([a.elapsed_time(b) for a, b in evs])

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    cold = timed(10)
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(20):
            call()
        torch.cuda.synchronize()
    st = timed(steps)
    bt = batched_us(call, steps)
    flops = acc.prefill_flops(cu, cu, hq, d)
    tflops = flops / (st["median_us"] * 1e-6) / 1e12
    log(f"[varlen prefill C3] {st['median_us']:.1f} us ({bt:.1f} us back to back) -> {tflops:.1f} TFLOP/s")
    return {"workload": "C3 prompts, contiguous K/V views of a packed qkv", "prefill_us": st["median_us"],
            "tflops": round(tflops, 2), "frac_of_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "back_to_back_us": round(bt, 2),
            "flop": flops, "prefill_call": st, "cold_prefill_call": cold, "settle_s": settle_s}


def bench_block_manager(reps=20):
    """Host cost of the C++ block manager on the long-context batch's shape: admit C5b's
    256 prompts (lengths log-uniform in [128, 32768], block_size 256; the first 64 share a
    4096-token prefix), then build the index arrays of one decode step for all 256 (one
    appended token each) and of a C3-shaped prefill (8 x 2048).  Median wall time per call."""
    import numpy as np
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import workloads as wl

    lens, _ = wl.c5_lengths("b", wl.SEED_BASE + 6)
    rng = np.random.default_rng(wl.SEED_BASE + 80)
    bs = 256
    shared = rng.integers(0, 151936, size=4096).astype(np.int32)
    prompts = []
    for i, n in enumerate(lens):
        t = rng.integers(0, 151936, size=int(n)).astype(np.int32)
        if i < 64 and n > 4096:
            t[:4096] = shared
        prompts.append(t)
    nblocks = sum(-(-int(n) // bs) + 1 for n in lens)
    maxb = max(-(-int(n) // bs) for n in lens) + 1

    def med(xs):
        return round(1e6 * sorted(xs)[len(xs) // 2], 1)

    admit, dec, cached = [], [], 0
    for r in range(max(3, reps // 4)):
        bm = nkv.BlockManager(nblocks, bs)
        t0 = time.perf_counter()
        cached = sum(bm.add_sequence(i, p) for i, p in enumerate(prompts))
        admit.append(time.perf_counter() - t0)
    ids = list(range(len(prompts)))
    for i in ids:
        bm.append_token(i, 7)
    for _ in range(reps):
        t0 = time.perf_counter()
        bm.prepare_decode(ids, maxb)
        dec.append(time.perf_counter() - t0)
    bm3 = nkv.BlockManager(8 * 8, bs)
    for i in range(8):
        bm3.add_sequence(i, rng.integers(0, 151936, size=2048).astype(np.int32))
    pre = []
    for _ in range(reps):
        t0 = time.perf_counter()
        bm3.prepare_prefill(list(range(8)), 8)
        pre.append(time.perf_counter() - t0)
    out = {"admit_256_prompts_us": med(admit), "prompt_tokens": int(sum(lens)), "cached_tokens": int(cached),
           "prepare_decode_256_us": med(dec), "prepare_prefill_8x2048_us": med(pre),
           "note": "host wall time through the Python binding, median"}
    log(f"[block manager] admit 256 prompts ({int(sum(lens))} tokens, {int(cached)} cached) "
        f"{out['admit_256_prompts_us']:.0f} us; decode arrays {out['prepare_decode_256_us']:.0f} us; "
        f"prefill arrays (8 x 2048) {out['prepare_prefill_8x2048_us']:.0f} us")
    return out


def bench_rope_store(dev, which, steps, warmup):
    """q/k RMSNorm + rotary + KV store over the new tokens of a leg: the 16384 prompt tokens
    of C3 (8 x 2048 at positions 0..2047) or the 64 decode tokens of C2 (at L_b - 1).
    Synthetic inputs: N(0,1) projection output, weights of ones, a uniform [-1, 1] table
    (its values do not change the work)."""
    import numpy as np
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import accounting as acc
    from paged_kv_cache_258_amd import workloads as wl

    if which == "C3":
        case = wl.c3_prefill(dev)
        lens = np.diff(case.cu_seqlens_q)
        pos = np.concatenate([np.arange(l) for l in lens]).astype(np.int32)
    else:
        case = wl.c2_decode(dev)
        pos = (np.asarray(case.context_lens) - 1).astype(np.int32)
    sh = case.shape
    t = len(case.slot_mapping)
    gen = torch.Generator(device=dev).manual_seed(wl.SEED_BASE + 77)
    width = (sh.num_q_heads + 2 * sh.num_kv_heads) * sh.head_dim
    qkv = wl.randn((t, width), gen, dev, "bf16")
    w = torch.ones(sh.head_dim, dtype=torch.bfloat16, device=dev)
    max_pos = 40960
    table = torch.rand((max_pos, sh.head_dim), generator=gen, device=dev, dtype=torch.float32) * 2 - 1
    pos_d, slots_d = i32(pos, dev), i32(case.slot_mapping, dev)
    q_out = torch.empty((t, sh.num_q_heads, sh.head_dim), dtype=torch.bfloat16, device=dev)

    def call():
        nkv.nkv_qk_norm_rope_store(qkv, pos_d, w, w, table, slots_d, case.k_cache, case.v_cache,
                                   sh.num_q_heads, 1e-6, q_out=q_out)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    st = stats_us([a.elapsed_time(b) for a, b in evs])
    bt = batched_us(call, steps)
    nbytes = acc.qk_norm_rope_store_bytes(case.slot_mapping, sh.num_q_heads, sh.num_kv_heads,
                                          sh.head_dim, sh.elem_bytes)
    gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
    bgbs = nbytes / (bt * 1e-6) / 1e9
    log(f"[qk-norm+rope+store {which}] {t} tokens: {st['mean_us']:.1f} us -> {gbs:.0f} GB/s "
        f"(batched {bt:.1f} us -> {bgbs:.0f} GB/s)")
    return {"workload": f"{which} tokens ({t})", "call": st, "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "batched_us": round(bt, 2),
            "batched_gbs": round(bgbs, 1), "batched_frac_of_hbm_peak": round(bgbs / HBM_PEAK_GBS, 4)}


def bench_add_rms_norm(dev, which, steps, warmup):
    """Residual add + RMSNorm over the 4096-wide hidden rows of a leg's new tokens: C3's
    16384 prompt tokens or C2's 64 decode tokens.  Inputs from workloads.norm_rows; out and
    residual_out are separate buffers (the in-place form moves the same bytes)."""
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import accounting as acc
    from paged_kv_cache_258_amd import workloads as wl

    t = 16384 if which == "C3" else 64
    h = wl.QWEN3_8B_HIDDEN
    x, r, w = wl.norm_rows(t, h, wl.SEED_BASE + 78, dev)
    out, res = torch.empty_like(x), torch.empty_like(x)

    def call():
        nkv.nkv_add_rms_norm(x, r, w, 1e-6, out=out, residual_out=res)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    st = stats_us([a.elapsed_time(b) for a, b in evs])
    bt = batched_us(call, steps)
    nbytes = acc.add_rms_norm_bytes(t, h, 2)
    gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
    bgbs = nbytes / (bt * 1e-6) / 1e9
    log(f"[add+rmsnorm {which}] {t} x {h}: {st['mean_us']:.1f} us -> {gbs:.0f} GB/s "
        f"(batched {bt:.1f} us -> {bgbs:.0f} GB/s)")
    return {"workload": f"{which} tokens ({t}) x hidden {h}", "call": st, "bytes": nbytes,
            "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "batched_us": round(bt, 2), "batched_gbs": round(bgbs, 1),
            "batched_frac_of_hbm_peak": round(bgbs / HBM_PEAK_GBS, 4)}


def blas_threads():
    try:
        import threadpoolctl
        blas = [p["num_threads"] for p in threadpoolctl.threadpool_info() if p["user_api"] == "blas"]
        return max(blas) if blas else 1
    except Exception:  # noqa: BLE001
        return 1


def cpu_baseline_layer(layer, lens, kind):
    """The float64 oracle's decode (decode_ref) of one full layer of a long-context
    workload on the host cores: the layer's q, pools and table copied to the host (timed
    apart), then decode_ref over every sequence.  Reported per layer and, extrapolated,
    for the 36 layers."""
    import numpy as np
    import torch
    from oracle import ref
    from paged_kv_cache_258_amd import accounting as acc
    from paged_kv_cache_258_amd import workloads as wl

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    q, kc, vc, table = layer
    sh = wl.QWEN3_8B
    t = time.perf_counter()
    qh, kh, vh = bits(q), bits(kc), bits(vc)
    t_copy = time.perf_counter() - t
    t = time.perf_counter()
    ref.decode_ref(qh, kh, vh, lens, table, sh.scale, elem="bf16")
    per = time.perf_counter() - t
    nbytes = acc.decode_bytes(lens, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                              sh.elem_bytes)
    log(f"[cpu oracle C5{kind}] layer 0: {per:.2f} s ({len(lens)} seqs, sum ctx {int(lens.sum())}), "
        f"D2H copy {t_copy:.2f}s")
    return {"workload": f"C5{kind}", "value": round(nbytes / per / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"full layer 0 of C5{kind} ({len(lens)} seqs, sum ctx {int(lens.sum())}): "
                      f"decode_ref in numpy float64, 1 run",
            "per_layer_s": round(per, 3), "all_layers_s_extrapolated": round(per * wl.NUM_LAYERS, 2),
            "d2h_copy_s": round(t_copy, 2), "cpu_model": cpu_model(),
            "host_cpus": len(os.sched_getaffinity(0))}


def bench_c5(dev, kind, reps, warmup, cpu=False):
    """C5a / C5b: layer-by-layer decode over all 36 layers' pools (no store: the pools
    are pre-filled).  Every layer has its own pools, so no layer finds another's K/V in
    cache.  If the 36 layers do not fit in free device memory minus an 8 GB margin, the
    next seed is tried (and reported)."""
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import accounting as acc
    from paged_kv_cache_258_amd import workloads as wl

    sh = wl.QWEN3_8B
    base_k = 5 if kind == "a" else 6
    torch.cuda.empty_cache()
    free = torch.cuda.mem_get_info(dev)[0]
    for seed_k in range(base_k, base_k + 5):
        lens, _ = wl.c5_lengths(kind, wl.SEED_BASE + seed_k)
        nb = sum(wl.blocks_needed(l, sh.block_size) for l in lens)
        need = 2 * nb * sh.block_size * sh.num_kv_heads * sh.head_dim * sh.elem_bytes * wl.NUM_LAYERS
        if need + 8e9 <= free:
            break
        log(f"[decode C5{kind}] seed {wl.SEED_BASE + seed_k} needs {need/1e9:.1f} GB of "
            f"{free/1e9:.1f} GB free: next seed")
    else:
        return {"workload": f"C5{kind}", "skipped": f"does not fit: {free/1e9:.1f} GB free"}
    t = time.perf_counter()
    try:
        mld = wl.c5_decode(kind, dev, seed_k=seed_k)
        torch.cuda.synchronize()
    except torch.OutOfMemoryError as e:
        torch.cuda.empty_cache()
        return {"workload": f"C5{kind}", "skipped": f"out of device memory: {e}"[:200]}
    gen_s = time.perf_counter() - t
    lens = mld.context_lens
    lens_d = i32(lens, dev)
    tables = [i32(layer[3], dev) for layer in mld.layers]
    nseq = len(lens)
    need = nkv.nkv_paged_attn_decode_workspace_size(nseq, sh.num_q_heads, sh.num_kv_heads,
                                                    sh.head_dim, mld.layers[0][3].shape[1],
                                                    sh.block_size)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    outs = [torch.empty_like(layer[0]) for layer in mld.layers]

    def run_all():
        for i, (q, kc, vc, _) in enumerate(mld.layers):
            nkv.nkv_paged_attn_decode(q, kc, vc, lens_d, tables[i], sh.scale, out=outs[i],
                                      workspace=ws)

    for _ in range(warmup):
        run_all()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run_all()
    e1.record()
    torch.cuda.synchronize()
    per_layer_ms = e0.elapsed_time(e1) / reps / wl.NUM_LAYERS
    nbytes = acc.decode_bytes(lens, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                              sh.elem_bytes)
    gbs = nbytes / per_layer_ms / 1e6
    log(f"[decode C5{kind}] {wl.NUM_LAYERS} layers, per layer {per_layer_ms*1e3:.1f} us -> "
        f"{gbs:.0f} GB/s (sum ctx {int(lens.sum())}, generated in {gen_s:.1f}s)")
    res = {"workload": f"C5{kind}", "seed": wl.SEED_BASE + seed_k, "num_seqs": nseq,
           "sum_context_tokens": int(lens.sum()), "layers": wl.NUM_LAYERS, "reps": reps,
           "per_layer_us": round(per_layer_ms * 1e3, 2),
           "all_layers_ms": round(per_layer_ms * wl.NUM_LAYERS, 3),
           "decode_bytes_per_layer": int(nbytes), "gbs": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del tables, outs, ws
    if cpu:
        res["cpu_baseline"] = cpu_baseline_layer(mld.layers[0], lens, kind)
    del mld
    torch.cuda.empty_cache()
    return res


def cpu_baseline(case, budget_s=10.0):
    """The float64 oracle (store_ref + decode_ref) on the full C2 batch, on host cores."""
    import numpy as np
    import torch
    from oracle import ref
    from paged_kv_cache_258_amd import accounting as acc

    def bits(t):
        return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    t_copy = time.perf_counter()
    q, k, v = bits(case.q), bits(case.k), bits(case.v)
    kc, vc = bits(case.k_cache), bits(case.v_cache)
    t_copy = time.perf_counter() - t_copy
    sh = case.shape
    runs, t_tot = 0, 0.0
    while runs == 0 or (t_tot < budget_s and runs < 20):
        t = time.perf_counter()
        kb, vb = ref.store_ref(k, v, kc, vc, case.slot_mapping)
        ref.decode_ref(q, kb, vb, case.context_lens, case.block_table, sh.scale, elem="bf16")
        t_tot += time.perf_counter() - t
        runs += 1
    per = t_tot / runs
    nbytes = acc.decode_bytes(case.context_lens, sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                              sh.block_size, sh.elem_bytes) + \
        acc.store_bytes(case.slot_mapping, sh.num_kv_heads, sh.head_dim, sh.elem_bytes)
    log(f"[cpu oracle] {per:.3f} s per C2 step ({runs} runs), D2H copy {t_copy:.2f}s")
    return {"value": round(nbytes / per / 1e9, 4), "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"full C2 batch (64 seqs, sum ctx {int(case.context_lens.sum())}): "
                      f"store_ref + decode_ref in numpy float64, {runs} run(s), "
                      f"{per:.2f} s each; host affinity {len(os.sched_getaffinity(0))} cpus",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


def traffic_from_counters(kernel_sha):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; otherwise None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("source_sha") != kernel_sha:
        return None
    return c.get("hbm_bytes_per_decode_call")


def counter_pass(dev, steps, warmup):
    """Workload of a rocprofv3 --pmc pass: a copy of known size, then the decode leg."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    d = bench_decode(dev, steps, warmup, graph=False)
    print(json.dumps({"counter_pass": True, "copy_bytes": COPY_BYTES, "copy_launches": 3,
                      "decode_calls": steps + warmup,
                      "algorithmic_bytes_per_decode_call": int(d["dec_bytes"])}), flush=True)


def summarize_counters(fetch_csv, write_csv):
    """Turn the two rocprofv3 counter CSVs of --counter-pass into profiles/ summaries."""
    import csv

    def per_dispatch(path, counter):
        rows = {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                e = rows.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
                e[1] += float(r["Counter_Value"])
        return list(rows.values())

    def split(rows, counter):
        copy = [v for n, v in rows if "neg_kernel" in n]
        calls = [v for n, v in rows if DECODE_KERNELS[0] in n]
        dec = [v for n, v in rows if any(k in n for k in DECODE_KERNELS)]
        if not copy or not calls:
            raise SystemExit(f"{counter}: no copy or decode dispatches found")
        return copy, len(calls), sum(dec)

    out = {"source_sha": kernel_source_sha(DECODE_SOURCES), "copy_bytes": COPY_BYTES}
    total = 0.0
    for path, counter, key in ((fetch_csv, "FETCH_SIZE", "fetch"), (write_csv, "WRITE_SIZE", "write")):
        copy, ncalls, dec_kib = split(per_dispatch(path, counter), counter)
        copy_kib = sum(copy) / len(copy)
        factor = COPY_BYTES / (copy_kib * 1024.0)
        per_call = dec_kib / ncalls * 1024.0 * factor
        total += per_call
        out[key] = {"copy_kib_per_launch": round(copy_kib, 1), "factor": round(factor, 5),
                    "decode_calls": ncalls, "kib_per_call_raw": round(dec_kib / ncalls, 1),
                    "bytes_per_call": int(per_call)}
    out["hbm_bytes_per_decode_call"] = int(total)
    out["commands"] = [
        "rocprofv3 --pmc FETCH_SIZE -d DIR_F -o pass --output-format csv -- "
        "python bench.py --counter-pass --steps 10 --warmup 2",
        "rocprofv3 --pmc WRITE_SIZE -d DIR_W -o pass --output-format csv -- "
        "python bench.py --counter-pass --steps 10 --warmup 2",
        "python bench.py --summarize-counters DIR_F/pass_counter_collection.csv "
        "DIR_W/pass_counter_collection.csv"]
    os.makedirs(os.path.dirname(COUNTERS), exist_ok=True)
    with open(COUNTERS, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def prefill_counter_pass(dev):
    """Workload of a rocprofv3 --pmc pass for the prefill legs: the copy of known size,
    then for C3 and C4 the store of the new tokens and PREFILL_CALLS prefill calls."""
    import torch
    import paged_kv_cache_258_amd as nkv
    from paged_kv_cache_258_amd import accounting as acc

    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    legs = {}
    for which in ("C3", "C4"):
        case, kc, vc, cu_q, cu_k, table, slots, out = prefill_inputs(dev, which)
        nkv.nkv_store_kvcache(case.k, case.v, kc, vc, slots)
        for _ in range(PREFILL_CALLS):
            nkv.nkv_paged_attn_prefill(case.q, kc, vc, cu_q, cu_k, table, case.max_seqlen_q,
                                       case.max_seqlen_k, case.shape.scale, out=out)
        torch.cuda.synchronize()
        legs[which] = acc.prefill_flops(case.cu_seqlens_q, case.cu_seqlens_k,
                                        case.shape.num_q_heads, case.shape.head_dim)
        del case, kc, vc, out
    print(json.dumps({"prefill_counter_pass": True, "calls_per_leg": PREFILL_CALLS,
                      "flop": legs}), flush=True)


# Prefill legs told apart by grid (threads): (sequence x KV head) x pairs of q-tiles x 512.
PREFILL_GRIDS = {"C3": 64 * 16 * 512, "C4": 128 * 4 * 512}
PREFILL_FLOP = {"C3": 275012124672, "C4": 171865800704}
# bytes the leg must read at least once: q, the K/V rows its sequences span (C4: the
# shared prefix once, every chunk), the tables
PREFILL_UNIQUE_READ = {"C3": 16384 * 32 * 128 * 2 + 2 * 16384 * 8 * 128 * 2,
                       "C4": 8192 * 32 * 128 * 2 + 2 * (1024 + 16 * 512) * 8 * 128 * 2}


def summarize_prefill_counters(paths):
    """Write profiles/prefill_c3_c4_counters.md from the CSVs of --prefill-counter-pass."""
    import csv
    import statistics as stx

    per = {}        # (leg, counter) -> per-dispatch values
    dur = {}        # leg -> durations (us)
    copy = {}       # counter -> per-launch values of the calibration copy
    simds, xcc = None, 1
    for path in paths:
        seen = {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                key = (int(r["Dispatch_Id"]), r["Counter_Name"])
                e = seen.setdefault(key, [r["Kernel_Name"], int(r["Grid_Size"]), 0.0,
                                          int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
                e[2] += float(r["Counter_Value"])
        agent = os.path.join(os.path.dirname(path), os.path.basename(path).replace(
            "counter_collection", "agent_info"))
        if simds is None and os.path.exists(agent):
            with open(agent, newline="") as f:
                for r in csv.DictReader(f):
                    if int(r.get("Simd_Count") or 0) > 0:
                        simds = int(r["Simd_Count"])
                        xcc = int(r.get("Num_Xcc") or 1)
        by_leg = {}
        for (disp, counter), (name, grid, val, ns) in sorted(seen.items()):
            if "neg_kernel" in name:
                copy.setdefault(counter, []).append(val)
            if "prefill_bf16_kernel" not in name:
                continue
            leg = next((k for k, g in PREFILL_GRIDS.items() if g == grid), None)
            if leg is None:
                continue
            by_leg.setdefault((leg, counter), []).append(val)
            dur.setdefault((leg, path), {})[disp] = ns / 1e3
        for k, v in by_leg.items():
            per[k] = v[2:] if len(v) > 4 else v            # skip the warm-up calls
    durs = {}
    for (leg, _), d in dur.items():
        v = list(d.values())
        durs.setdefault(leg, []).extend(v[2:] if len(v) > 4 else v)
    simds = simds or 1024

    def m(leg, c):
        v = per.get((leg, c))
        return stx.mean(v) if v else None

    lines = ["# Prefill counters: C3 and C4 (`prefill_bf16_kernel`), MFMA utilisation, LDS, L2 and HBM",
             "",
             f"Prefill sources sha {kernel_source_sha(PREFILL_SOURCES)} (`prefill.hip`, `common.hpp`, "
             "`launch.hpp`).  Qwen3-8B heads (32 Q / 8 KV, head_dim 128), block_size 256, bf16.",
             "",
             "Commands (repo root, MI355X, ROCm 7.2; one rocprofv3 pass per counter group):",
             ""]
    for i, grp in enumerate(PREFILL_COUNTER_GROUPS):
        lines.append(f"    rocprofv3 --pmc {' '.join(grp)} -d DIR{i} -o pass --output-format csv -- "
                     "python bench.py --prefill-counter-pass")
    lines += ["    python bench.py --summarize-prefill-counters DIR0/pass_counter_collection.csv "
              "DIR1/pass_counter_collection.csv DIR2/pass_counter_collection.csv", "",
              f"Each pass runs {PREFILL_CALLS} calls per leg; the first 2 are dropped.  Values are per "
              "dispatch, summed over the chip; SQ_* cycle counters count shader-clock cycles "
              "(SQ_WAVE_CYCLES, SQ_ACTIVE_INST_*, SQ_WAIT_* in units of 4 cycles), "
              f"GRBM_GUI_ACTIVE counts GPU-busy cycles summed over the {xcc} XCDs; the chip has "
              f"{simds} SIMDs.  The dispatches run one at a time under the counters, so their "
              "durations are longer than bench.py's steady-state calls.", "",
              "| counter | C3 | C4 |", "|---|---|---|"]
    counters = [c for grp in PREFILL_COUNTER_GROUPS for c in grp]
    for c in counters + ["duration_us"]:
        vals = []
        for leg in ("C3", "C4"):
            x = stx.mean(durs[leg]) if c == "duration_us" and durs.get(leg) else m(leg, c)
            vals.append("—" if x is None else (f"{x:,.2f}" if c == "duration_us" else f"{x:,.0f}"))
        lines.append(f"| {c} | {vals[0]} | {vals[1]} |")
    fetch_copy = stx.mean(copy["FETCH_SIZE"]) if copy.get("FETCH_SIZE") else None
    factor = COPY_BYTES / (fetch_copy * 1024.0) if fetch_copy else None
    lines += ["", "Derived:", "", "| figure | C3 | C4 |", "|---|---|---|"]

    def row(label, f):
        out = []
        for leg in ("C3", "C4"):
            try:
                x = f(leg)
            except (TypeError, ZeroDivisionError, KeyError):
                x = None
            out.append("—" if x is None else x)
        lines.append(f"| {label} | {out[0]} | {out[1]} |")

    d = lambda leg: stx.mean(durs[leg])
    gui = lambda leg: m(leg, "GRBM_GUI_ACTIVE") / xcc          # busy cycles of one XCD
    row("shader clock, MHz (GRBM_GUI_ACTIVE per XCD / duration)", lambda leg: f"{gui(leg) / d(leg):,.0f}")
    row("TFLOP/s in the counted dispatches (algorithmic flop / duration)",
        lambda leg: f"{PREFILL_FLOP[leg] / d(leg) / 1e6:,.1f}")
    row("of the 2.5 PFLOP/s dense bf16 peak", lambda leg: f"{PREFILL_FLOP[leg] / d(leg) / 1e6 / MFMA_BF16_PEAK_TFLOPS:.3f}")
    row("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x GRBM_GUI_ACTIVE per XCD)",
        lambda leg: f"{m(leg, 'SQ_VALU_MFMA_BUSY_CYCLES') / (simds * gui(leg)):.3f}")
    row("MFMA busy cycles / the flop's cycles at 1024 flop per SIMD-cycle",
        lambda leg: f"{m(leg, 'SQ_VALU_MFMA_BUSY_CYCLES') / (PREFILL_FLOP[leg] / 1024):.3f}")
    row("VALU-MFMA co-execution / MFMA busy",
        lambda leg: f"{m(leg, 'SQ_VALU_MFMA_COEXEC_CYCLES') / m(leg, 'SQ_VALU_MFMA_BUSY_CYCLES'):.3f}")
    row("LDS bank conflicts / LDS active (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)",
        lambda leg: f"{m(leg, 'SQ_LDS_BANK_CONFLICT') / m(leg, 'SQ_LDS_IDX_ACTIVE'):.3f}")
    row("LDS waits / all instruction waits (SQ_WAIT_INST_LDS / SQ_WAIT_INST_ANY)",
        lambda leg: f"{m(leg, 'SQ_WAIT_INST_LDS') / m(leg, 'SQ_WAIT_INST_ANY'):.3f}")
    row("L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))",
        lambda leg: f"{m(leg, 'TCC_HIT_sum') / (m(leg, 'TCC_HIT_sum') + m(leg, 'TCC_MISS_sum')):.3f}")
    row(f"bytes read from beyond L2, MALL hits included (FETCH_SIZE x {factor:.3f})" if factor
        else "bytes read from beyond L2, MALL hits included",
        lambda leg: f"{m(leg, 'FETCH_SIZE') * 1024 * factor / 1e6:,.1f} MB")
    row("... / bytes the leg must read once (q, K/V, tables)",
        lambda leg: f"{m(leg, 'FETCH_SIZE') * 1024 * factor / PREFILL_UNIQUE_READ[leg]:.2f}")
    lines += ["", f"Calibration: a torch.neg over {COPY_BYTES >> 20} MiB of bf16 reads {COPY_BYTES >> 20} MiB; "
              f"FETCH_SIZE reads it as {fetch_copy:,.0f} KiB per launch." if fetch_copy else ""]
    text = "\n".join(lines) + "\n"
    with open(PREFILL_COUNTERS, "w") as f:
        f.write(text)
    print(text)
    # the figures bench.py's prefill roofline blocks quote, behind the same source check
    legs = {}
    for leg in ("C3", "C4"):
        def val(f):
            try:
                return f()
            except (TypeError, ZeroDivisionError, KeyError):
                return None
        legs[leg] = {
            "duration_us": val(lambda: round(d(leg), 2)),
            "clock_mhz": val(lambda: round(gui(leg) / d(leg))),
            "mfma_busy": val(lambda: round(m(leg, "SQ_VALU_MFMA_BUSY_CYCLES") / (simds * gui(leg)), 4)),
            "coexec_of_mfma_busy": val(lambda: round(m(leg, "SQ_VALU_MFMA_COEXEC_CYCLES") /
                                                     m(leg, "SQ_VALU_MFMA_BUSY_CYCLES"), 4)),
            "fetch_bytes_per_call": val(lambda: int(m(leg, "FETCH_SIZE") * 1024 * factor)),
            "lds_bank_conflict_share": val(lambda: round(m(leg, "SQ_LDS_BANK_CONFLICT") /
                                                         m(leg, "SQ_LDS_IDX_ACTIVE"), 4)),
        }
    with open(PREFILL_COUNTERS_JSON, "w") as f:
        json.dump({"source_sha": kernel_source_sha(PREFILL_SOURCES), "legs": legs}, f, indent=1)


PREFILL_COUNTER_GROUPS = [
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES",
     "SQ_WAIT_INST_ANY", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
     "TCC_HIT_sum", "TCC_MISS_sum"],
    ["FETCH_SIZE"],
]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill legs")
    ap.add_argument("--no-c5", action="store_true", help="skip the 36-layer C5a/C5b decode legs")
    ap.add_argument("--counter-pass", action="store_true",
                    help="copy calibration + decode leg only (run under rocprofv3 --pmc)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/decode_c2_counters.json from two --pmc passes")
    ap.add_argument("--prefill-counter-pass", action="store_true",
                    help="copy calibration + C3 and C4 prefill calls only (run under rocprofv3 --pmc)")
    ap.add_argument("--summarize-prefill-counters", nargs=3, metavar="CSV",
                    help="write profiles/prefill_c3_c4_counters.md from the three --pmc passes")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_prefill_counters:
        summarize_prefill_counters(args.summarize_prefill_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the data plane shards by KV head; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_258_amd as nkv

    nkv.load()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} ({getattr(props, 'gcnArchName', '?')}), "
        f"{props.multi_processor_count} CUs")

    torch.cuda.synchronize()
    if args.counter_pass:
        counter_pass(dev, args.steps, args.warmup)
        return
    if args.prefill_counter_pass:
        prefill_counter_pass(dev)
        return
    d = bench_decode(dev, args.steps, args.warmup)
    prefill = []
    if not args.no_prefill:
        prefill.append(bench_prefill(dev, "C3", args.steps, 2))
        prefill.append(bench_prefill(dev, "C4", args.steps, 2))
        prefill.append(bench_varlen_prefill(dev, args.steps, 2))
    rope_store = []
    if not args.no_prefill:
        for which in ("C3", "C2"):
            rope_store.append(bench_rope_store(dev, which, args.steps, 3))
    add_rms = []
    if not args.no_prefill:
        for which in ("C3", "C2"):
            add_rms.append(bench_add_rms_norm(dev, which, args.steps, 3))
    long_decode = []
    if not args.no_c5:
        for kind in ("a", "b"):
            long_decode.append(bench_c5(dev, kind, 5, 1, cpu=not args.no_cpu))
    cpu = None if args.no_cpu else cpu_baseline(d["case"])
    block_manager = bench_block_manager()

    step_bytes = d["dec_bytes"] + d["st_bytes"]
    value = step_bytes / d["graph_ms_step"] / 1e6
    achieved = d["dec_bytes"] / d["dec_batched_ms"] / 1e6
    sha = kernel_source_sha(DECODE_SOURCES)
    case = d["case"]
    line = {
        "metric": "paged decode attn HBM GB/s (% peak); prefill attn TFLOP/s (% MFMA peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["graph_ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "C2 Qwen3-8B-shaped single-layer paged decode step (store 64 new "
                        "tokens + decode): 64 seqs, context U[512,4096], 32 Q / 8 KV heads, "
                        "head_dim 128, block_size 256, bf16",
            "num_seqs": len(case.context_lens),
            "sum_context_tokens": int(case.context_lens.sum()),
            "num_blocks": int(case.k_cache.shape[0]),
            "step_bytes": int(step_bytes),
            "pool_copies_rotated": 3,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "nkv_paged_attn_decode (decode_streamk_kernel + decode_fixup_kernel)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_counters(sha),
            "algorithmic_bytes_per_launch": int(d["dec_bytes"]),
            "avg_launch_us": round(d["dec_batched_ms"] * 1e3, 2),
            "timing": f"{args.steps} decode calls back to back over the 3 rotated pool copies "
                      "between one event pair on the launch stream, per call",
            "per_call_event_us": round(d["dec_ms"] * 1e3, 2),
            "kernel_source_sha": sha,
        },
        "decode_call": d["dec_stats"],
        "eager_step": {"ms_per_step": round(d["ms_step"], 5),
                       "value": round(step_bytes / d["ms_step"] / 1e6, 1), "unit": "GB/s"},
        "peaks": device_peaks(props),
        "engine_clock": {"decode_graph_steps": d.get("engine_clock"),
                         "prefill_C3": prefill[0].get("engine_clock") if prefill else None,
                         "prefill_C4": prefill[1].get("engine_clock") if len(prefill) > 1 else None},
        "host": {"cpu_model": cpu_model(), "cpus": len(os.sched_getaffinity(0))},
        "store": {"avg_launch_us": round(d["store_ms"] * 1e3, 2), "call": d["store_stats"],
                  "gbs": round(d["st_bytes"] / d["store_ms"] / 1e6, 1)},
        "prefill": prefill,
        "qk_norm_rope_store": rope_store,
        "add_rms_norm": add_rms,
        "long_decode": long_decode,
        "block_manager": block_manager,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
