#!/usr/bin/env python3
"""Benchmark of the sliding-window GQA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the prefill hot path over the 8192-token Mistral-7B
attention layer (batch 1, 32 query / 8 KV heads, head_dim 128, W = 4096,
bf16, RoPE theta 10000): key rotation, the band-restricted attention, and the
rolling-buffer write of the chunk's keys and values.  `value` is the
algorithmic prefill FLOP rate of that step (4*D*Hq*sum_i |A(i)|).  The decode
half of the metric is measured on the batched-decode workload (64 sequences,
256 steps of cache write + decode) and reported under "decode".

Inputs are synthetic (seeded N(0,1), bf16) and resident in HBM before timing.
Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SWA prefill TFLOP/s + decode HBM GB/s, W=4096 GQA 32/8 hd128 bf16"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E peak (published)


def profiled_traffic(name, sources):
    """HBM bytes per launch from the committed rocprofv3 summary profiles/<name>.txt
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a plain
    256 MiB copy), or None when the summary is missing or was taken on other
    kernel sources than the ones built now."""
    try:
        text = open(os.path.join(ROOT, "profiles", name + ".txt")).read()
    except OSError:
        return None
    h = re.search(r"source_sha256_16: (\w+)", text)
    t = re.search(r"traffic_bytes: (\d+)", text)
    if not h or not t:
        return None
    return int(t.group(1)) if source_hash(sources) == h.group(1) else None


def profiled_avg_us(name, sources):
    """rocprofv3's average duration (us) of the profile's kernel from the
    committed summary profiles/<name>.txt, or None when it was taken on other
    sources than the ones built now."""
    try:
        text = open(os.path.join(ROOT, "profiles", name + ".txt")).read()
    except OSError:
        return None
    h = re.search(r"source_sha256_16: (\w+)", text)
    a = re.search(r"kernel_avg_us: ([0-9.]+)", text)
    if not h or not a or h.group(1) != source_hash(sources):
        return None
    return float(a.group(1))


def source_hash(sources):
    sha = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "sliding_window_gqa_amd", "csrc", f), "rb") as fh:
            sha.update(fh.read())
    return sha.hexdigest()[:16]


def prewarm(fn, seconds, torch):
    """Run fn untimed for about `seconds` (then synchronize)."""
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()


def band_pairs(N, W, start=0, n_sink=0):
    """sum over queries i in [start, start+N) of |A(i)| (all earlier keys exist)."""
    tot = 0
    for i in range(start, start + N):
        lo = max(0, i - W + 1)
        tot += i - lo + 1 + min(n_sink, lo)
    return tot


def attn_flops(pairs, D=128, Hq=32):
    return 4 * D * Hq * pairs


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prewarm-s", type=float, default=0.3,
                    help="untimed seconds of the same step before the warmup steps, so that the timed "
                         "region runs at the GPU's sustained clocks (they ramp over the first ~50 ms)")
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the chunked / full-causal / sink timings")
    ap.add_argument("--only", choices=["prefill", "decode", "chunked", "sink", "dilated", "mixed", "all"], default="all",
                    help="restrict the GPU work (for profiler runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (scales HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import sliding_window_gqa_amd as swa
    from sliding_window_gqa_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    result = {"metric": METRIC}

    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib << 20
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nb
        del src, dst

    # ------------------------------------------------------------------
    # prefill: N=8192, W=4096 (the headline workload)
    # ------------------------------------------------------------------
    wl = synth.workload(2)
    N, Hq, Hkv, D, W = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    p = swa.make_params(1, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
    q = synth.normal((1, N, Hq, D), 2, "q").to(dev)
    k = synth.normal((1, N, Hkv, D), 2, "k").to(dev)
    v = synth.normal((1, N, Hkv, D), 2, "v").to(dev)
    kc = torch.zeros((1, W, Hkv, D), dtype=bf, device=dev)
    vc = torch.zeros_like(kc)
    start = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((1, N, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
    k_rot = torch.empty_like(k)
    pairs2 = band_pairs(N, W)
    flops2 = attn_flops(pairs2)

    def prefill_step(ev=None):
        # The layer's first chunk: its attention reads no cache, so the key
        # rotation and the cache write run as one pass before it.
        # ev: events around the attention (two per step: the pass before it
        # is the interval from the previous step's second event)
        swa.swa_rope_keys_cache_write(p, k, v, start, kc, vc, k_rot)
        if ev is not None:
            ev[0].record()
        swa.swa_prefill_attention(p, q, k_rot, v, None, None, start, out, lse)
        if ev is not None:
            ev[1].record()

    if args.only in ("prefill", "all"):
        prewarm(prefill_step, args.prewarm_s, torch)
        for _ in range(args.warmup):
            prefill_step()
        torch.cuda.synchronize()
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record()
        for s in range(args.steps):
            prefill_step(evs[s])
        t1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_step = t0.elapsed_time(t1) / args.steps
        attn_times = sorted(e[0].elapsed_time(e[1]) for e in evs)
        attn_ms = sum(attn_times) / args.steps
        achieved = flops2 / (attn_ms * 1e-3) / 1e12
        both_ms = (t0.elapsed_time(evs[0][0]) + sum(evs[s - 1][1].elapsed_time(evs[s][0])
                                                    for s in range(1, args.steps))) / args.steps

        # the two passes the fused one replaces, timed inside the step they
        # would make (rotation, attention, cache write; 20 steps, events around
        # each small launch, the attention keeping the GPU ahead of the host)
        ev3 = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(20)]
        for e in ev3:
            e[0].record()
            swa.swa_rope_keys(p, k, start, k_rot)
            e[1].record()
            swa.swa_prefill_attention(p, q, k_rot, v, None, None, start, out, lse)
            e[2].record()
            swa.swa_cache_write(p, k, v, start, kc, vc)
            e[3].record()
        torch.cuda.synchronize()
        rope_ms = sum(e[0].elapsed_time(e[1]) for e in ev3) / len(ev3)
        write_ms = sum(e[2].elapsed_time(e[3]) for e in ev3) / len(ev3)
        # key rotation: every key read and its rotation written; cache write:
        # the surviving last W tokens' k and v read and stored (digest
        # "쓰기(write) 단계": one writer per slot); the fused pass: k read
        # once and rotated once, v of the survivors read
        row = Hkv * D * 2
        rope_bytes = 2 * N * row
        write_bytes = 2 * 2 * min(N, W) * row
        both_bytes = 2 * N * row + 3 * min(N, W) * row
        prof_us = profiled_avg_us("prefill_bf16_d128_g4_kernel.prefill_n8192_w4096",
                                  ["swa_prefill.hip", "swa_device.hpp"])
        result.update({
            "value": round(flops2 / (ms_step * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4), "prewarm_s": args.prewarm_s,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": wl.name, "batch": 1, "seq_len": N, "window": W,
                       "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "rope_theta": wl.rope_theta,
                       "step": "rope_keys_cache_write + prefill_attention (the layer's first chunk: "
                               "its attention reads no cache)",
                       "algorithmic_flops_per_step": flops2, "key_pairs": pairs2},
            "roofline": {"bound": "mfma", "kernel": "prefill_bf16_d128_g4_kernel",
                         "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                         "traffic": profiled_traffic("prefill_bf16_d128_g4_kernel.prefill_n8192_w4096",
                                                     ["swa_prefill.hip", "swa_device.hpp"]),
                         "algorithmic_bytes": N * Hq * D * 2 * 2 + 2 * N * Hkv * D * 2 + Hq * N * 4,
                         "avg_kernel_ms": round(attn_ms, 4),
                         "median_kernel_ms": round(attn_times[len(attn_times) // 2], 4),
                         "min_kernel_ms": round(attn_times[0], 4),
                         "timing": "HIP events around each attention launch in the timed region",
                         "rocprof_avg_us": prof_us,
                         "frac_from_rocprof_avg": (round(flops2 / (prof_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
                                                   if prof_us else None)},
            "small_kernels": {
                "rope_keys_cache_write": {"kernel": "cache_write_kernel (both mode), in the step",
                                          "avg_us": round(both_ms * 1e3, 2), "bytes": both_bytes,
                                          "gbps": round(both_bytes / (both_ms * 1e-3) / 1e9, 1),
                                          "frac_hbm_peak": round(both_bytes / (both_ms * 1e-3) / 1e9
                                                                 / PEAK_HBM_GBPS, 4), "bound": "hbm"},
                "key_rotation": {"kernel": "cache_write_kernel (dense mode)", "avg_us": round(rope_ms * 1e3, 2),
                                 "bytes": rope_bytes, "gbps": round(rope_bytes / (rope_ms * 1e-3) / 1e9, 1),
                                 "frac_hbm_peak": round(rope_bytes / (rope_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
                "cache_write": {"kernel": "cache_write_kernel", "avg_us": round(write_ms * 1e3, 2),
                                "bytes": write_bytes, "gbps": round(write_bytes / (write_ms * 1e-3) / 1e9, 1),
                                "frac_hbm_peak": round(write_bytes / (write_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                                "bound": "hbm"},
                "timing": "HIP events (launch included): the fused pass in the timed region, as the "
                          "interval between attention launches; the two passes it replaces in 20 "
                          "three-launch steps after it, events around each"},
            "wall_s_timed_region": round(wall, 4),
        })

    # ------------------------------------------------------------------
    # decode: 64 sequences, positions U[1, 32768], 256 steps
    # ------------------------------------------------------------------
    if args.only in ("decode", "all"):
        wl4 = synth.workload(4)
        B4, S4 = wl4.batch, wl4.n_slots
        p4 = swa.make_params(B4, Hq, Hkv, D, wl4.window, 0, 0.0, wl4.rope_theta, bf)
        g = torch.Generator(device=dev).manual_seed(4004)
        kc4 = torch.randn((B4, S4, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        vc4 = torch.randn((B4, S4, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        T = args.decode_steps
        qs = torch.randn((T, B4, Hq, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        ks = torch.randn((T, B4, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        vs = torch.randn((T, B4, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        p0 = synth.positions(4, B4, wl4.pos_lo, wl4.pos_hi).to(torch.int64)
        pos = (p0[None, :] + torch.arange(T)[:, None]).to(torch.int32).to(dev)    # [T][B]
        o4 = torch.empty((B4, Hq, D), dtype=bf, device=dev)
        l4 = torch.empty((B4, Hq), dtype=torch.float32, device=dev)
        ws4 = torch.empty(swa.swa_decode_workspace_bytes(p4), dtype=torch.uint8, device=dev)
        row_bytes = Hkv * D * 2 * 2                       # K and V of one slot
        kv_bytes = sum(int(min(int(pp) + 1, S4)) * row_bytes for pp in pos.cpu().flatten())
        qo_bytes = T * B4 * Hq * D * 2 * 2
        write_bytes = T * B4 * Hkv * D * 2 * 2 * 2        # read k,v + write k,v
        dec_bytes = kv_bytes + qo_bytes

        def dstep(s, ev=None):
            # one launch: the new entry into slot(pos), then attention
            if ev is not None:
                ev[0].record()
            swa.swa_decode_step(p4, qs[s], ks[s], vs[s], kc4, vc4, pos[s], o4, l4, ws4)
            if ev is not None:
                ev[1].record()

        prewarm(lambda: [dstep(s) for s in range(min(8, T))], args.prewarm_s, torch)
        for s in range(min(8, T)):
            dstep(s)
        torch.cuda.synchronize()
        kc4_0, vc4_0 = kc4.clone(), vc4.clone()
        # the T steps back to back, events only around the loop (per-step
        # events would sit between the launches): the loop's throughput
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for s in range(T):
            dstep(s)
        t1.record()
        torch.cuda.synchronize()
        total_ms = t0.elapsed_time(t1)
        # the same steps from the same cache state, events around each call
        kc4.copy_(kc4_0)
        vc4.copy_(vc4_0)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(T)]
        for s in range(T):
            dstep(s, evs[s])
        torch.cuda.synchronize()
        dec_times = sorted(a.elapsed_time(b) for a, b in evs)
        dec_ms = sum(dec_times)
        dec_achieved = (dec_bytes + write_bytes) / (dec_ms * 1e-3) / 1e9
        # the same 256 steps again, from the same cache state, with the
        # Infinity Cache (MALL, 256 MB) flushed before each step by a 1 GiB fill
        kc4.copy_(kc4_0)
        vc4.copy_(vc4_0)
        del kc4_0, vc4_0
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(T)]
        for s in range(T):
            flush.fill_(s & 255)
            dstep(s, evf[s])
        torch.cuda.synchronize()
        del flush
        fl_ms = sum(a.elapsed_time(b) for a, b in evf)
        fl_gbps = (dec_bytes + write_bytes) / (fl_ms * 1e-3) / 1e9
        result["decode"] = {
            "workload": wl4.name, "batch": B4, "steps": T, "window": wl4.window,
            "value": round((dec_bytes + write_bytes) / (total_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(total_ms / T, 4),
            "step": "decode_step (cache write + attention, one launch)",
            "timing": "value: the steps back to back, events around the loop; roofline: events around "
                      "each call, a second pass of the same steps from the same cache state",
            "algorithmic_bytes_per_step": round((dec_bytes + write_bytes) / T),
            "roofline": {"bound": "hbm", "kernel": "decode_bf16_d128_g4_kernel",
                         "achieved": round(dec_achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(dec_achieved / PEAK_HBM_GBPS, 4),
                         "traffic": profiled_traffic("decode_bf16_d128_g4_kernel.decode_b64_w4096",
                                                     ["swa_decode.hip", "swa_passes.hpp", "swa_device.hpp"]),
                         "algorithmic_bytes": round((dec_bytes + write_bytes) / T),
                         "avg_call_ms": round(dec_ms / T, 4),
                         "median_call_ms": round(dec_times[len(dec_times) // 2], 4),
                         "bytes": "valid K/V slots read once + Q + O + new k/v read and stored"},
            "mall_flushed": {"avg_call_ms": round(fl_ms / T, 4), "gbps": round(fl_gbps, 1),
                             "frac": round(fl_gbps / PEAK_HBM_GBPS, 4),
                             "note": "same steps from the same cache state, a 1 GiB fill before each call"},
        }
        del kc4, vc4, qs, ks, vs

    # ------------------------------------------------------------------
    # context: chunked SWA vs full causal at 16K, sink streaming decode
    # ------------------------------------------------------------------
    if not args.no_context and args.only in ("chunked", "sink"):
        result["context"] = context_timings(swa, synth, torch, dev, args.only)
    if not args.no_context and args.only == "dilated":
        result["context"] = {"dilated_windows": dilated_windows(swa, synth, torch, dev)}
    if not args.no_context and args.only == "mixed":
        result["context"] = {"varlen_mixed_batch": varlen_mixed(swa, synth, torch, dev)}
    if not args.no_context and args.only == "all":
        result["context"] = context_timings(swa, synth, torch, dev)
        result["context"]["decode_32_layers"] = decode_layers(swa, synth, torch, dev)
        result["context"]["varlen_mixed_batch"] = varlen_mixed(swa, synth, torch, dev)
        result["context"]["vanilla_vs_swa_16k"] = vanilla_vs_swa_decode(swa, synth, torch, dev,
                                                                        result["context"])
        result["context"]["decode_small_batches"] = decode_small_batches(swa, synth, torch, dev)
        result["context"]["tiny_fp32_prefill"] = tiny_fp32(swa, synth, torch, dev)
        result["context"]["dilated_windows"] = dilated_windows(swa, synth, torch, dev)

    # ------------------------------------------------------------------
    # CPU baseline: the oracle on a bounded sample of the prefill workload
    # ------------------------------------------------------------------
    if not args.no_cpu_baseline and args.only in ("prefill", "all"):
        result["cpu_baseline"] = cpu_baseline(q.cpu(), k.cpu(), v.cpu(), W, wl.rope_theta, args.cpu_seconds)

    if args.only == "all":
        result["device"] = device_info(torch, dev)
    result["host"] = {"cpu": cpu_model(), "os_cpu_count": os.cpu_count(),
                      "affinity_cpus": len(os.sched_getaffinity(0))}
    print(json.dumps(result), flush=True)


def device_info(torch, dev, nbytes=1 << 30, reps=10):
    """The GPU as the runtime reports it, the matrix peak its CU count and
    clock give, and a measured device-to-device copy: the achievable HBM line
    the decode and write rates can also be read against."""
    props = torch.cuda.get_device_properties(dev)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "hbm_bytes": props.total_memory}
    clock_khz = None
    try:   # hipDeviceAttributeClockRate (kHz) from the HIP runtime torch already loaded
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        attr = 5   # hipDeviceAttributeClockRate
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev.index or 0) == 0 and v.value > 0:
            clock_khz = v.value
    except OSError:
        pass
    if clock_khz:
        info["max_clock_mhz"] = clock_khz / 1e3
        # bf16 dense MFMA: 4096 flops per clock per CU
        info["bf16_peak_at_max_clock_tflops"] = round(props.multi_processor_count * clock_khz * 1e3 * 4096 / 1e12, 1)
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    prewarm(lambda: dst.copy_(src), 0.1, torch)
    times = []
    for _ in range(5):
        # back to back, a copy in flight before the first event
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        dst.copy_(src)
        a.record()
        for _ in range(reps):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / reps)
    times.sort()
    med = times[len(times) // 2]
    info["copy_1gib"] = {"ms": round(med, 4), "gbps": round(2 * nbytes / (med * 1e-3) / 1e9, 1),
                         "frac_hbm_peak": round(2 * nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                         "note": "device-to-device copy of 1 GiB (the runtime's copy kernel), bytes read + "
                                 "written, median of 5 runs of 10 back-to-back copies: the streaming rate "
                                 "a plain copy reaches on this box"}
    del src, dst
    return info


def decode_layers(swa, synth, torch, dev, n_layers=32, tokens=16):
    """A decode token through a stack of n_layers attention layers, each with
    its own rolling K/V buffers (the batched-decode shape: 64 sequences,
    window 4096, positions U[1, 32768]): per layer one swa_decode_step
    (cache write + attention).  Reports the per-token latency of the stack
    and the KV memory of the rolling buffers against full caches."""
    bf = torch.bfloat16
    wl = synth.workload(4)
    B, Hq, Hkv, D, W = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    p = swa.make_params(B, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
    g = torch.Generator(device=dev).manual_seed(4032)
    kcs, vcs = [], []
    for _ in range(n_layers):
        kcs.append(torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf))
        vcs.append(torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf))
    qs = torch.randn((n_layers, B, Hq, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    ks = torch.randn((n_layers, B, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    vs = torch.randn((n_layers, B, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    p0 = synth.positions(4, B, wl.pos_lo, wl.pos_hi).to(torch.int64)
    pos = (p0[None, :] + torch.arange(tokens + 4)[:, None]).to(torch.int32).to(dev)
    out = torch.empty((B, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(swa.swa_decode_workspace_bytes(p), dtype=torch.uint8, device=dev)

    def token(t):
        for layer in range(n_layers):
            swa.swa_decode_step(p, qs[layer], ks[layer], vs[layer], kcs[layer], vcs[layer], pos[t],
                                out, lse, ws)

    for t in range(4):
        token(t)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for t in range(4, 4 + tokens):
        token(t)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / tokens
    slot_bytes = Hkv * D * 2 * 2                      # K and V of one position, one layer
    read = sum(min(int(x) + 1, W) for x in pos[4:4 + tokens].cpu().flatten()) * slot_bytes * n_layers
    moved = read / tokens + n_layers * B * (Hq * D * 2 * 2 + Hkv * D * 2 * 2 * 2)
    rolling = n_layers * B * W * slot_bytes
    full_now = n_layers * sum(int(x) + 1 for x in pos[3 + tokens].cpu()) * slot_bytes
    full_32k = n_layers * B * 32768 * slot_bytes
    res = {
        "workload": f"decode_b{B}_w{W}_x{n_layers}_layers", "layers": n_layers, "tokens": tokens,
        "ms_per_token": round(ms, 4), "ms_per_layer": round(ms / n_layers, 4),
        "gbps": round(moved / (ms * 1e-3) / 1e9, 1),
        "step": "per layer one decode_step (cache write + attention)",
        "kv_bytes_rolling": rolling,
        "kv_bytes_full_cache_at_current_positions": full_now,
        "kv_bytes_full_cache_at_32k": full_32k,
        "full_32k_over_rolling": round(full_32k / rolling, 3),
    }
    del kcs, vcs
    return res


def varlen_mixed(swa, synth, torch, dev, n_prefill=4, chunk=1024, reps=10):
    """One step of a mixed batch of 64 sequences at the batched-decode shape
    (window 4096, full windows): n_prefill sequences prefill a chunk of
    `chunk` tokens, the others decode one token.  As one varlen call (key
    rotation + attention, then the cache write) against the fixed-length
    calls it replaces (prefill chunk + cache write, then decode steps)."""
    bf = torch.bfloat16
    wl = synth.workload(4)
    B, Hq, Hkv, D, W = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    nd = B - n_prefill
    lens = [chunk] * n_prefill + [1] * nd
    T = sum(lens)
    p = swa.make_params(B, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
    pp = swa.make_params(n_prefill, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
    pd = swa.make_params(nd, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
    g = torch.Generator(device=dev).manual_seed(4064)
    kc = torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    vc = torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    q = torch.randn((T, Hq, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    k = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    v = torch.randn((T, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
    st = synth.positions(4, B, W, 32768).to(torch.int32).to(dev)   # every window full
    out = torch.empty((T, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    ws = torch.empty(swa.swa_prefill_varlen_workspace_bytes(p, lens), dtype=torch.uint8, device=dev)
    P = n_prefill * chunk
    qp, kp, vp = (x[:P].reshape(n_prefill, chunk, *x.shape[1:]) for x in (q, k, v))
    qd, kd, vd = q[P:], k[P:], v[P:]
    outp = torch.empty((n_prefill, chunk, Hq, D), dtype=bf, device=dev)
    lsep = torch.empty((n_prefill, Hq, chunk), dtype=torch.float32, device=dev)
    wsp = torch.empty(swa.swa_prefill_workspace_bytes(pp, chunk), dtype=torch.uint8, device=dev)
    outd = torch.empty((nd, Hq, D), dtype=bf, device=dev)
    lsed = torch.empty((nd, Hq), dtype=torch.float32, device=dev)
    wsd = torch.empty(swa.swa_decode_workspace_bytes(pd), dtype=torch.uint8, device=dev)

    wss = torch.empty(swa.swa_step_varlen_workspace_bytes(p, lens), dtype=torch.uint8, device=dev)

    def one_call():
        swa.swa_prefill_chunk_varlen(p, q, k, v, kc, vc, st, lens, out, lse, ws)
        swa.swa_cache_write_varlen(p, k, v, st, lens, kc, vc)

    def step():
        swa.swa_step_varlen(p, q, k, v, kc, vc, st, lens, out, lse, wss)

    def separate():
        swa.swa_prefill_chunk(pp, qp, kp, vp, kc[:n_prefill], vc[:n_prefill], st[:n_prefill], outp, lsep, wsp)
        swa.swa_cache_write(pp, kp, vp, st[:n_prefill], kc[:n_prefill], vc[:n_prefill])
        swa.swa_decode_step(pd, qd, kd, vd, kc[n_prefill:], vc[n_prefill:], st[n_prefill:], outd, lsed, wsd)

    def timeit(fn):
        # a call in flight when the first event is recorded, so that the GPU
        # does not wait for the host's first launch: back-to-back calls
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        fn()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # the three paths in turn, five rounds after a prewarm of all three: the
    # median of each (the clock drifts over a run; turns keep it fair)
    prewarm(lambda: (one_call(), step(), separate()), 0.2, torch)
    times = {"one": [], "step": [], "sep": []}
    for _ in range(5):
        times["one"].append(timeit(one_call))
        times["step"].append(timeit(step))
        times["sep"].append(timeit(separate))
    ms_one, ms_step, ms_sep = (sorted(times[x])[2] for x in ("one", "step", "sep"))
    pairs = n_prefill * chunk * W + nd * W
    res = {
        "workload": f"mixed_b{B}_{n_prefill}x{chunk}_prefill_{nd}_decode_w{W}",
        "lens": f"{n_prefill} x {chunk} + {nd} x 1", "tokens": T,
        "ms_step_varlen": round(ms_step, 4),
        "ms_prefill_chunk_varlen_and_cache_write_varlen": round(ms_one, 4),
        "ms_fixed_length_calls": round(ms_sep, 4),
        "tflops_step_varlen": round(attn_flops(pairs) / (ms_step * 1e-3) / 1e12, 1),
        "step": "step_varlen (one call: equal-length chunks on the fixed-length prefill kernel, one-token "
                "sequences on the decode kernel with its fused cache write) vs prefill_chunk_varlen + "
                "cache_write_varlen vs prefill_chunk + cache_write + decode_step",
        "timing": "median of 5 turns of the three paths, 10 back-to-back calls each (one more in flight "
                  "before the first event), HIP events",
    }
    del kc, vc
    return res


def vanilla_vs_swa_decode(swa, synth, torch, dev, ctx16, B=64, steps=64, n_gen=256):
    """Decode at 16K context, full cache (window 16384 = every position: plain
    causal attention) against the 4096-slot rolling buffer, 64 sequences;
    with the 16K prefill timings, the time of prefilling 16K tokens and
    generating n_gen more, both ways."""
    bf = torch.bfloat16
    wl = synth.workload(3)
    N, Hq, Hkv, D = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    g = torch.Generator(device=dev).manual_seed(3016)
    res = {}
    for name, W in (("swa", wl.window), ("full", N)):
        p = swa.make_params(B, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
        kc = torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        vc = torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        q = torch.randn((B, Hq, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        k = torch.randn((B, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        v = torch.randn((B, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        out = torch.empty((B, Hq, D), dtype=bf, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        ws = torch.empty(swa.swa_decode_workspace_bytes(p), dtype=torch.uint8, device=dev)
        # positions 16384 - steps .. 16383: the last tokens of a 16K context
        pos = [torch.full((B,), N - steps + s, dtype=torch.int32, device=dev) for s in range(steps)]
        for s in range(4):
            swa.swa_decode_step(p, q, k, v, kc, vc, pos[s], out, lse, ws)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for s in range(steps):
            swa.swa_decode_step(p, q, k, v, kc, vc, pos[s], out, lse, ws)
        b.record()
        torch.cuda.synchronize()
        res[name] = a.elapsed_time(b) / steps
        del kc, vc
    swa_total = ctx16["chunked_swa_prefill"]["ms"] + n_gen * res["swa"]
    full_total = ctx16["full_causal_prefill"]["ms"] + n_gen * res["full"]
    return {
        "batch": B, "context": N, "window": wl.window,
        "ms_per_decode_step_swa": round(res["swa"], 4), "ms_per_decode_step_full": round(res["full"], 4),
        "decode_full_over_swa_time": round(res["full"] / res["swa"], 3),
        "note": f"end to end = the 16K prefill (batch 1) + {n_gen} decode steps of the batch",
        "end_to_end_ms_swa": round(swa_total, 3), "end_to_end_ms_full": round(full_total, 3),
        "end_to_end_full_over_swa_time": round(full_total / swa_total, 3),
    }


def dilated_windows(swa, synth, torch, dev, dils=(2, 4), steps=64):
    """The dilated sliding window (keys i, i-d, i-2d, ... inside the W span) at
    the headline prefill shape (8192 tokens, W = 4096, no sinks: the fast
    kernel per residue class) and at the batched-decode shape (64 sequences,
    full windows: the fast decode over the window's keys)."""
    bf = torch.bfloat16
    wl = synth.workload(2)
    N, Hq, Hkv, D, W = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    g = torch.Generator(device=dev).manual_seed(2202)
    q = torch.randn((1, N, Hq, D), generator=g, device=dev).to(bf)
    k = torch.randn((1, N, Hkv, D), generator=g, device=dev).to(bf)
    v = torch.randn((1, N, Hkv, D), generator=g, device=dev).to(bf)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((1, N, Hq, D), dtype=bf, device=dev)
    lse = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
    res = {"prefill_workload": wl.name, "decode_workload": "decode_b64_w4096 (full windows)"}
    wl4 = synth.workload(4)
    B = wl4.batch
    kc = torch.randn((B, W, Hkv, D), generator=g, device=dev).to(bf)
    vc = torch.randn((B, W, Hkv, D), generator=g, device=dev).to(bf)
    qd = torch.randn((B, Hq, D), generator=g, device=dev).to(bf)
    kd = torch.randn((B, Hkv, D), generator=g, device=dev).to(bf)
    vd = torch.randn((B, Hkv, D), generator=g, device=dev).to(bf)
    od = torch.empty((B, Hq, D), dtype=bf, device=dev)
    ld = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    # full windows at each sequence's own position (equal positions would put
    # every sequence's reads at the same cache offsets at the same time)
    p0 = synth.positions(4, B, W, 32768).to(torch.int64)
    pos = [(p0 + s).to(torch.int32).to(dev) for s in range(steps)]
    for d in dils:
        p = swa.make_params(1, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf, d)
        # (the key rotation is common to every window; the attention is timed)
        kr = swa.swa_rope_keys(p, k, st)
        ms = timeit(lambda: swa.swa_prefill_attention(p, q, kr, v, None, None, st, out, lse), torch, 10)
        pairs = sum(min(-(-W // d), i // d + 1) for i in range(N))
        pd = swa.make_params(B, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf, d)
        ws = torch.empty(swa.swa_decode_workspace_bytes(pd), dtype=torch.uint8, device=dev)
        t = {"s": 0}

        def dstep():
            swa.swa_decode_step(pd, qd, kd, vd, kc, vc, pos[t["s"] % steps], od, ld, ws)
            t["s"] += 1

        dms = timeit(dstep, torch, steps)
        dbytes = B * (-(-W // d)) * Hkv * D * 2 * 2 + B * Hq * D * 2 * 2 + B * Hkv * D * 2 * 2 * 2
        res[f"d{d}"] = {
            "prefill_ms": round(ms, 4), "prefill_key_pairs": pairs,
            "prefill_tflops": round(attn_flops(pairs) / (ms * 1e-3) / 1e12, 1),
            "prefill_frac_bf16_peak": round(attn_flops(pairs) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "decode_ms_per_step": round(dms, 4), "decode_bytes": dbytes,
            "decode_gbps": round(dbytes / (dms * 1e-3) / 1e9, 1),
            "decode_frac_hbm_peak": round(dbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        }
    res["step"] = ("prefill_attention (rotated keys given) and decode_step (cache write + attention) with "
                   "a dilated window: keys at distances 0, d, 2d, ... inside the W span")
    del kc, vc
    return res


def tiny_fp32(swa, synth, torch, dev, reps=50):
    """The tiny float32 prefill (batch 1, N = 256, 4 query / 1 KV head,
    head_dim 64, scale 1/8, no RoPE) at W = 64 and W = 256 (full causal):
    absolute time of one swa_prefill_chunk call (parity workload; launch-bound)."""
    wl = synth.workload(1)
    N, Hq, Hkv, D = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    f32 = torch.float32
    q = synth.normal((1, N, Hq, D), 1, "q", dtype=f32).to(dev)
    k = synth.normal((1, N, Hkv, D), 1, "k", dtype=f32).to(dev)
    v = synth.normal((1, N, Hkv, D), 1, "v", dtype=f32).to(dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    res = {"workload": wl.name}
    for W in (wl.window, wl.extra["full_window"]):
        p = swa.make_params(1, Hq, Hkv, D, W, 0, wl.scale, 0.0, f32)
        out = torch.empty((1, N, Hq, D), dtype=f32, device=dev)
        lse = torch.empty((1, Hq, N), dtype=f32, device=dev)
        ws = torch.empty(swa.swa_prefill_workspace_bytes(p, N), dtype=torch.uint8, device=dev)
        ms = timeit(lambda: swa.swa_prefill_chunk(p, q, k, v, None, None, st, out, lse, ws), torch, reps)
        pairs = band_pairs(N, W)
        res[f"w{W}"] = {"us_per_call": round(ms * 1e3, 2), "key_pairs": pairs,
                        "gflops": round(4 * D * Hq * pairs / (ms * 1e-3) / 1e9, 2)}
    res["step"] = "prefill_chunk (key copy + float32 attention, generic kernel)"
    return res


def decode_small_batches(swa, synth, torch, dev, batches=(1, 8), steps=64):
    """Per-token latency of one decode step (swa_decode_step: cache write +
    split-K attention + combine) at small batches, full windows of 4096."""
    bf = torch.bfloat16
    wl = synth.workload(4)
    Hq, Hkv, D, W = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    g = torch.Generator(device=dev).manual_seed(4100)
    res = {}
    for B in batches:
        p = swa.make_params(B, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
        kc = torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        vc = torch.randn((B, W, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        q = torch.randn((B, Hq, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        k = torch.randn((B, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        v = torch.randn((B, Hkv, D), generator=g, device=dev, dtype=torch.float32).to(bf)
        out = torch.empty((B, Hq, D), dtype=bf, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        ws = torch.empty(swa.swa_decode_workspace_bytes(p), dtype=torch.uint8, device=dev)
        pos = [torch.full((B,), 10000 + s, dtype=torch.int32, device=dev) for s in range(steps)]

        def run():
            for s in range(steps):
                swa.swa_decode_step(p, q, k, v, kc, vc, pos[s], out, lse, ws)

        def timed(fn):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / steps * 1e3

        run()
        torch.cuda.synchronize()
        us_eager = timed(run)
        # the same steps captured once in a graph (no host work per step)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            run()
        graph.replay()
        torch.cuda.synchronize()
        us = timed(graph.replay)
        nbytes = B * W * Hkv * D * 2 * 2
        res[f"b{B}"] = {"us_per_step_graph": round(us, 2), "gbps_graph": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "us_per_step_eager_launches": round(us_eager, 2), "kv_bytes": nbytes}
        del graph, kc, vc
    res["note"] = ("4096-slot windows full; each step = decode_step (+ combine); graph: the steps captured "
                   "in one HIP graph and replayed; eager: one Python call per step (host-bound at batch 1)")
    return res


def context_timings(swa, synth, torch, dev, only="all"):
    """Chunked SWA prefill (4 x 4096 into a 4096-slot buffer) vs one full
    causal pass at N = 16384 ("chunked"), and the sink-streaming workload's
    decode rate and prefill chunk ("sink")."""
    ctx = {}
    if only in ("all", "chunked"):
        ctx.update(chunked_vs_full(swa, synth, torch, dev))
    if only in ("all", "sink"):
        ctx.update(sink_workload(swa, synth, torch, dev))
    return ctx


def timeit(fn, torch, reps=5, prewarm_s=0.1):
    """Mean ms of fn over reps back-to-back calls, timed with events after
    about prewarm_s seconds of untimed calls (the clocks rise over the first
    ~50 ms of load).  One untimed call is still in flight when the first
    event is recorded, so the GPU never waits for the host's first launch."""
    prewarm(fn, prewarm_s, torch)
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    fn()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def chunked_vs_full(swa, synth, torch, dev):
    bf = torch.bfloat16
    wl = synth.workload(3)
    N, Hq, Hkv, D, W, C = wl.seq_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.chunk
    g = torch.Generator(device=dev).manual_seed(3003)
    q = torch.randn((1, N, Hq, D), generator=g, device=dev).to(bf)
    k = torch.randn((1, N, Hkv, D), generator=g, device=dev).to(bf)
    v = torch.randn((1, N, Hkv, D), generator=g, device=dev).to(bf)
    p = swa.make_params(1, Hq, Hkv, D, W, 0, 0.0, wl.rope_theta, bf)
    kc = torch.zeros((1, W, Hkv, D), dtype=bf, device=dev)
    vc = torch.zeros_like(kc)
    ws = torch.empty(swa.swa_prefill_workspace_bytes(p, C), dtype=torch.uint8, device=dev)
    outc = torch.empty((1, C, Hq, D), dtype=bf, device=dev)
    lsec = torch.empty((1, Hq, C), dtype=torch.float32, device=dev)
    starts = [torch.tensor([c * C], dtype=torch.int32, device=dev) for c in range(N // C)]

    qs = [q[:, c * C:(c + 1) * C].contiguous() for c in range(N // C)]
    ks_ = [k[:, c * C:(c + 1) * C].contiguous() for c in range(N // C)]
    vs_ = [v[:, c * C:(c + 1) * C].contiguous() for c in range(N // C)]

    kr0 = torch.empty_like(ks_[0])

    def chunked_calls():
        # the first chunk reads no cache: its rotation and cache write are one
        # pass before its attention; the others read the cache before writing
        # it.  The chunks are W tokens long from position 0, so every start is
        # a multiple of W and the aligned entry reads the cache in slot order.
        swa.swa_rope_keys_cache_write(p, ks_[0], vs_[0], starts[0], kc, vc, kr0)
        swa.swa_prefill_attention(p, qs[0], kr0, vs_[0], None, None, starts[0], outc, lsec)
        for c in range(1, N // C):
            swa.swa_prefill_chunk_aligned(p, qs[c], ks_[c], vs_[c], kc, vc, starts[c], outc, lsec, ws)
            swa.swa_cache_write(p, ks_[c], vs_[c], starts[c], kc, vc)

    def chunked2():
        # the same chunks with each boundary's cache write (chunk c - 1) and
        # key rotation (chunk c) in one pass: a launch fewer per boundary
        swa.swa_rope_keys_cache_write(p, ks_[0], vs_[0], starts[0], kc, vc, kr0)
        swa.swa_prefill_attention(p, qs[0], kr0, vs_[0], None, None, starts[0], outc, lsec)
        swa.swa_prefill_chunk_aligned(p, qs[1], ks_[1], vs_[1], kc, vc, starts[1], outc, lsec, ws)
        for c in range(2, N // C):
            swa.swa_prefill_chunk_aligned_write_prev(p, ks_[c - 1], vs_[c - 1], starts[c - 1], qs[c], ks_[c],
                                                     vs_[c], kc, vc, starts[c], outc, lsec, ws)
        swa.swa_cache_write(p, ks_[-1], vs_[-1], starts[-1], kc, vc)

    def chunked_parts(reps=5):
        # the same loop with events around each call: where the loop's time
        # goes.  Chunks 1.. run the aligned entry (rotation + attention in one
        # call); their attention is that call less the rotation pass, timed
        # on its own (swa_rope_keys) in the same turn.
        kr = torch.empty_like(ks_[0])
        acc = {"key_rotation": 0.0, "attention": [0.0] * (N // C), "cache_write": 0.0}
        for _ in range(reps):
            evs = []
            for c in range(N // C):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
                e[0].record()
                if c == 0:
                    swa.swa_rope_keys_cache_write(p, ks_[c], vs_[c], starts[c], kc, vc, kr)
                else:
                    swa.swa_rope_keys(p, ks_[c], starts[c], kr)
                e[1].record()
                if c == 0:
                    swa.swa_prefill_attention(p, qs[c], kr, vs_[c], None, None, starts[c], outc, lsec)
                e[2].record()
                if c > 0:
                    swa.swa_prefill_chunk_aligned(p, qs[c], ks_[c], vs_[c], kc, vc, starts[c], outc, lsec, ws)
                e[3].record()
                if c > 0:
                    swa.swa_cache_write(p, ks_[c], vs_[c], starts[c], kc, vc)
                e[4].record()
                evs.append(e)
            torch.cuda.synchronize()
            for c, e in enumerate(evs):
                rot = e[0].elapsed_time(e[1])
                acc["key_rotation"] += rot / reps
                att = e[1].elapsed_time(e[2]) if c == 0 else e[2].elapsed_time(e[3]) - rot
                acc["attention"][c] += att / reps
                acc["cache_write"] += e[3].elapsed_time(e[4]) / reps
        return acc

    pf = swa.make_params(1, Hq, Hkv, D, N, 0, 0.0, wl.rope_theta, bf)
    wsf = torch.empty(swa.swa_prefill_workspace_bytes(pf, N), dtype=torch.uint8, device=dev)
    outf = torch.empty((1, N, Hq, D), dtype=bf, device=dev)
    lsef = torch.empty((1, Hq, N), dtype=torch.float32, device=dev)
    z = torch.zeros(1, dtype=torch.int32, device=dev)

    def full():
        swa.swa_prefill_chunk(pf, q, k, v, None, None, z, outf, lsef, wsf)

    # the two loops in turn, the median of five turns each (the clock drifts)
    turns = [(timeit(chunked2, torch), timeit(chunked_calls, torch)) for _ in range(5)]
    swa_ms = sorted(t[0] for t in turns)[2]
    calls_ms = sorted(t[1] for t in turns)[2]
    parts = chunked_parts()
    full_ms = timeit(full, torch)
    swa_flops = attn_flops(band_pairs(N, W))
    full_flops = attn_flops(band_pairs(N, N))
    attn_ms = sum(parts["attention"])
    ctx = {
        "chunked_swa_prefill": {"workload": wl.name, "ms": round(swa_ms, 4),
                                "tflops": round(swa_flops / (swa_ms * 1e-3) / 1e12, 1),
                                "step": "rope_keys_cache_write + prefill_attention (chunk 0), "
                                        "prefill_chunk_aligned (chunk 1), 2 x prefill_chunk_aligned_write_prev "
                                        "(chunk c-1's cache write and chunk c's key rotation in one pass), "
                                        "cache_write (chunk 3): chunks of W tokens from position 0, every "
                                        "start a multiple of W",
                                "ms_separate_calls": round(calls_ms, 4),
                                "separate_calls": "the same chunks with prefill_chunk_aligned + cache_write "
                                                  "for chunks 1..3",
                                "attention_ms_per_chunk": [round(x, 4) for x in parts["attention"]],
                                "attention_tflops": round(swa_flops / (attn_ms * 1e-3) / 1e12, 1),
                                "key_rotation_ms_total": round(parts["key_rotation"], 4),
                                "key_rotation_note": "chunk 0's entry is its fused rotation + cache write",
                                "cache_write_ms_total": round(parts["cache_write"], 4),
                                "breakdown_note": "events around each call of the separate-calls loop "
                                                  "(launch included); chunks 1..3: attention = "
                                                  "prefill_chunk_aligned less the rotation pass timed alone"},
        "full_causal_prefill": {"seq_len": N, "ms": round(full_ms, 4),
                                "tflops": round(full_flops / (full_ms * 1e-3) / 1e12, 1)},
        "full_over_swa_time": round(full_ms / swa_ms, 3),
        "pages_claim": "about 2x faster than vanilla attention at 16K tokens, W=4096 (no hardware stated)",
    }
    del q, k, v, outf, wsf
    return ctx


def sink_workload(swa, synth, torch, dev):
    """Sink streaming (B=16, 4 sinks + 4092 window): 256 decode steps with and
    without a MALL flush, and the 4096-token prefill chunk per sequence."""
    bf = torch.bfloat16
    g = torch.Generator(device=dev).manual_seed(3005)
    ctx = {}
    # sink streaming decode (B=16, 4 sinks + 4092 window): 256 steps
    wl5 = synth.workload(5)
    Hq, Hkv, D = wl5.n_q_heads, wl5.n_kv_heads, wl5.head_dim
    B, S = wl5.batch, wl5.n_slots
    p5 = swa.make_params(B, Hq, Hkv, D, wl5.window, wl5.n_sink, 0.0, wl5.rope_theta, bf)
    kc5 = torch.randn((B, S, Hkv, D), generator=g, device=dev).to(bf)
    vc5 = torch.randn((B, S, Hkv, D), generator=g, device=dev).to(bf)
    T = 256
    qs5 = torch.randn((T, B, Hq, D), generator=g, device=dev).to(bf)
    ks5 = torch.randn((T, B, Hkv, D), generator=g, device=dev).to(bf)
    vs5 = torch.randn((T, B, Hkv, D), generator=g, device=dev).to(bf)
    p0 = synth.positions(5, B, wl5.pos_lo, wl5.pos_hi).to(torch.int64)
    pos = (p0[None, :] + torch.arange(T)[:, None]).to(torch.int32).to(dev)
    o5 = torch.empty((B, Hq, D), dtype=bf, device=dev)
    l5 = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws5 = torch.empty(swa.swa_decode_workspace_bytes(p5), dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def run5(flush_each):
        # flushed: a 1 GiB fill before each step; warm: the steps back to back
        evs = []
        for s in range(T):
            if flush_each:
                flush.fill_(s & 255)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            swa.swa_decode_step(p5, qs5[s], ks5[s], vs5[s], kc5, vc5, pos[s], o5, l5, ws5)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / T

    run5(False)
    ms_flushed = run5(True)
    ms_warm = run5(False)
    bytes5 = B * S * Hkv * D * 2 * 2 + B * Hq * D * 2 * 2 + B * Hkv * D * 2 * 2 * 2
    # sink workload's prefill chunk: one 4096-token chunk per sequence after
    # the decode steps, against the rolling cache with its 4 sink slots
    C5 = wl5.chunk
    st5 = pos[T - 1] + 1
    q5c = torch.randn((B, C5, Hq, D), generator=g, device=dev).to(bf)
    k5c = torch.randn((B, C5, Hkv, D), generator=g, device=dev).to(bf)
    v5c = torch.randn((B, C5, Hkv, D), generator=g, device=dev).to(bf)
    o5c = torch.empty((B, C5, Hq, D), dtype=bf, device=dev)
    l5c = torch.empty((B, Hq, C5), dtype=torch.float32, device=dev)
    ws5c = torch.empty(swa.swa_prefill_workspace_bytes(p5, C5), dtype=torch.uint8, device=dev)

    def chunk5():
        swa.swa_prefill_chunk(p5, q5c, k5c, v5c, kc5, vc5, st5, o5c, l5c, ws5c)

    chunk_ms = timeit(chunk5, torch)
    chunk_pairs = sum(band_pairs(C5, wl5.window, int(x), wl5.n_sink) for x in st5.cpu().tolist())
    ctx["sink_chunk_prefill"] = {
        "workload": wl5.name, "batch": B, "chunk": C5, "ms": round(chunk_ms, 4),
        "flops": attn_flops(chunk_pairs),
        "tflops": round(attn_flops(chunk_pairs) / (chunk_ms * 1e-3) / 1e12, 1),
        "step": "prefill_chunk (key rotation + attention over cache and chunk)",
    }
    ctx["sink_decode"] = {
        "workload": wl5.name, "bytes_per_step": bytes5,
        "step": "decode_step (cache write + split attention + combine)",
        "ms_per_decode_mall_flushed": round(ms_flushed, 4),
        "gbps_mall_flushed": round(bytes5 / (ms_flushed * 1e-3) / 1e9, 1),
        "ms_per_decode_warm": round(ms_warm, 4),
        "gbps_warm_cache_resident": round(bytes5 / (ms_warm * 1e-3) / 1e9, 1),
        "note": "working set 256 MiB fits the 256 MB Infinity Cache; the flushed figure writes 1 GiB before each step",
    }
    return ctx


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(q, k, v, W, theta, target_s):
    """The fp64 oracle, untuned, on a bounded sample of query rows of the
    prefill workload; reported as algorithmic TFLOP/s on the host cores."""
    import numpy as np
    import oracle.swa_oracle as so

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:  # pragma: no cover
        blas_threads = 0
    q64 = q[0].to(dtype=__import__("torch").float64).numpy()
    k64 = k[0].to(dtype=__import__("torch").float64).numpy()
    v64 = v[0].to(dtype=__import__("torch").float64).numpy()
    N = q64.shape[0]
    rng = np.random.default_rng(0)
    order = rng.permutation(N)
    done = 0
    pairs = 0
    t0 = time.perf_counter()
    block = 128
    while done < N:
        rows = np.sort(order[done:done + block])
        cache = so.RollingCache(k64.shape[1], k64.shape[2], W)
        so.prefill_chunk(cache, q64, k64, v64, 0, theta, rows=rows)
        pairs += sum(min(int(r) + 1, W) for r in rows)
        done += len(rows)
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    flops = attn_flops(pairs)
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{done} of {N} query rows (random) of the n8192 w4096 prefill, fp64 NumPy, {el:.1f} s",
            "seconds": round(el, 2), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_threads": blas_threads, "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
