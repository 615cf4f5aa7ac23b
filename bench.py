#!/usr/bin/env python3
"""Benchmark of the masked flash-attention path on one MI355X.

One step = the whole path for one batch: mask description -> tile CSR -> schedule
(host, inside the library) -> metadata upload -> forward kernel, for the varlen
causal workload (16384 packed tokens in 8 documents, 16 heads, head dim 128,
bf16).  Q, K and V are resident in HBM before the timed region starts.

Printed: one JSON line with the effective forward TFLOPS (4 * d * unmasked pairs *
heads / step time), the forward kernel's roofline figures (HIP events on the launch
stream), the fp64 oracle timed on host cores for a bounded sample, and, unless
--quick, the other four workloads (KV-split + merge included) measured the same way.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_fwd_varlen_causal_t16384_h16_d128_hbm_traffic.md")
KERNEL_SOURCES = ("block_sparse_flash_csr_amd/csrc/attn_fwd.hip",
                  "block_sparse_flash_csr_amd/csrc/bsfa_internal.h",
                  "block_sparse_flash_csr_amd/csrc/schedule.cpp")


def kernel_digest() -> str:
    """sha256 over the sources that decide the forward kernel's memory traffic."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary, or None
    when the kernel sources have changed since those counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            fields = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
        if fields.get("kernel_source_sha256", "").strip() != kernel_digest():
            return None
        return int(fields["traffic_bytes_per_launch"].split()[0])
    except (OSError, KeyError, ValueError):
        return None


MFMA_PROFILE = os.path.join(ROOT, "profiles", "mfma_busy_and_stalls_default_workloads.md")


def measured_mfma_busy():
    """Percent of cycles the matrix cores were busy in the headline forward kernel
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) from the committed counter
    summary, or None when the kernel sources have changed since it was taken."""
    try:
        with open(MFMA_PROFILE) as f:
            fields = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
        if fields.get("kernel_source_sha256", "").strip() != kernel_digest():
            return None
        return float(fields["headline_forward_mfma_busy_pct"].split()[0])
    except (OSError, KeyError, ValueError):
        return None


MERGE_PROFILE = os.path.join(ROOT, "profiles", "merge_and_backward_hbm_traffic.md")


def measured_merge_traffic():
    """HBM bytes per launch of the merge kernel (8 partials x 8192 tokens x 32 heads) from
    the committed FETCH_SIZE / WRITE_SIZE summary, or None when attn_merge.hip changed."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "block_sparse_flash_csr_amd/csrc/attn_merge.hip"), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
        with open(MERGE_PROFILE) as f:
            fields = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith(" "))
        if fields.get("merge_kernel_source_sha256", "").strip() != digest:
            return None
        return int(fields["merge_traffic_bytes_per_launch"].split()[0])
    except (OSError, KeyError, ValueError):
        return None


COUNTERS_PROFILE = os.path.join(ROOT, "profiles", "attn_fwd_and_merge_all_workloads_counters.md")


def measured_workload_counters():
    """Per-workload MFMA busy %, L2 hit % and HBM bytes per launch of the forward (and the
    merge) from the committed counter summary; a workload's entry is left out once the
    sources of its kernel have changed since the counters were taken."""
    import hashlib
    out = {}
    try:
        with open(os.path.join(ROOT, "block_sparse_flash_csr_amd/csrc/attn_merge.hip"), "rb") as f:
            merge_digest = hashlib.sha256(f.read()).hexdigest()
        with open(COUNTERS_PROFILE) as f:
            lines = [line.rstrip("\n") for line in f]
    except OSError:
        return out
    fields = dict(line.split(":", 1) for line in lines if ":" in line and not line.startswith((" ", "|")))
    fwd_ok = fields.get("kernel_source_sha256", "").strip() == kernel_digest()
    merge_ok = fields.get("merge_kernel_source_sha256", "").strip() == merge_digest
    for key, val in fields.items():
        if not key.startswith("counters."):
            continue
        name = key[len("counters."):]
        if not (merge_ok if name.endswith("_merge") else fwd_ok):
            continue
        try:
            kv = dict(item.split("=", 1) for item in val.split())
            out[name] = {"mfma_busy_pct": float(kv["mfma_busy_pct"]), "l2_hit_pct": float(kv["l2_hit_pct"]),
                         "hbm_bytes_per_launch": int(kv["hbm_bytes_per_launch"])}
        except (KeyError, ValueError):
            continue
    return out


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def event_times(fn, reps, stream):
    """Per-launch durations (ms) of fn() measured with events on the launch stream."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def headline(args, api, W):
    """Varlen causal workload: timed steps of plan build + upload + forward."""
    import torch
    w = W.varlen_causal_t16384()
    q, k, v = api.to_device_bf16(w.q), api.to_device_bf16(w.k), api.to_device_bf16(w.v)
    stream = torch.cuda.current_stream()
    o = torch.empty((w.sq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.hq, w.sq), dtype=torch.float32, device="cuda")

    def make_plan():
        return api.Plan.from_varlen(w.cu_seqlens, w.hq, w.hkv, w.d, causal=True).upload(stream)

    # One plan built and uploaded per step, for the next step's batch (the host prepares
    # batch i+1's metadata while batch i runs); the forward runs on the plan the step
    # before uploaded, whose copy has finished by then, so the launch carries no
    # cross-stream wait.
    ahead = [make_plan()]

    def step():
        plan = ahead[0]
        ahead[0] = make_plan()
        api.attn_fwd(q, k, v, plan, w.scale, out=o, lse=lse, stream=stream)
        plan.close()     # device metadata freed stream-ordered after the kernel

    info = api.Plan.from_varlen(w.cu_seqlens, w.hq, w.hkv, w.d, causal=True).info()
    flops = 4.0 * w.d * info["pairs"] * w.hq

    # untimed: bring the GPU to its sustained clock, then the W warmup steps
    t_end = time.perf_counter() + args.prewarm_s
    while time.perf_counter() < t_end:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    t_host = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    host_ms = (t_host - t0) * 1e3 / args.steps   # host issue time per step (overlaps the GPU)
    ahead[0].close()

    # forward kernel alone, HIP events on its launch stream, inside the same process
    plan = api.Plan.from_varlen(w.cu_seqlens, w.hq, w.hkv, w.d, causal=True).upload(stream)
    kt = event_times(lambda: api.attn_fwd(q, k, v, plan, w.scale, out=o, lse=lse, stream=stream),
                     max(args.steps, 20), stream)
    kernel_ms = float(np.mean(kt))
    # the core clock the forward runs at (the published peak assumes 2.4 GHz)
    clock = gfx_clock(lambda: api.attn_fwd(q, k, v, plan, w.scale, out=o, lse=lse, stream=stream), 2.0)
    plan.close()
    return w, info, flops, ms_per_step, kernel_ms, host_ms, clock


def gfx_clock(fn, seconds):
    """GPU core clock while fn() runs back to back: the driver's GPU metrics table
    (current_gfxclks, MHz, one value per XCD) read through amdsmi every 10 ms over
    `seconds` of launches.  The table refreshes coarsely, so only the samples of the
    window's second half count.  None when amdsmi is not usable here."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception:
        return None
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
        h = None
        for x in handles:
            try:
                if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(x).split(":")[1], 16) == bus:
                    h = x
            except Exception:
                pass
        if h is None:
            if len(handles) != 1:
                return None
            h = handles[0]
        samples, stop = [], [False]

        def sampler():
            while not stop[0]:
                try:
                    c = amdsmi.amdsmi_get_gpu_metrics_info(h).get("current_gfxclks")
                    if isinstance(c, list):
                        vals = [v for v in c if isinstance(v, int) and 0 < v < 10000]
                        if vals:
                            samples.append((time.perf_counter(), vals))
                except Exception:
                    pass
                time.sleep(0.01)

        th = threading.Thread(target=sampler, daemon=True)
        t0 = time.perf_counter()
        th.start()
        while time.perf_counter() < t0 + seconds:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
        stop[0] = True
        th.join()
        late = [v for t, v in samples if t >= t0 + seconds / 2]
        n = min((len(v) for v in late), default=0)
        if not late or n == 0:
            return None
        per_xcd = np.mean(np.array([v[:n] for v in late], dtype=np.float64), axis=0)
        return {"mhz_mean": float(np.mean(per_xcd)), "mhz_per_xcd": [int(round(x)) for x in per_xcd],
                "samples": len(late)}
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def sustain(f, seconds):
    """Untimed launches of f for about `seconds`: the GPU clock ramps up over the first
    few hundred milliseconds of load, so every timed figure starts from the sustained
    clock, as the headline's pre-warm does."""
    import torch
    t_end = time.perf_counter() + seconds
    while True:
        for _ in range(4):
            f()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return


def gemm_reference(W, n=8192, reps=20, warm_s=1.0):
    """What dense bf16 matrix work reaches on this part in the same run: torch.mm of two
    contiguous n x n bf16 matrices (the vendor's tuned GEMM library), event-timed after
    warm_s seconds of untimed launches, with the core clock sampled while it runs.  A
    measured reference beside the attention kernel's fraction of the published peak; not
    part of the path."""
    import torch
    a = W.device_normal_bf16((n, n), 811)
    b = W.device_normal_bf16((n, n), 812)
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    f = lambda: torch.mm(a, b, out=c)
    sustain(f, warm_s)
    ms = float(np.median(event_times(f, reps, stream)))
    clock = gfx_clock(f, 2.0)
    tflops = 2.0 * n ** 3 / (ms * 1e-3) * 1e-12
    out = {"op": f"torch.mm bf16 {n}x{n} @ {n}x{n} (fp32 accumulation, bf16 output)",
           "ms": ms, "tflops": tflops, "frac_of_peak": tflops / PEAK_BF16_TFLOPS,
           "clock_mhz": None if clock is None else clock["mhz_mean"]}
    if clock is not None:
        out["frac_at_measured_clock"] = tflops / (PEAK_BF16_TFLOPS * clock["mhz_mean"] / 2400.0)
    del a, b, c
    torch.cuda.empty_cache()
    return out


def other_workloads(api, W, reps=10, warm_s=0.5):
    """Kernel-time figures of the remaining workloads (event-timed, plan prebuilt, each
    after warm_s seconds of untimed launches of the same call)."""
    import torch
    stream = torch.cuda.current_stream()
    out = {}
    counters = measured_workload_counters()   # committed rocprofv3 summary (digest-checked)
    for cfg in (1, 3, 4):
        w = W.WORKLOADS[cfg]()
        q, k, v = api.to_device_bf16(w.q), api.to_device_bf16(w.k), api.to_device_bf16(w.v)
        plan = api.plan_from_workload(w, stream=stream)
        info = plan.info()
        fl = 4.0 * w.d * info["pairs"] * w.hq
        o = torch.empty((w.sq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((w.hq, w.sq), dtype=torch.float32, device="cuda")
        f = lambda: api.attn_fwd(q, k, v, plan, w.scale, out=o, lse=lse, stream=stream)
        sustain(f, warm_s)
        ms = float(np.median(event_times(f, reps, stream)))
        out[w.name] = {"kernel_ms": ms, "tflops": fl / ms * 1e-9,
                       "frac_of_peak": fl / ms * 1e-9 / PEAK_BF16_TFLOPS,
                       "pairs_per_head": info["pairs"], "tiles_full": info["n_full"],
                       "tiles_partial": info["n_partial"]}
        ctr = counters.get(w.name)
        if ctr is not None:
            out[w.name].update(mfma_busy_pct=ctr["mfma_busy_pct"], l2_hit_pct=ctr["l2_hit_pct"],
                               hbm_bytes_per_launch=ctr["hbm_bytes_per_launch"],
                               hbm_gbs=ctr["hbm_bytes_per_launch"] / ms * 1e-6)
        # the same roofline figures as the headline's, for this workload's kernel launch
        out[w.name]["roofline"] = {
            "bound": "mfma", "achieved": fl / ms * 1e-9, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": fl / ms * 1e-9 / PEAK_BF16_TFLOPS, "kernel": f"attn_fwd_kernel<{w.d}>", "kernel_ms": ms,
            "flops_per_launch": fl,
            "algorithmic_bytes": w.sq * w.hq * (4 * w.d + 4) + w.sk * w.hkv * 4 * w.d,
            "traffic": None if ctr is None else ctr["hbm_bytes_per_launch"],
            "traffic_unit": "bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, copy-calibrated; "
                            "null once the kernel changed since the counters were taken)"}
        log(f"{w.name}: {ms:.3f} ms  {fl / ms * 1e-9:.1f} TFLOPS")
        plan.close()
        del q, k, v, o, lse
        torch.cuda.empty_cache()

    # Head dim 64 on the headline mask (not a reference workload): per admitted pair the
    # softmax's vector work is the same as at d = 128 and the matrix work half of it, so
    # this line shows how far the vector units bound the smaller head dim.
    w = W.varlen_causal_t16384(with_inputs=False)
    hd = 64
    q, k, v = (W.device_normal_bf16((w.sq, w.hq, hd), s) for s in (641, 642, 643))
    plan = api.Plan.from_slices(w.slices, w.sq, w.sk, w.hq, w.hkv, hd).upload(stream)
    info = plan.info()
    fl = 4.0 * hd * info["pairs"] * w.hq
    o = torch.empty((w.sq, w.hq, hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.hq, w.sq), dtype=torch.float32, device="cuda")
    f = lambda: api.attn_fwd(q, k, v, plan, 1.0 / np.sqrt(hd), out=o, lse=lse, stream=stream)
    sustain(f, warm_s)
    ms = float(np.median(event_times(f, reps * 2, stream)))
    name = "varlen_causal_t16384_docs8_h16_d64"
    out[name] = {"kernel_ms": ms, "tflops": fl / ms * 1e-9, "frac_of_peak": fl / ms * 1e-9 / PEAK_BF16_TFLOPS,
                 "pairs_per_head": info["pairs"],
                 "note": "not a reference workload: the headline mask at head dim 64 (vector-bound)"}
    ctr = counters.get(name)
    if ctr is not None:
        out[name].update(mfma_busy_pct=ctr["mfma_busy_pct"], l2_hit_pct=ctr["l2_hit_pct"],
                         hbm_bytes=ctr["hbm_bytes_per_launch"], hbm_gbs=ctr["hbm_bytes_per_launch"] / ms * 1e-6)
    log(f"{name}: {ms:.3f} ms  {fl / ms * 1e-9:.1f} TFLOPS")
    plan.close()
    del q, k, v, o, lse
    torch.cuda.empty_cache()

    # Backward at the varlen causal workload: one call runs the D kernel (D_i = sum_j P_ij
    # dP_ij by query tile), the dQ kernel (by query tile) and the dK/dV kernel (by key tile).
    # Algorithmic work is 5 products of 2*d flops per admitted pair (S, dP, dV, dK, dQ); the
    # kernels execute 9 (S and dP are recomputed by all three kernels instead of storing
    # P or using atomics).
    w = W.varlen_causal_t16384()
    q, k, v = api.to_device_bf16(w.q), api.to_device_bf16(w.k), api.to_device_bf16(w.v)
    g = api.to_device_bf16(W.random_grad(np.random.default_rng(2002), w.sq, w.hq, w.d))
    plan = api.plan_from_workload(w, stream=stream)
    info = plan.info()
    fl = 10.0 * w.d * info["pairs"] * w.hq
    o, lse = api.attn_fwd(q, k, v, plan, w.scale, stream=stream)
    dq = torch.empty((w.sq, w.hq, w.d), dtype=torch.float32, device="cuda")
    dk = torch.empty((w.sk, w.hkv, w.d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    delta = torch.empty_like(lse)
    f = lambda: api.attn_bwd(q, k, v, g, lse, plan, w.scale, dq=dq, dk=dk, dv=dv, delta=delta,
                             stream=stream)
    sustain(f, warm_s)
    ms = float(np.median(event_times(f, reps * 2, stream)))
    name = w.name + "_backward"
    out[name] = {"kernel_ms": ms, "tflops": fl / ms * 1e-9, "frac_of_peak": fl / ms * 1e-9 / PEAK_BF16_TFLOPS,
                 "flops_per_pair": 10 * w.d, "pairs_per_head": info["pairs"],
                 "note": "dQ, dK, dV (fp32) from LSE and dO; algorithmic flops = 2.5x the forward's"}
    log(f"{name}: {ms:.3f} ms  {fl / ms * 1e-9:.1f} TFLOPS (algorithmic)")
    # the same backward given the forward's fp32 O: D_i = dO_i . O_i inside the dQ kernel,
    # no D pass (two kernels)
    o32, _ = api.attn_fwd(q, k, v, plan, w.scale, stream=stream, out_dtype=torch.float32)
    f32 = lambda: api.attn_bwd(q, k, v, g, lse, plan, w.scale, dq=dq, dk=dk, dv=dv, delta=delta,
                               stream=stream, o=o32)
    sustain(f32, warm_s)
    ms32 = float(np.median(event_times(f32, reps * 2, stream)))
    out[name]["from_fp32_o"] = {"kernel_ms": ms32, "tflops": fl / ms32 * 1e-9,
                                "frac_of_peak": fl / ms32 * 1e-9 / PEAK_BF16_TFLOPS,
                                "note": "D from the forward's fp32 O (bsfa_attn_bwd_o32): dQ and dK/dV kernels only"}
    log(f"{name} from fp32 O: {ms32:.3f} ms  {fl / ms32 * 1e-9:.1f} TFLOPS (algorithmic)")
    torch.cuda.synchronize()
    plan.close()
    del q, k, v, g, o, o32, lse, dq, dk, dv, delta
    torch.cuda.empty_cache()

    # Mask compile: host plan creation (compile + column view + schedule) against the
    # device compiler's tile CSR (host pair listing, allocation, upload and kernels, wall
    # time to a finished CSR; events time the part on the stream).  Both take the slice
    # array in its C layout.
    mc = {}
    S = 524288
    cases = [("varlen_causal_t16384_docs8", W.varlen_causal_t16384(with_inputs=False).slices, 16384),
             ("causal_s524288", [(0, S, 0, S, 1)], S),
             ("strided_blocks_s524288", W.block_slices(W.strided_block_codes(S // 128, 8), 128, 128, S, S), S)]
    for name, sl, s_ in cases:
        sl = api.slice_array(sl)               # int32 [n, 5], the C layout, built untimed
        t0 = time.perf_counter()
        hp = api.Plan.from_slices(sl, s_, s_, 16, 16, 128)
        host_ms = (time.perf_counter() - t0) * 1e3
        nnz = hp.info()["nnz"]
        hp.close()
        wc = api.DeviceCsr(sl, s_, s_)          # warm (first-use costs: module loads, pools)
        wc.plan(16, 16, 128).close()
        wc.close()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        dc = api.DeviceCsr(sl, s_, s_, stream=stream)
        e1.record(stream)
        v = dc.view()
        dev_ms = (time.perf_counter() - t0) * 1e3
        assert v["nnz"] == nnz
        # a full plan (column view and schedule too) from the device CSR, until its device
        # image is complete
        t0 = time.perf_counter()
        dp = dc.plan(16, 16, 128)
        torch.cuda.synchronize()
        dplan_ms = dev_ms + (time.perf_counter() - t0) * 1e3
        dp.close()
        mc[name] = {"slices": len(sl), "nnz": nnz, "touches": v["touches"], "host_plan_ms": host_ms,
                    "device_csr_ms": dev_ms, "device_stream_ms": e0.elapsed_time(e1),
                    "plan_from_device_csr_ms": dplan_ms}
        log(f"mask compile {name}: host plan {host_ms:.1f} ms, device CSR {dev_ms:.2f} ms "
            f"(stream {e0.elapsed_time(e1):.2f} ms), plan from device CSR {dplan_ms:.1f} ms, nnz {nnz}")
        dc.close()
        if name.startswith("strided_blocks"):
            # the same mask as its block-code map (blocks = tiles), compiled on the device
            # without slices, and the host plan from the map
            codes = W.strided_block_codes(s_ // 128, 8)
            t0 = time.perf_counter()
            api.Plan.from_blocks(codes, 128, 128, s_, s_, 16, 16, 128).close()
            host_b_ms = (time.perf_counter() - t0) * 1e3
            wc = api.DeviceCsr.from_blocks(codes, s_, s_)
            wc.plan(16, 16, 128).close()
            wc.close()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            dc = api.DeviceCsr.from_blocks(codes, s_, s_, stream=stream)
            v = dc.view()
            dev_b_ms = (time.perf_counter() - t0) * 1e3
            assert v["nnz"] == nnz
            t0 = time.perf_counter()
            dp = dc.plan(16, 16, 128)
            torch.cuda.synchronize()
            dplan_b_ms = dev_b_ms + (time.perf_counter() - t0) * 1e3
            dp.close()
            dc.close()
            mc[name].update({"host_plan_from_block_map_ms": host_b_ms, "device_csr_from_block_map_ms": dev_b_ms,
                             "plan_from_device_block_map_ms": dplan_b_ms})
            log(f"mask compile {name} as a {codes.shape[0]}x{codes.shape[1]} block map: host plan {host_b_ms:.1f} ms, "
                f"device CSR {dev_b_ms:.2f} ms, plan from it {dplan_b_ms:.1f} ms")
    out["mask_compile"] = mc

    # Few query rows against a long context (a prefill chunk): 1 query tile x 32 heads is
    # 32 items for 512 workgroup slots, so the plan splits every row's key range into
    # parts whose partial results a second kernel merges inside the same call.
    sq, sk, hq, hkv, d = 128, 65536, 32, 8, 128
    rng = np.random.default_rng(6)
    qb, kb, vb = W.random_inputs(rng, sq, sk, hq, hkv, d)
    q, k, v = api.to_device_bf16(qb), api.to_device_bf16(kb), api.to_device_bf16(vb)
    plan = api.Plan.from_slices([(0, sq, 0, sk, 1)], sq, sk, hq, hkv, d).upload(stream)
    info = plan.info()
    fl = 4.0 * d * info["pairs"] * hq
    o = torch.empty((sq, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, sq), dtype=torch.float32, device="cuda")
    ws = api.workspace_for(plan)              # the split rows' partial results
    f = lambda: api.attn_fwd(q, k, v, plan, 1.0 / np.sqrt(d), out=o, lse=lse, workspace=ws, stream=stream)
    sustain(f, warm_s)
    ms = float(np.median(event_times(f, reps * 2, stream)))
    name = f"prefill_chunk_q{sq}_ctx{sk}_gqa{hq}x{hkv}_d{d}"
    out[name] = {"kernel_ms": ms, "tflops": fl / ms * 1e-9, "frac_of_peak": fl / ms * 1e-9 / PEAK_BF16_TFLOPS,
                 "pairs_per_head": info["pairs"], "units": info["n_units"], "split_rows": info["n_splits"],
                 "note": "not a reference workload; shows the in-call KV split (forward + part merge)"}
    log(f"{name}: {ms:.3f} ms  {fl / ms * 1e-9:.1f} TFLOPS ({info['n_units']} units, {info['n_splits']} split rows)")
    plan.close()
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()

    # KV split: 8 partial forwards over 8192-token KV chunks, then the merge
    w = W.kv_split_q8192()
    c, nc = w.extra["chunk"], w.extra["n_chunks"]
    q, k, v = api.to_device_bf16(w.q), api.to_device_bf16(w.k), api.to_device_bf16(w.v)
    plans = [api.Plan.from_slices(sl, c, c, w.hq, w.hkv, w.d).upload(stream)
             for sl in w.extra["chunk_slices"]]
    pairs = sum(p.info()["pairs"] for p in plans)
    fl = 4.0 * w.d * pairs * w.hq
    os_ = [torch.empty((c, w.hq, w.d), dtype=torch.bfloat16, device="cuda") for _ in range(nc)]
    ls_ = [torch.empty((w.hq, c), dtype=torch.float32, device="cuda") for _ in range(nc)]
    om = torch.empty((c, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
    lm = torch.empty((w.hq, c), dtype=torch.float32, device="cuda")

    def fwd_all():
        for t in range(nc):
            api.attn_fwd(q, k[t * c:(t + 1) * c], v[t * c:(t + 1) * c], plans[t], w.scale,
                         out=os_[t], lse=ls_[t], stream=stream)

    def merge():
        api.attn_merge(os_, ls_, out=om, lse=lm, stream=stream)

    sustain(lambda: (fwd_all(), merge()), warm_s)
    fwd_ms = float(np.median(event_times(fwd_all, reps, stream)))
    merge_ms = float(np.median(event_times(merge, reps * 2, stream)))
    merge_bytes = (nc + 1) * c * w.hq * (2 * w.d + 4)
    merge_traffic = measured_merge_traffic()    # HBM bytes per merge launch (counters)
    out[w.name] = {"forward_ms": fwd_ms, "merge_ms": merge_ms,
                   "forward_tflops": fl / fwd_ms * 1e-9,
                   "forward_frac_of_peak": fl / fwd_ms * 1e-9 / PEAK_BF16_TFLOPS,
                   "forward_plus_merge_tflops": fl / (fwd_ms + merge_ms) * 1e-9,
                   "merge_gbs": merge_bytes / merge_ms * 1e-6,
                   "merge_frac_of_hbm_peak": merge_bytes / merge_ms * 1e-6 / PEAK_HBM_GBS,
                   "merge_traffic": merge_traffic,
                   "merge_gbs_from_counters": None if merge_traffic is None else merge_traffic / merge_ms * 1e-6,
                   "pairs_per_head": pairs}
    ctr = counters.get(w.name)
    if ctr is not None:   # per chunk forward; a call runs nc of them
        out[w.name].update(forward_mfma_busy_pct=ctr["mfma_busy_pct"], forward_l2_hit_pct=ctr["l2_hit_pct"],
                           forward_hbm_bytes=nc * ctr["hbm_bytes_per_launch"],
                           forward_hbm_gbs=nc * ctr["hbm_bytes_per_launch"] / fwd_ms * 1e-6)
    log(f"{w.name}: fwd {fwd_ms:.3f} ms ({fl / fwd_ms * 1e-9:.1f} TFLOPS), merge {merge_ms:.3f} ms "
        f"({merge_bytes / merge_ms * 1e-6:.0f} GB/s)")
    # the same split with fp32 partial outputs (the chunk forwards write fp32 O, the merge
    # reads fp32 partials and writes the bf16 result)
    torch.cuda.synchronize()
    del os_
    os32 = [torch.empty((c, w.hq, w.d), dtype=torch.float32, device="cuda") for _ in range(nc)]

    def fwd_all32():
        for t in range(nc):
            api.attn_fwd(q, k[t * c:(t + 1) * c], v[t * c:(t + 1) * c], plans[t], w.scale,
                         out=os32[t], lse=ls_[t], stream=stream)

    def merge32():
        api.attn_merge(os32, ls_, out=om, lse=lm, stream=stream)

    sustain(lambda: (fwd_all32(), merge32()), warm_s)
    fwd32_ms = float(np.median(event_times(fwd_all32, reps, stream)))
    merge32_ms = float(np.median(event_times(merge32, reps * 2, stream)))
    merge32_bytes = nc * c * w.hq * (4 * w.d + 4) + c * w.hq * (2 * w.d + 4)
    out[w.name]["fp32_partials"] = {
        "forward_ms": fwd32_ms, "forward_tflops": fl / fwd32_ms * 1e-9, "merge_ms": merge32_ms,
        "merge_bytes": merge32_bytes, "merge_gbs": merge32_bytes / merge32_ms * 1e-6,
        "merge_frac_of_hbm_peak": merge32_bytes / merge32_ms * 1e-6 / PEAK_HBM_GBS}
    log(f"{w.name} with fp32 partials: fwd {fwd32_ms:.3f} ms ({fl / fwd32_ms * 1e-9:.1f} TFLOPS), merge "
        f"{merge32_ms:.3f} ms ({merge32_bytes / merge32_ms * 1e-6:.0f} GB/s)")
    torch.cuda.synchronize()
    del os32
    for p in plans:
        p.close()
    return out


COUNTER_ORDER = ((1, 20), (2, 20), (3, 20), (4, 5), (5, 5))


def counter_pass(api, W):
    """Fixed launch sequence for hardware-counter runs: for each workload in
    COUNTER_ORDER, its forward launched that many times back to back (workload 5: the
    8 chunk forwards and the merge, repeated), and after workload 2 its backward 5 times,
    one forward with fp32 output and the backward from that O 5 times, then the headline
    mask at head dim 64 20 times.
    No other forward or merge kernel runs, so a counter file maps onto workloads by
    dispatch order and kernel name."""
    import torch
    stream = torch.cuda.current_stream()
    for cfg, reps in COUNTER_ORDER:
        w = W.WORKLOADS[cfg]()
        q, k, v = api.to_device_bf16(w.q), api.to_device_bf16(w.k), api.to_device_bf16(w.v)
        torch.cuda.synchronize()
        if cfg == 5:
            c, nc = w.extra["chunk"], w.extra["n_chunks"]
            plans = [api.Plan.from_slices(sl, c, c, w.hq, w.hkv, w.d).upload(stream)
                     for sl in w.extra["chunk_slices"]]
            os_ = [torch.empty((c, w.hq, w.d), dtype=torch.bfloat16, device="cuda") for _ in range(nc)]
            ls_ = [torch.empty((w.hq, c), dtype=torch.float32, device="cuda") for _ in range(nc)]
            om = torch.empty((c, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
            lm = torch.empty((w.hq, c), dtype=torch.float32, device="cuda")
            for _ in range(reps):
                for t in range(nc):
                    api.attn_fwd(q, k[t * c:(t + 1) * c], v[t * c:(t + 1) * c], plans[t], w.scale,
                                 out=os_[t], lse=ls_[t], stream=stream)
                api.attn_merge(os_, ls_, out=om, lse=lm, stream=stream)
        else:
            plans = [api.plan_from_workload(w, stream=stream)]
            o = torch.empty((w.sq, w.hq, w.d), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((w.hq, w.sq), dtype=torch.float32, device="cuda")
            for _ in range(reps):
                api.attn_fwd(q, k, v, plans[0], w.scale, out=o, lse=lse, stream=stream)
        torch.cuda.synchronize()
        log(f"counter pass: workload {cfg} ({w.name}) x {reps}")
        if cfg == 2:
            # the backward of the headline workload (D, dQ and dK/dV kernels) x 5
            g = api.to_device_bf16(W.random_grad(np.random.default_rng(2002), w.sq, w.hq, w.d))
            for _ in range(5):
                api.attn_bwd(q, k, v, g, lse, plans[0], w.scale, stream=stream)
            torch.cuda.synchronize()
            log(f"counter pass: backward of workload {cfg} x 5")
            # the backward from the forward's fp32 O (dQ with D from O, dK/dV) x 5, after one
            # forward with fp32 output (a kernel of its own name)
            o32, lse32 = api.attn_fwd(q, k, v, plans[0], w.scale, stream=stream, out_dtype=torch.float32)
            for _ in range(5):
                api.attn_bwd(q, k, v, g, lse32, plans[0], w.scale, stream=stream, o=o32)
            torch.cuda.synchronize()
            log(f"counter pass: backward from the fp32 O of workload {cfg} x 5")
            del g, o32, lse32
            # the headline mask at head dim 64 x 20 (the benchmark's d = 64 line)
            q64, k64, v64 = (W.device_normal_bf16((w.sq, w.hq, 64), sd) for sd in (641, 642, 643))
            p64 = api.Plan.from_slices(w.slices, w.sq, w.sk, w.hq, w.hkv, 64).upload(stream)
            o64 = torch.empty((w.sq, w.hq, 64), dtype=torch.bfloat16, device="cuda")
            for _ in range(20):
                api.attn_fwd(q64, k64, v64, p64, 1.0 / np.sqrt(64), out=o64, lse=lse, stream=stream)
            torch.cuda.synchronize()
            log("counter pass: the headline mask at d = 64 x 20")
            p64.close()
            del q64, k64, v64, o64
        for p in plans:
            p.close()
        del q, k, v
        torch.cuda.empty_cache()


def _host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((line.split(":", 1)[1].strip() for line in f if line.startswith("model name")), None)
    except OSError:
        return None


def cpu_baseline(w, target_s, bq=128):
    """The fp64 oracle on host cores for workload w (its unsplit mask, every head).  Whole
    when a first timed query tile extrapolates to within twice target_s; otherwise every
    k-th query tile (k a power of two chosen from that rate), all heads, extrapolated by
    admitted-pair count.  TFLOPS = 4 * d * (sampled pairs) / wall time."""
    import oracle
    threads = oracle.default_threads()
    n_qt = (w.sq + bq - 1) // bq
    row_pairs = {}

    def pairs_of(i):
        if i not in row_pairs:
            row_pairs[i] = sum(hi - lo for lo, hi in oracle.row_key_set(w.slices, i))
        return row_pairs[i]

    def tile_rows(qt):
        return [(h, i) for h in range(w.hq) for i in range(qt * bq, min((qt + 1) * bq, w.sq))]

    def run(rows):
        t0 = time.perf_counter()
        oracle.attn_fwd(w.q, w.k, w.v, w.slices, w.scale, rows=rows, n_threads=threads)
        return time.perf_counter() - t0

    total_pairs = oracle.pair_count(w.slices, w.sq) * w.hq
    probe_qt = n_qt - 1                          # the last tile: the most keys in a causal mask
    probe = tile_rows(probe_qt)
    probe_pairs = sum(pairs_of(i) for _, i in probe)
    t_probe = run(probe)
    rate = probe_pairs / max(t_probe, 1e-6)      # pairs per second
    k = 1
    while total_pairs / k / rate > (2 * target_s if k == 1 else target_s) and k < n_qt:
        k *= 2
    if k == 1:
        rows = None
        pairs = total_pairs
        dt = run(None) if w.sq * w.hq > len(probe) else t_probe
        what = f"the whole workload: {w.sq * w.hq} (head, row) outputs"
    else:
        qts = list(range(0, n_qt, k))
        rows = [r for qt in qts for r in tile_rows(qt)]
        pairs = sum(pairs_of(i) for _, i in rows)
        dt = run(rows)
        what = (f"every {k}th query tile of 128 rows ({len(qts)} of {n_qt}), all {w.hq} heads: "
                f"{len(rows)} (head, row) outputs")
    tflops = 4.0 * w.d * pairs / dt * 1e-12
    return {"value": tflops, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "host_cpu": _host_cpu_model(), "host_cpu_count": os.cpu_count(),
            "compiler_flags": " ".join(oracle.CFLAGS),
            "sample": f"{what}, {pairs} unmasked pairs ({pairs / total_pairs:.3f} of the workload's), "
                      f"{dt:.1f} s wall on {threads} threads",
            "workload_s_extrapolated": dt * total_pairs / pairs}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="only the headline workload")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="untimed seconds of headline steps before the warmup steps (GPU clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time budget for the headline workload")
    ap.add_argument("--other-cpu-seconds", type=float, default=10.0,
                    help="oracle time budget for each of the other workloads")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="run only the fixed launch sequence used for hardware-counter summaries")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU mode here "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_flash_csr_amd import api
    from block_sparse_flash_csr_amd import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))
        return
    api.library()
    if args.counter_pass:
        counter_pass(api, W)
        return

    w, info, flops, ms_per_step, kernel_ms, host_ms, clock = headline(args, api, W)
    value = flops / (ms_per_step * 1e-3) * 1e-12
    achieved = flops / (kernel_ms * 1e-3) * 1e-12
    log(f"headline: step {ms_per_step:.4f} ms ({value:.1f} TFLOPS; host issue {host_ms:.4f} ms), "
        f"forward kernel {kernel_ms:.4f} ms "
        f"({achieved:.1f} TFLOPS, {achieved / PEAK_BF16_TFLOPS:.3f} of peak)")
    if clock is not None:
        log(f"clock under the headline forward: {clock['mhz_mean']:.0f} MHz (XCDs {clock['mhz_per_xcd']}); "
            f"{achieved / (PEAK_BF16_TFLOPS * clock['mhz_mean'] / 2400.0):.3f} of the bf16 peak at that clock")
    others = {} if args.quick else other_workloads(api, W, warm_s=0.5 * args.prewarm_s)
    gemm = gemm_reference(W)
    log(f"reference bf16 GEMM ({gemm['op']}): {gemm['ms']:.3f} ms, {gemm['tflops']:.1f} TFLOPS, "
        f"{gemm['frac_of_peak']:.3f} of peak"
        + ("" if gemm["clock_mhz"] is None else
           f", clock {gemm['clock_mhz']:.0f} MHz ({gemm['frac_at_measured_clock']:.3f} at that clock)"))
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_seconds)
    if not args.no_cpu_baseline:
        # the oracle beside every other workload, after all GPU timing (the GPU is idle)
        for cfg in (1, 3, 4, 5):
            wc = W.WORKLOADS[cfg]()
            if wc.name in others:
                others[wc.name]["cpu_baseline"] = cpu_baseline(wc, args.other_cpu_seconds)
                log(f"oracle {wc.name}: {others[wc.name]['cpu_baseline']['value']:.4f} TFLOPS "
                    f"({others[wc.name]['cpu_baseline']['sample']})")
            del wc

    result = {
        "metric": "effective fwd TFLOPS (unmasked pairs) and % of bf16 MFMA peak, 1 GPU",
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "host_ms_per_step": host_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) Q/K/V; document lengths drawn U[512,4096) and "
                "rescaled to 16384 tokens, seed 2)",
        "config": {"workload": w.name, "tokens": w.sq, "documents": len(w.extra["lengths"]),
                   "doc_lengths": w.extra["lengths"], "heads": w.hq, "head_dim": w.d,
                   "mask": "varlen causal", "tile": [128, 128], "parallelism": "single GPU",
                   "step": "plan build (CSR + schedule) + metadata upload + forward; each step "
                           "uploads the next step's plan and runs the forward on the one "
                           "uploaded the step before"},
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                     "traffic_unit": "bytes per launch (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, copy-calibrated)",
                     "algorithmic_bytes": w.sq * w.hq * (4 * w.d + 4) + w.sk * w.hkv * 4 * w.d,
                     "kernel": "attn_fwd_kernel<128>", "kernel_ms": kernel_ms,
                     "flops_per_launch": flops, "mfma_busy_pct": measured_mfma_busy(),
                     "l2_hit_pct": measured_workload_counters().get(w.name, {}).get("l2_hit_pct"),
                     "mfma_busy_source": "rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs), "
                                         "committed counter summary; null once the kernel changed"},
        "cpu_baseline": cpu,
        "clock": None if clock is None else dict(
            clock, source="amdsmi GPU metrics (current_gfxclks per XCD) sampled while the headline forward "
                          "runs back to back, after the timed steps",
            peak_at_measured_clock=PEAK_BF16_TFLOPS * clock["mhz_mean"] / 2400.0,
            frac_at_measured_clock=achieved / (PEAK_BF16_TFLOPS * clock["mhz_mean"] / 2400.0)),
        "gemm_reference": gemm,
        "other_workloads": others,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
