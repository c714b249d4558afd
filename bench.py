"""Benchmark: masked-attention prefill effective TFLOP/s on one MI355X.

The step (the N=1 line): one layer of masked prefill over the largest
single-GPU workload, the large irregular custom mask - one sequence of 32768
queries over 29576 keys; queries 0..27767 see keys [0, 24576) and the last
5000 queries form 50 blocks of 100, block b adding a causal 100 x 100
triangle on keys [24576 + 100 b, 24576 + 100 b + 100) - given as a range list
(one FULL range and 50 CAUSAL ranges), 32 query heads over 8 K/V heads,
head_dim 128, bf16 inputs and output, fp32 accumulation.  The plan is
compiled once per batch (reused by every head and layer) and is resident with
the inputs when timing starts; its compile time is reported beside the step.
The same mask as a bit-packed matrix, causal at the same shape, and the
chunk-causal 16384-token workload appear as extra keys of the same line.

Effective TFLOP/s counts 4 * d * Hq FLOPs per unmasked (query, key) entry
(2d for Q K^T and 2d for P V); masked entries, skipped tiles and the softmax
are not counted.

Backward lines (--backward, and under --all) time dQ, dK and dV of the
chunk-causal workload through the same plan, counting 10 * d * Hq FLOPs per
unmasked entry (the five products S, dP, dV, dQ, dK; the kernels recompute S
and dP once more, which is not counted).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--decode] [--classify] [--backward]
                       [--fp8] [--only CASE]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0      # MI355X published dense fp8 matrix-core peak
PEAK_FP32_TFLOPS = 157.3      # MI355X published fp32 (vector and matrix) peak
PEAK_HBM_GBS = 8000.0
METRIC = "masked-attn prefill effective TFLOP/s (unmasked FLOPs) and % of bf16 MFMA peak"
KERNEL_SOURCES = ["masked_flash_attention_mask_amd/csrc/attn_fwd.hip",
                  "masked_flash_attention_mask_amd/csrc/tile_bf16.h",
                  "masked_flash_attention_mask_amd/csrc/tile_dma_bf16.h",
                  "masked_flash_attention_mask_amd/csrc/kernels_common.h"]
PROFILES = os.path.join(ROOT, "profiles")
# Counter summaries (key = value lines) of the kernels the lines report, each
# tied to the kernel sources it was taken with.
TRAFFIC_FILE = os.path.join(PROFILES, "prefill_bf16_d128_block_triangle_32k_traffic.txt")
COUNTERS_FILE = os.path.join(PROFILES, "prefill_bf16_d128_block_triangle_32k_counters.txt")
TRAFFIC_FILE_CFG4 = os.path.join(PROFILES, "prefill_bf16_d128_chunk_causal_16k_traffic.txt")
COUNTERS_FILE_CFG4 = os.path.join(PROFILES, "prefill_bf16_d128_chunk_causal_16k_counters.txt")
# Host cores a GPU machine gives one GPU's jobs.
MAX_CPU_WORKERS = 16


def kernel_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_summary(path, sources=KERNEL_SOURCES):
    """key = value pairs of a committed counter summary, or None when it is
    missing or was taken with other kernel sources than those in the tree."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_hash") != kernel_hash(sources):
        return None
    return vals


def read_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch from a committed FETCH_SIZE / WRITE_SIZE summary,
    or None when the kernel sources changed since the counters were taken."""
    vals = read_summary(path)
    try:
        return float(vals["hbm_bytes_per_launch"]) if vals else None
    except (KeyError, ValueError):
        return None


def read_counters(path=COUNTERS_FILE):
    """Matrix-core busy figures from a committed counter summary (same
    kernel-source rule as the traffic)."""
    vals = read_summary(path)
    if not vals:
        return None
    out = {}
    for k in ("mfma_busy_pct", "mfma_flops_executed", "valu_active_pct", "mfma_coexec_pct"):
        if k in vals:
            out[k] = float(vals[k])
    return out or None


# ------------------------------------------------------ visible entries --
def chunk_unmasked(seq, prefix, cs):
    """Visible (query, key) pairs of the chunk-causal workload, by rows."""
    total = prefix * (prefix + 1) // 2
    start = prefix
    while start < seq:
        end = min(seq, start + cs)
        total += (end - start) * end
        start = end
    return total


def block_triangle_unmasked(q_len, dense_keys, blocks, block):
    """Visible pairs of the block mask with causal triangles: every row sees
    dense_keys keys, row i of a triangle block i + 1 more."""
    return q_len * dense_keys + blocks * block * (block + 1) // 2


def causal_unmasked(q_len, kv_len):
    """Bottom-right causal: row t sees keys <= t + kv_len - q_len."""
    return sum(max(0, min(kv_len, t + kv_len - q_len + 1)) for t in range(q_len))


def _anc(parents, i):
    out = [i]
    while i != 0:
        i = int(parents[i])
        out.append(i)
    return out


def count_unmasked(w, name):
    """Visible pairs per head, read off the host plan: FULL tiles count their
    in-bounds area, PARTIAL tiles the set bits of their words."""
    import numpy as np
    import masked_flash_attention_mask_amd as ma
    from workloads.device import plan_kwargs
    kind, kw = plan_kwargs(w, name, host=True)
    plan = ma.mask_compile_host(kind, w.cu_seqlens_q, w.kv_lens, **kw)
    cls, words = plan.export()
    total = 0
    info = plan.info()
    t = 0
    for b in range(w.batch):
        ql, kl = int(w.q_lens[b]), int(w.kv_lens[b])
        nqt, nkt = -(-ql // info.tile_q), -(-kl // 64)
        c = cls[t:t + nqt * nkt].reshape(nqt, nkt)
        rows = np.minimum(info.tile_q, ql - np.arange(nqt) * info.tile_q)
        keys = np.minimum(64, kl - np.arange(nkt) * 64)
        total += int((np.outer(rows, keys) * (c == 1)).sum())
        wb = words[t:t + nqt * nkt]
        pc = np.unpackbits(wb.view(np.uint8), axis=1).sum(axis=1)
        total += int(pc[(c == 2).reshape(-1)].sum())
        t += nqt * nkt
    return total


# ------------------------------------------------------------ CPU oracle --
_ORACLE_JOB = None
_BLAS_LIMIT = None


def _one_blas_thread():
    global _BLAS_LIMIT
    from threadpoolctl import threadpool_limits
    _BLAS_LIMIT = threadpool_limits(1)


def _oracle_unit(i):
    """One (sequence, query head, row block) unit of the oracle."""
    from oracle import attention as OA
    w, masks, units = _ORACLE_JOB
    b, h, r0, r1 = units[i]
    q0, kl = int(w.cu_seqlens_q[b]), int(w.kv_lens[b])
    g = h // (w.hq // w.hkv)
    k = OA.gather_paged(w.k_cache, w.page_table[b], kl, g)
    v = OA.gather_paged(w.v_cache, w.page_table[b], kl, g)
    OA.attend(w.q[q0 + r0:q0 + r1, h, :], k, v, masks[b][r0:r1], w.scale)
    return int(masks[b][r0:r1].sum())


def cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, MAX_CPU_WORKERS))


def cpu_oracle(w, masks, units, sample):
    """The oracle as it stands (fp64 NumPy, oracle/attention.py) over the given
    (sequence, head, row start, row end) units: a fork pool with one worker per
    host core (sched_getaffinity, at most 16), one BLAS thread each.  Run it
    before anything touches the GPU.  Returns the cpu_baseline object:
    effective TFLOP/s over the visible pairs of the sampled rows."""
    import multiprocessing as mp
    global _ORACLE_JOB
    _ORACLE_JOB = (w, masks, units)
    workers = min(cpu_workers(), len(units))
    with mp.get_context("fork").Pool(workers, initializer=_one_blas_thread) as pool:
        pool.map(_oracle_unit, range(min(workers, len(units))))   # warm the workers
        t0 = time.perf_counter()
        visible = sum(pool.map(_oracle_unit, range(len(units)), chunksize=1))
        dt = time.perf_counter() - t0
    _ORACLE_JOB = None
    flops = 4.0 * w.d * visible
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(workers), "kind": "oracle",
            "sample": sample + f"; {len(units)} units on {workers} worker processes, {dt:.1f} s",
            "seconds": round(dt, 2), "visible_pairs": visible}


def cfg5_cpu_baseline(w, rows_per_head=16384, unit_rows=4096):
    """Oracle on a bounded sample of the headline workload: query head h
    takes rows_per_head rows starting at row h * rows_per_head / 4 (wrapped),
    in units of unit_rows rows, so the sample spans the dense rows and the
    triangle blocks."""
    from oracle import masks as OM
    q_len, kv_len = int(w.q_lens[0]), int(w.kv_lens[0])
    dense = OM.ranges(q_len, kv_len, w.masks["custom_ranges"].ranges[0])
    units = []
    for h in range(w.hq):
        first = (h * rows_per_head // 4) % q_len
        for r in range(0, rows_per_head, unit_rows):
            r0 = (first + r) % q_len
            units.append((0, h, r0, min(q_len, r0 + unit_rows)))
    out = cpu_oracle(w, [dense], units, f"{rows_per_head} query rows per head over all {w.hq} heads (head h: "
                                        f"rows from h * {rows_per_head // 4}, wrapped), all {kv_len} keys, "
                                        f"fp64 NumPy")
    del dense
    return out


def sampled_units(w, budget_flops=3e11, row_block=512):
    """Units (b, h, r0, r1) of a workload, rows in blocks of row_block, taken
    round-robin over sequences and heads until the dense fp64 work
    (4 d rows kv_len) reaches budget_flops."""
    units, spent = [], 0.0
    blocks = []
    for b in range(w.batch):
        ql = int(w.q_lens[b])
        blocks.append([(r, min(ql, r + row_block)) for r in range(0, ql, row_block)])
    i = 0
    while spent < budget_flops:
        added = False
        for h in range(w.hq):
            for b in range(w.batch):
                if i < len(blocks[b]):
                    r0, r1 = blocks[b][(i + h) % len(blocks[b])]
                    units.append((b, h, r0, r1))
                    spent += 4.0 * w.d * (r1 - r0) * int(w.kv_lens[b])
                    added = True
                    if spent >= budget_flops:
                        return units
        i += 1
        if not added or i > max(len(x) for x in blocks):
            break
    return units


def oracle_line(w, name, budget_flops=1e12):
    """cpu_baseline-style oracle timing for one workload and mask."""
    from oracle import masks as OM
    mi = w.masks[name]
    masks = []
    if mi.kind in ("packed", "dense"):
        masks = (OM.packed_from_flat if mi.kind == "packed" else OM.dense_from_flat)(mi.data, w.q_lens, w.kv_lens)
    for b in range(w.batch if not masks else 0):
        ql, kl = int(w.q_lens[b]), int(w.kv_lens[b])
        if mi.kind == "causal":
            masks.append(OM.causal(ql, kl))
        elif mi.kind == "window":
            masks.append(OM.sliding_window(ql, kl, mi.window))
        elif mi.kind == "prefix_lm":
            masks.append(OM.prefix_lm(ql, kl, int(mi.prefix_len[b])))
        elif mi.kind == "ranges":
            masks.append(OM.ranges(ql, kl, mi.ranges[b]))
        else:
            raise ValueError(mi.kind)
    units = sampled_units(w, budget_flops)
    return cpu_oracle(w, masks, units, f"{len(units)} (sequence, head, <=512-row) blocks, fp64 NumPy")


# ---------------------------------------------------------------- timing --
def time_steps(fn, steps, warmup, stream):
    """Mean ms per call over `steps` calls after `warmup`, by HIP events
    recorded on the launch stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def run_config(w, mask_name, steps, warmup, out_dtype, tile_q=128, dev=None):
    import torch
    import masked_flash_attention_mask_amd as ma
    from workloads.device import device_inputs, plan_kwargs
    dev = dev or device_inputs(w)
    kind, kw = plan_kwargs(w, mask_name)
    stream = torch.cuda.current_stream()

    def compile_once():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        pl = ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, tile_q=tile_q, **kw)
        torch.cuda.synchronize()
        return pl, (time.perf_counter() - t0) * 1e3

    # The first compile in a process also allocates the plan's device and
    # pinned staging buffers; a destroyed plan hands them to the next one, so
    # the steady-state cost is the median of three compiles after it.
    plan, cold_ms = compile_once()
    warm = []
    for _ in range(3):
        del plan
        plan, t = compile_once()
        warm.append(t)
    compile_ms = sorted(warm)[1]
    plan.compile_cold_ms = cold_ms
    out = torch.empty(dev["q"].shape, dtype=out_dtype, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")

    def step():
        ma.attn_prefill_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], w.scale, out=out, lse=lse)

    ms = time_steps(step, steps, warmup, stream)
    return ms, compile_ms, plan


def prefill_bytes(w, out_bytes=2):
    """Algorithmic HBM bytes of one prefill launch: Q, the visible sequences'
    K and V once per K/V head, O and the fp32 LSE."""
    el = 4 if w.dtype == "f32" else 2
    tq = int(w.cu_seqlens_q[-1])
    kv = int(w.kv_lens.sum())
    return tq * w.hq * w.d * el + 2 * kv * w.hkv * w.d * el + tq * w.hq * (w.d * out_bytes + 4)


def roofline(tflops, flops, nbytes, kernel, traffic, counters):
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = flops / nbytes
    bound = "mfma" if intensity > ridge else "hbm"
    if bound == "mfma":
        achieved, peak, unit = tflops, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = nbytes / (flops / (tflops * 1e12)) / 1e9, PEAK_HBM_GBS, "GB/s"
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel,
         "flops_per_launch": flops, "algorithmic_bytes": nbytes,
         "intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
         "timing": "HIP events on the launch stream around the timed steps; one kernel per step"}
    if counters:
        r["counters"] = counters
    return r


# ------------------------------------------------------------ the cases --
def _case(name):
    """(workload, mask name, visible pairs per head, description) of a
    prefill case by name."""
    import workloads as W
    if name.startswith("cfg5_"):
        w = W.config5()
        mask = {"cfg5_ranges": "custom_ranges", "cfg5_packed": "custom_packed", "cfg5_causal": "causal"}[name]
        n = (causal_unmasked(int(w.q_lens[0]), int(w.kv_lens[0])) if mask == "causal" else
             block_triangle_unmasked(int(w.q_lens[0]), w.info["dense_keys"], w.info["blocks"], w.info["block"]))
        return w, mask, n
    if name.startswith("cfg4_"):
        w = W.config4(chunk_sizes=(2,))
        mask = name[5:]
        n = 16384 * 16385 // 2 if mask == "causal" else chunk_unmasked(16384, 1024, 2)
        return w, mask, n
    if name.startswith("cfg3b_"):
        layer = 0 if name == "cfg3b_window" else 1
        w = W.config3b(layer)
        mask = "window" if layer == 0 else "causal"
        return w, mask, count_unmasked(w, mask)
    if name.startswith("cfg3a_"):
        w = W.config3a()
        mask = name[6:]
        return w, mask, count_unmasked(w, mask)
    if name.startswith("cfg1_"):
        w = W.config1()
        mask = name[5:]
        return w, mask, count_unmasked(w, mask)
    raise ValueError(name)


CASES = ["cfg5_ranges", "cfg5_packed", "cfg5_causal", "cfg4_chunk2", "cfg4_causal", "cfg3a_prefix_lm",
         "cfg3a_causal", "cfg3b_window", "cfg3b_causal", "cfg2_packed", "cfg2_dense", "cfg2_causal",
         "cfg1_causal", "cfg1_custom"]


def only_case(name, steps, warmup):
    """Time one case alone (for profilers): one JSON line."""
    import torch
    if name.startswith("cfg2_"):
        r = verify_case(name[5:], steps, warmup)
        print(json.dumps({"only": name, **r}), flush=True)
        return
    w, mask, n = _case(name)
    f32 = w.dtype == "f32"   # config 1: fp32 in and out, against the fp32 peak
    ms, _, _ = run_config(w, mask, steps, warmup, torch.float32 if f32 else torch.bfloat16)
    tf = 4.0 * w.d * w.hq * n / (ms * 1e-3) / 1e12
    print(json.dumps({"only": name, "ms": round(ms, 5 if f32 else 4), "tflops": round(tf, 4 if f32 else 2),
                      "pct_of_peak": round(100 * tf / (PEAK_FP32_TFLOPS if f32 else PEAK_BF16_TFLOPS), 3)}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--all", action="store_true", help="also print lines for the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baselines")
    ap.add_argument("--only", choices=CASES, help="time one case alone (no comparators, no CPU): for profilers")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--decode", action="store_true", help="print only the decode lines")
    ap.add_argument("--classify", action="store_true",
                    help="print only the device mask-classify lines (block mask, packed and dense)")
    ap.add_argument("--backward", action="store_true", help="print only the backward lines")
    ap.add_argument("--fp8", action="store_true", help="print only the fp8 (e4m3) prefill lines")
    ap.add_argument("--cpu-rows", type=int, default=16384, help="query rows per head in the CPU baseline sample")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    if args.calib_copy_mib:
        import torch
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_each_way": n * 4}), flush=True)
        del src, dst
    if args.only:
        only_case(args.only, args.steps, args.warmup)
        return
    if args.decode or args.classify or args.backward or args.fp8:
        if args.fp8:
            fp8_lines(args.steps, args.warmup)
        if args.decode:
            decode_lines(args.steps, args.warmup)
        if args.classify:
            classify_lines(args.steps)
        if args.backward:
            backward_lines(args.steps, args.warmup)
        return

    import workloads as W
    w5 = W.config5()
    # The oracle runs first, in forked workers, before anything touches the GPU.
    cpu = None if args.no_cpu else cfg5_cpu_baseline(w5, args.cpu_rows)

    import torch
    from workloads.device import device_inputs
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    q_len, kv_len = int(w5.q_lens[0]), int(w5.kv_lens[0])
    n_unmasked = block_triangle_unmasked(q_len, w5.info["dense_keys"], w5.info["blocks"], w5.info["block"])
    flops = 4.0 * w5.d * w5.hq * n_unmasked
    dev5 = device_inputs(w5)
    ms, compile_ms, plan5 = run_config(w5, "custom_ranges", args.steps, args.warmup, torch.bfloat16, dev=dev5)
    compile_cold_ms = plan5.compile_cold_ms
    del plan5
    tflops = flops / (ms * 1e-3) / 1e12
    cmp_steps, cmp_warm = max(3, args.steps // 2), max(2, args.warmup // 2)
    pk_ms, pk_cms, _ = run_config(w5, "custom_packed", cmp_steps, cmp_warm, torch.bfloat16, dev=dev5)
    pk_tflops = flops / (pk_ms * 1e-3) / 1e12
    n_causal = causal_unmasked(q_len, kv_len)
    c_ms, _, _ = run_config(w5, "causal", cmp_steps, cmp_warm, torch.bfloat16, dev=dev5)
    c_tflops = 4.0 * w5.d * w5.hq * n_causal / (c_ms * 1e-3) / 1e12
    nbytes = prefill_bytes(w5)
    del dev5

    # the chunk-causal 16384-token workload and its causal comparator
    w4 = W.config4(chunk_sizes=(2,))
    dev4 = device_inputs(w4)
    n4 = chunk_unmasked(16384, 1024, 2)
    flops4 = 4.0 * w4.d * w4.hq * n4
    ms4, _, _ = run_config(w4, "chunk2", args.steps, args.warmup, torch.bfloat16, dev=dev4)
    tf4 = flops4 / (ms4 * 1e-3) / 1e12
    ms4c, _, _ = run_config(w4, "causal", args.steps, args.warmup, torch.bfloat16, dev=dev4)
    tf4c = 4.0 * w4.d * w4.hq * (16384 * 16385 // 2) / (ms4c * 1e-3) / 1e12
    del dev4

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "large irregular custom mask: 1 sequence, 32768 queries x 29576 keys; queries "
                               "0-27767 see keys [0,24576), queries 27768-32767 form 50 blocks of 100 each adding "
                               "a causal 100x100 triangle on keys [24576+100b, 24576+100b+100); given as a range "
                               "list (1 FULL + 50 CAUSAL ranges); 32 query heads / 8 K/V heads, head_dim 128, "
                               "bf16 in/out, fp32 accumulation",
                   "global_batch": 1, "q_len": q_len, "kv_len": kv_len, "heads": w5.hq, "kv_heads": w5.hkv,
                   "head_dim": w5.d, "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "unmasked_entries_per_head": n_unmasked,
        "plan_compile_ms": round(compile_ms, 3),
        "plan_compile_cold_ms": round(compile_cold_ms, 3),
        "packed_form": {"ms": round(pk_ms, 4), "tflops": round(pk_tflops, 2),
                        "pct_of_peak": round(100.0 * pk_tflops / PEAK_BF16_TFLOPS, 2),
                        "plan_compile_ms": round(pk_cms, 3),
                        "note": "device-classified bit-packed mask (121 MB of words)"},
        "causal_same_shape": {"ms": round(c_ms, 4), "tflops": round(c_tflops, 2),
                              "pct_of_peak": round(100.0 * c_tflops / PEAK_BF16_TFLOPS, 2),
                              "unmasked_entries_per_head": n_causal,
                              "ratio_masked_over_causal": round(tflops / c_tflops, 3)},
        "chunk_causal_16k": {"workload": "1 x 16384 tokens: 1024-token causal prefix + 7680 (token, latent) pairs, "
                                         "chunk_size 2 as one CHUNK_CAUSAL range; 16 heads, head_dim 128",
                             "ms": round(ms4, 4), "tflops": round(tf4, 2),
                             "pct_of_peak": round(100.0 * tf4 / PEAK_BF16_TFLOPS, 2),
                             "causal_ms": round(ms4c, 4), "causal_tflops": round(tf4c, 2),
                             "causal_pct_of_peak": round(100.0 * tf4c / PEAK_BF16_TFLOPS, 2),
                             "traffic": read_traffic(TRAFFIC_FILE_CFG4),
                             "counters": read_counters(COUNTERS_FILE_CFG4)},
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "roofline": roofline(tflops, flops, nbytes, "prefill_bf16_kernel<128,128,bf16,DMA gather>",
                             read_traffic(), read_counters()),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)

    if args.all:
        extra(args)
        decode_lines(args.steps, args.warmup)
        backward_lines(args.steps, args.warmup)
        fp8_lines(args.steps, args.warmup)


def verify_case(form, steps, warmup, w2=None, dev=None):
    """Tree verify (config 2) with the mask as packed or dense rows, or the
    causal comparator at the same shape: ms, TFLOP/s and K/V GB/s."""
    import numpy as np
    import torch
    import workloads as W
    import masked_flash_attention_mask_amd as ma
    from workloads.device import device_inputs
    w2 = w2 or W.config2()
    dev = dev or device_inputs(w2)
    max_q, max_kv = 64, int(w2.kv_lens.max())
    out = torch.empty(dev["q"].shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    if form == "causal":
        ws = torch.empty(max(ma.attn_decode_workspace(w2.batch, max_q, max_kv, w2.hq, w2.hkv, w2.d), 1),
                         dtype=torch.uint8, device="cuda")

        def step():
            ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], max_q, max_kv, w2.scale,
                           mask_kind="causal", workspace=ws, out=out, lse=lse)
        n = sum(64 * int(c) + 64 * 65 // 2 for c in w2.info["ctx"])
    else:
        mi = w2.masks["tree_" + form]
        data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
        mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
        ws = torch.empty(max(ma.attn_verify_tree_workspace(w2.batch, max_q, max_kv, w2.hq, w2.hkv, w2.d), 1),
                         dtype=torch.uint8, device="cuda")

        def step():
            ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, mi.kind, max_q,
                                max_kv, w2.scale, workspace=ws, out=out, lse=lse)
        n = sum(64 * int(c) for c in w2.info["ctx"]) + sum(
            int(np.sum([len(_anc(p, i)) for i in range(64)])) for p in w2.info["parents"])
    ms = time_steps(step, steps, warmup, stream)
    cold = cold_steps(step, min(steps, 20), stream)
    flops = 4.0 * w2.d * w2.hq * n
    tf = flops / (ms * 1e-3) / 1e12
    kv_bytes = 2 * int(w2.kv_lens.sum()) * w2.hkv * w2.d * 2
    qo_bytes = int(w2.cu_seqlens_q[-1]) * w2.hq * (w2.d * 2 * 2 + 4)
    bound_us = max(flops / (PEAK_BF16_TFLOPS * 1e12), (kv_bytes + qo_bytes) / (PEAK_HBM_GBS * 1e9)) * 1e6
    return {"ms": round(ms, 4), "tflops": round(tf, 2), "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1),
            "roofline_us": round(bound_us, 2), "frac_of_roofline": round(bound_us / (ms * 1e3), 4),
            "cold_ms": round(cold, 4), "cold_frac_of_roofline": round(bound_us / (cold * 1e3), 4),
            "flops": flops, "bytes": kv_bytes + qo_bytes}


FLUSH_BYTES = 512 << 20   # more than the 256 MB of last-level cache (MALL)


def cold_steps(step, reps, stream):
    """Mean ms of `reps` single steps, each after a write of FLUSH_BYTES
    (outside the timed region) that evicts the caches: the cold time."""
    import torch
    buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    total = 0.0
    for i in range(reps):
        buf.fill_(i & 0xFF)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        total += a.elapsed_time(b)
    del buf
    return total / reps


def extra(args):
    """One informational line per other workload (not the headline), each
    with the oracle timed on a bounded sample unless --no-cpu."""
    import torch
    import workloads as W
    import masked_flash_attention_mask_amd as ma
    from workloads.device import device_inputs
    # config 1: fp32, 128 x 128, one head (latency, far from any roof)
    w1 = W.config1()
    dev1 = device_inputs(w1)
    for name in ("causal", "custom"):
        ms, cms, _ = run_config(w1, name, 200, 50, torch.float32, dev=dev1)
        n = count_unmasked(w1, name)
        tf = 4.0 * w1.d * w1.hq * n / (ms * 1e-3) / 1e12
        print(json.dumps({"workload": "cfg1", "mask": name, "ms": round(ms, 5), "tflops": round(tf, 4),
                          "pct_of_fp32_peak": round(100 * tf / PEAK_FP32_TFLOPS, 3), "compile_ms": round(cms, 3),
                          "unmasked_per_head": n}), flush=True)
    rows = []
    w4 = W.config4()
    for name in ("chunk4", "chunk16", "chunk2_full", "causal"):
        ms, cms, plan = run_config(w4, name, args.steps, args.warmup, torch.bfloat16)
        rows.append(("cfg4", name, ms, cms, w4))
    w3a = W.config3a()
    for name in ("prefix_lm", "causal"):
        ms, cms, plan = run_config(w3a, name, args.steps, args.warmup, torch.bfloat16)
        rows.append(("cfg3a", name, ms, cms, w3a))
    for layer in (0, 1):
        w3b = W.config3b(layer)
        name = "window" if layer == 0 else "causal"
        ms, cms, plan = run_config(w3b, name, args.steps, args.warmup, torch.bfloat16)
        rows.append((f"cfg3b_l{layer}", name, ms, cms, w3b))
    for cfg, name, ms, cms, w in rows:
        n = count_unmasked(w, name)
        tf = 4.0 * w.d * w.hq * n / (ms * 1e-3) / 1e12
        print(json.dumps({"workload": cfg, "mask": name, "ms": round(ms, 4), "tflops": round(tf, 2),
                          "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "compile_ms": round(cms, 3),
                          "unmasked_per_head": n}), flush=True)
    w2 = W.config2()
    dev2 = device_inputs(w2)
    for form in ("packed", "dense", "causal"):
        r = verify_case(form, 100, 20, w2, dev2)
        print(json.dumps({"workload": "cfg2", "mask": "tree_" + form if form != "causal" else "causal", **r}),
              flush=True)
    if not args.no_cpu:
        for wl, name in ((w1, "causal"), (w2, "tree_packed"), (w3a, "prefix_lm"), (W.config3b(0), "window"),
                         (w4, "chunk2")):
            print(json.dumps({"workload": wl.name, "mask": name, "cpu_oracle": oracle_line(wl, name)}), flush=True)


def decode_lines(steps, warmup):
    """Decode (memory bound): K/V bytes the visible keys need, per second,
    against HBM."""
    import torch
    import workloads as W
    import numpy as np
    import masked_flash_attention_mask_amd as ma
    from workloads.device import device_inputs
    import copy
    w4 = W.decode(q_len=4)
    for q_len in (1, 4):
        if q_len == 4:
            w = w4
        else:   # each sequence's last query: the same position, q_len 1
            w = copy.copy(w4)
            w.q = w4.q[3::4].copy()
            w.cu_seqlens_q = np.arange(w4.batch + 1, dtype=np.int32)
        dev = device_inputs(w)
        max_kv = int(w.kv_lens.max())
        ws = torch.empty(max(ma.attn_decode_workspace(w.batch, q_len, max_kv, w.hq, w.hkv, w.d), 1),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty(dev["q"].shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
        for name in ("causal", "window"):
            win = w.masks[name].window if name == "window" else 0

            def step():
                ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], q_len, max_kv,
                               w.scale, mask_kind=name, window=win, workspace=ws, out=out, lse=lse)
            ms = time_steps(step, steps, warmup, torch.cuda.current_stream())
            keys = [int(k) if name == "causal" else min(int(k), win + q_len - 1) for k in w.kv_lens]
            kv_bytes = 2 * sum(keys) * w.hkv * w.d * 2
            gbs = kv_bytes / (ms * 1e-3) / 1e9
            print(json.dumps({"workload": f"decode_q{q_len}", "mask": name, "ms": round(ms, 4),
                              "kv_gbs": round(gbs, 1), "pct_of_hbm": round(100 * gbs / 8000.0, 1),
                              "batch": w.batch, "kv_total": int(w.kv_lens.sum())}), flush=True)
        if q_len == 1:
            # the same batch over e4m3 caches (half the bytes per key)
            f8 = W.fp8_inputs(w)
            k8 = torch.from_numpy(np.ascontiguousarray(f8["k8"])).cuda()
            v8 = torch.from_numpy(np.ascontiguousarray(f8["v8"])).cuda()
            for name in ("causal", "window"):
                win = w.masks[name].window if name == "window" else 0

                def step8():
                    ma.attn_decode_kv8(dev["q"], k8, v8, dev["pt"], dev["cu"], dev["kv"], q_len, max_kv, w.scale,
                                       f8["k_s"], f8["v_s"], mask_kind=name, window=win, workspace=ws, out=out,
                                       lse=lse)
                ms = time_steps(step8, steps, warmup, torch.cuda.current_stream())
                keys = [int(k) if name == "causal" else min(int(k), win + q_len - 1) for k in w.kv_lens]
                kv_bytes = 2 * sum(keys) * w.hkv * w.d
                gbs = kv_bytes / (ms * 1e-3) / 1e9
                print(json.dumps({"workload": "decode_q1_kv8", "mask": name, "ms": round(ms, 4),
                                  "kv_gbs": round(gbs, 1), "pct_of_hbm": round(100 * gbs / 8000.0, 1),
                                  "batch": w.batch, "kv_total": int(w.kv_lens.sum())}), flush=True)
        del dev


def backward_lines(steps, warmup):
    """Backward (dQ, dK, dV) of the chunk-causal workload and of causal at
    the same shape, each through its plan, forward outputs resident."""
    import torch
    import workloads as W
    import masked_flash_attention_mask_amd as ma
    from workloads.device import device_inputs, plan_kwargs
    seq, prefix, cs, hq, d = 16384, 1024, 2, 16, 128
    w = W.config4(seq=seq, prefix=prefix, hq=hq, d=d, chunk_sizes=(cs,))
    dev = device_inputs(w)
    do = torch.from_numpy(W.upstream_grad(w, 4001)).cuda().to(torch.bfloat16).contiguous()
    stream = torch.cuda.current_stream()
    for name, n_unmasked in ((f"chunk{cs}", chunk_unmasked(seq, prefix, cs)), ("causal", seq * (seq + 1) // 2)):
        kind, kw = plan_kwargs(w, name)
        plan = ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, **kw)
        out, lse = ma.attn_prefill_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], w.scale)
        dq = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
        dk = torch.zeros(dev["k"].shape, dtype=torch.float32, device="cuda")
        dv = torch.zeros_like(dk)
        ws = torch.empty(ma.attn_backward_workspace(plan, hq), dtype=torch.uint8, device="cuda")

        def step():
            ma.attn_backward_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], out, lse, do, w.scale, dq=dq,
                                    dk_cache=dk, dv_cache=dv, workspace=ws)
        ms = time_steps(step, steps, warmup, stream)
        tf = 10.0 * d * hq * n_unmasked / (ms * 1e-3) / 1e12
        print(json.dumps({"workload": f"backward_{name}_16k", "mask": name, "ms": round(ms, 4),
                          "tflops": round(tf, 2), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                          "flops_per_step": 10.0 * d * hq * n_unmasked,
                          "kernels": "bwd_prep, bwd_dq<128,128>, bwd_dkdv<128>"}), flush=True)
        del plan
    # the Gemma2-like global layer (d 256, causal, 8 / 4 heads)
    w3 = W.config3b(1)
    dev3 = device_inputs(w3)
    do3 = torch.from_numpy(W.upstream_grad(w3, 4003)).cuda().to(torch.bfloat16).contiguous()
    kind, kw = plan_kwargs(w3, "causal")
    plan = ma.mask_compile(kind, w3.cu_seqlens_q, w3.kv_lens, **kw)
    out3, lse3 = ma.attn_prefill_masked(plan, dev3["q"], dev3["k"], dev3["v"], dev3["pt"], w3.scale)
    dq3 = torch.empty(dev3["q"].shape, dtype=torch.float32, device="cuda")
    dk3 = torch.zeros(dev3["k"].shape, dtype=torch.float32, device="cuda")
    dv3 = torch.zeros_like(dk3)
    ws3 = torch.empty(ma.attn_backward_workspace(plan, w3.hq), dtype=torch.uint8, device="cuda")

    def step3():
        ma.attn_backward_masked(plan, dev3["q"], dev3["k"], dev3["v"], dev3["pt"], out3, lse3, do3, w3.scale, dq=dq3,
                                dk_cache=dk3, dv_cache=dv3, workspace=ws3)
    ms = time_steps(step3, steps, warmup, stream)
    n3 = 16384 * 16385 // 2
    tf = 10.0 * w3.d * w3.hq * n3 / (ms * 1e-3) / 1e12
    print(json.dumps({"workload": "backward_gemma2_global_16k_d256", "mask": "causal", "ms": round(ms, 4),
                      "tflops": round(tf, 2), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                      "flops_per_step": 10.0 * w3.d * w3.hq * n3,
                      "kernels": "bwd_prep, bwd_dq<256,128>, bwd_dkdv<256>"}), flush=True)
    del plan


def fp8_lines(steps, warmup):
    """fp8 (e4m3) prefill of the chunk-causal workload and of causal at the
    same shape: the bf16 inputs quantized per tensor, bf16 output."""
    import numpy as np
    import torch
    import workloads as W
    import masked_flash_attention_mask_amd as ma
    from workloads.device import plan_kwargs
    seq, prefix, cs, hq, d = 16384, 1024, 2, 16, 128
    w = W.config4(seq=seq, prefix=prefix, hq=hq, d=d, chunk_sizes=(cs,))
    f8 = W.fp8_inputs(w)
    dev = {k: torch.from_numpy(np.ascontiguousarray(f8[k])).cuda() for k in ("q8", "k8", "v8")}
    pt = torch.from_numpy(w.page_table).cuda().contiguous()
    out = torch.empty(dev["q8"].shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(dev["q8"].shape[:2], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for name, n_unmasked in ((f"chunk{cs}", chunk_unmasked(seq, prefix, cs)), ("causal", seq * (seq + 1) // 2)):
        kind, kw = plan_kwargs(w, name)
        plan = ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, **kw)

        def step():
            ma.attn_prefill_masked_fp8(plan, dev["q8"], dev["k8"], dev["v8"], pt, w.scale, f8["q_s"], f8["k_s"],
                                       f8["v_s"], out=out, lse=lse)
        ms = time_steps(step, steps, warmup, stream)
        tf = 4.0 * d * hq * n_unmasked / (ms * 1e-3) / 1e12
        print(json.dumps({"workload": f"prefill_fp8_{name}_16k", "mask": name, "ms": round(ms, 4),
                          "tflops": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                          "pct_of_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
                          "flops_per_step": 4.0 * d * hq * n_unmasked,
                          "kernel": "prefill_fp8_kernel<128,bf16>"}), flush=True)
        del plan
    # the Gemma2-like layers (d 256): window 4096 and global causal
    for layer in (0, 1):
        w3 = W.config3b(layer)
        name = "window" if layer == 0 else "causal"
        g8 = W.fp8_inputs(w3)
        dev3 = {k: torch.from_numpy(np.ascontiguousarray(g8[k])).cuda() for k in ("q8", "k8", "v8")}
        pt3 = torch.from_numpy(w3.page_table).cuda().contiguous()
        out3 = torch.empty(dev3["q8"].shape, dtype=torch.bfloat16, device="cuda")
        lse3 = torch.empty(dev3["q8"].shape[:2], dtype=torch.float32, device="cuda")
        kind, kw = plan_kwargs(w3, name)
        plan = ma.mask_compile(kind, w3.cu_seqlens_q, w3.kv_lens, **kw)

        def step3():
            ma.attn_prefill_masked_fp8(plan, dev3["q8"], dev3["k8"], dev3["v8"], pt3, w3.scale, g8["q_s"], g8["k_s"],
                                       g8["v_s"], out=out3, lse=lse3)
        ms = time_steps(step3, steps, warmup, stream)
        n_unmasked = count_unmasked(w3, name)
        tf = 4.0 * w3.d * w3.hq * n_unmasked / (ms * 1e-3) / 1e12
        print(json.dumps({"workload": f"prefill_fp8_gemma2_l{layer}_16k", "mask": name, "ms": round(ms, 4),
                          "tflops": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                          "pct_of_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
                          "flops_per_step": 4.0 * w3.d * w3.hq * n_unmasked,
                          "kernel": "prefill_fp8_kernel<256,bf16>"}), flush=True)
        del plan, dev3


def classify_lines(steps):
    """Device mask classify (an HBM scan) on the 32768 x 29576 block mask,
    packed (121 MB) and dense (969 MB): wall time of mask_compile per call
    (host part included); the kernel's own time comes from a kernel trace."""
    import numpy as np
    import torch
    import workloads as W
    import masked_flash_attention_mask_amd as ma
    w = W.config5()
    q, k = int(w.q_lens[0]), int(w.kv_lens[0])
    words = w.masks["custom_packed"].data
    dense = np.unpackbits(words.view(np.uint8).reshape(q, -1), axis=1, bitorder="little")[:, :k]
    forms = (("packed", torch.from_numpy(np.ascontiguousarray(words.view(np.int64))).cuda()),
             ("dense", torch.from_numpy(np.ascontiguousarray(dense)).cuda()))
    for kind, m in forms:
        for _ in range(3):
            ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, mask=m)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(steps):
            ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, mask=m)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t) / steps * 1e3
        nbytes = m.numel() * m.element_size()
        print(json.dumps({"workload": "cfg5_classify", "form": kind, "mask_bytes": nbytes,
                          "compile_ms": round(ms, 4)}), flush=True)


if __name__ == "__main__":
    main()
