"""Benchmark: masked-attention prefill effective TFLOP/s on one MI355X.

Workload (the step): one layer of masked prefill over the chunk-causal
interleaved-pairs shape — one packed sequence of 16384 tokens, a 1024-token
causal prefix then 7680 (token, latent) pairs with chunk size 2 given as one
CHUNK_CAUSAL range, 16 heads, head_dim 128, bf16 inputs and output, fp32
accumulation.  The plan is compiled once per batch (it is reused by every
head and layer) and is resident with the inputs when timing starts; its
compile time is reported beside the step.

Effective TFLOP/s counts 4 * d * Hq FLOPs per unmasked (query, key) entry
(2d for Q K^T and 2d for P V); masked entries, skipped tiles and the softmax
are not counted.

Backward lines (--backward, and under --all) time dQ, dK and dV of the same
workload through the same plan, counting 10 * d * Hq FLOPs per unmasked entry
(the five products S, dP, dV, dQ, dK; the kernels recompute S and dP once
more, which is not counted).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--decode] [--classify] [--backward]
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
PEAK_HBM_GBS = 8000.0
METRIC = "masked-attn prefill effective TFLOP/s (unmasked FLOPs) and % of bf16 MFMA peak"
KERNEL_SOURCES = ["masked_flash_attention_mask_amd/csrc/attn_fwd.hip",
                  "masked_flash_attention_mask_amd/csrc/tile_bf16.h",
                  "masked_flash_attention_mask_amd/csrc/tile_dma_bf16.h",
                  "masked_flash_attention_mask_amd/csrc/kernels_common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bf16_d128_chunk_causal_16k_traffic.txt")


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_hash") != kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def unmasked_entries(plan_dense_counts):
    return int(plan_dense_counts)


def chunk_unmasked(seq, prefix, cs):
    """Visible (query, key) pairs of the chunk-causal workload, by rows."""
    total = prefix * (prefix + 1) // 2
    start = prefix
    while start < seq:
        end = min(seq, start + cs)
        total += (end - start) * end
        start = end
    return total


def time_steps(fn, steps, warmup, stream):
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


def cpu_baseline(w, mask_name, n_unmasked_head, heads=8):
    """The oracle, as it stands, on a bounded sample of the same workload:
    `heads` query heads over the whole sequence."""
    import numpy as np
    from oracle import attention as OA
    from oracle import masks as OM
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    mi = w.masks[mask_name]
    q_len = int(w.q_lens[0])
    dense = OM.ranges(q_len, int(w.kv_lens[0]), mi.ranges[0])
    t0 = time.perf_counter()
    OA.attention(w.q, w.k_cache, w.v_cache, w.page_table, w.cu_seqlens_q, w.kv_lens, [dense], w.scale,
                 heads=list(range(heads)))
    dt = time.perf_counter() - t0
    flops = 4.0 * w.d * n_unmasked_head * heads
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads} of {w.hq} query heads, all {q_len} rows (fp64 NumPy), {dt:.1f} s",
            "seconds": round(dt, 2)}


def run_config(w, mask_name, steps, warmup, out_dtype, tile_q=128):
    import torch
    import masked_flash_attention_mask_amd as ma
    from workloads.device import device_inputs, plan_kwargs
    dev = device_inputs(w)
    kind, kw = plan_kwargs(w, mask_name)
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    plan = ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, tile_q=tile_q, **kw)
    torch.cuda.synchronize()
    compile_ms = (time.perf_counter() - t0) * 1e3
    out = torch.empty(dev["q"].shape, dtype=out_dtype, device="cuda")
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")

    def step():
        ma.attn_prefill_masked(plan, dev["q"], dev["k"], dev["v"], dev["pt"], w.scale, out=out, lse=lse)

    ms = time_steps(step, steps, warmup, stream)
    return ms, compile_ms, plan


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--all", action="store_true", help="also print lines for the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline kernel (no comparator, no CPU baseline): for profilers")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--decode", action="store_true", help="print only the decode lines")
    ap.add_argument("--classify", action="store_true",
                    help="print only the device mask-classify lines (block mask, packed and dense)")
    ap.add_argument("--backward", action="store_true", help="print only the backward lines")
    ap.add_argument("--fp8", action="store_true", help="print only the fp8 (e4m3) prefill lines")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
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

    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_each_way": n * 4}), flush=True)
        del src, dst

    seq, prefix, cs, hq, d = 16384, 1024, 2, 16, 128
    w = W.config4(seq=seq, prefix=prefix, hq=hq, d=d, chunk_sizes=(cs,))
    name = f"chunk{cs}"
    ms, compile_ms, _ = run_config(w, name, args.steps, args.warmup, torch.bfloat16)
    if args.headline_only:
        tf = 4.0 * d * hq * chunk_unmasked(seq, prefix, cs) / (ms * 1e-3) / 1e12
        print(json.dumps({"headline_ms": round(ms, 4), "tflops": round(tf, 2)}), flush=True)
        return
    n_unmasked = chunk_unmasked(seq, prefix, cs)
    flops = 4.0 * d * hq * n_unmasked
    tflops = flops / (ms * 1e-3) / 1e12
    causal_ms, _, _ = run_config(w, "causal", args.steps, args.warmup, torch.bfloat16)
    causal_tflops = 4.0 * d * hq * (seq * (seq + 1) // 2) / (causal_ms * 1e-3) / 1e12

    traffic = read_traffic()
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
        "config": {"workload": "chunk-causal interleaved (token, latent) pairs: 1 sequence x 16384 tokens, "
                               "1024-token causal prefix + 7680 pairs, chunk_size 2 as one CHUNK_CAUSAL range; "
                               "16 heads, head_dim 128, bf16 in/out, fp32 accumulation",
                   "global_batch": 1, "seq_len": seq, "heads": hq, "head_dim": d, "chunk_size": cs,
                   "parallelism": "single GPU"},
        "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "unmasked_entries_per_head": n_unmasked,
        "plan_compile_ms": round(compile_ms, 3),
        "causal_same_shape": {"ms": round(causal_ms, 4), "tflops": round(causal_tflops, 2),
                              "ratio_masked_over_causal": round(tflops / causal_tflops, 3)},
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "prefill_bf16_kernel<128,128,bf16>", "flops_per_launch": flops,
                     "timing": "HIP events on the launch stream around the timed steps; one kernel per step"},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, name, n_unmasked)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)

    if args.all:
        extra(args)
        decode_lines(args.steps, args.warmup)
        backward_lines(args.steps, args.warmup)
        fp8_lines(args.steps, args.warmup)


def extra(args):
    """One informational line per other workload (not the headline)."""
    import torch
    import workloads as W
    import masked_flash_attention_mask_amd as ma
    from workloads.device import device_inputs
    rows = []
    w = W.config4()
    for name in ("chunk4", "chunk16", "chunk2_full", "causal"):
        ms, cms, plan = run_config(w, name, args.steps, args.warmup, torch.bfloat16)
        rows.append(("cfg4", name, ms, cms, plan, w))
    w5 = W.config5()
    for name in ("custom_ranges", "custom_packed", "causal"):
        ms, cms, plan = run_config(w5, name, max(3, args.steps // 4), 2, torch.bfloat16)
        rows.append(("cfg5", name, ms, cms, plan, w5))
    w3a = W.config3a()
    for name in ("prefix_lm", "causal"):
        ms, cms, plan = run_config(w3a, name, args.steps, args.warmup, torch.bfloat16)
        rows.append(("cfg3a", name, ms, cms, plan, w3a))
    for layer in (0, 1):
        w3b = W.config3b(layer)
        name = "window" if layer == 0 else "causal"
        ms, cms, plan = run_config(w3b, name, args.steps, args.warmup, torch.bfloat16)
        rows.append((f"cfg3b_l{layer}", name, ms, cms, plan, w3b))
    for cfg, name, ms, cms, plan, w in rows:
        n = count_unmasked(w, name)
        tf = 4.0 * w.d * w.hq * n / (ms * 1e-3) / 1e12
        print(json.dumps({"workload": cfg, "mask": name, "ms": round(ms, 4), "tflops": round(tf, 2),
                          "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "compile_ms": round(cms, 3),
                          "unmasked_per_head": n}), flush=True)
    # tree verify
    w2 = W.config2()
    dev = device_inputs(w2)
    for form in ("tree_packed", "tree_dense"):
        import numpy as np
        mi = w2.masks[form]
        data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
        mask = torch.from_numpy(np.ascontiguousarray(data)).cuda()
        need = ma.attn_verify_tree_workspace(w2.batch, 64, int(w2.kv_lens.max()), w2.hq, w2.hkv, w2.d)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        out = torch.empty(dev["q"].shape, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")

        def step():
            ma.attn_verify_tree(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], mask, mi.kind, 64,
                                int(w2.kv_lens.max()), w2.scale, workspace=ws, out=out, lse=lse)
        ms = time_steps(step, 50, 10, torch.cuda.current_stream())
        n = sum(64 * int(c) for c in w2.info["ctx"]) + sum(
            int(np.sum([len(_anc(p, i)) for i in range(64)])) for p in w2.info["parents"])
        tf = 4.0 * w2.d * w2.hq * n / (ms * 1e-3) / 1e12
        kv_bytes = 2 * int(w2.kv_lens.sum()) * w2.hkv * w2.d * 2
        print(json.dumps({"workload": "cfg2", "mask": form, "ms": round(ms, 4), "tflops": round(tf, 2),
                          "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    # causal comparator at the same shape (the same queries, kernel and splits)
    need = ma.attn_decode_workspace(w2.batch, 64, int(w2.kv_lens.max()), w2.hq, w2.hkv, w2.d)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def cstep():
        ma.attn_decode(dev["q"], dev["k"], dev["v"], dev["pt"], dev["cu"], dev["kv"], 64, int(w2.kv_lens.max()),
                       w2.scale, mask_kind="causal", workspace=ws, out=out, lse=lse)
    ms = time_steps(cstep, 50, 10, torch.cuda.current_stream())
    n = sum(64 * int(c) + 64 * 65 // 2 for c in w2.info["ctx"])
    tf = 4.0 * w2.d * w2.hq * n / (ms * 1e-3) / 1e12
    print(json.dumps({"workload": "cfg2", "mask": "causal", "ms": round(ms, 4), "tflops": round(tf, 2),
                      "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1)}), flush=True)


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
    """Backward (dQ, dK, dV) of the headline workload and of causal at the
    same shape, each through its plan, forward outputs resident."""
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


def fp8_lines(steps, warmup):
    """fp8 (e4m3) prefill of the headline workload and of causal at the same
    shape: the bf16 inputs quantized per tensor, bf16 output."""
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


def classify_lines(steps):
    """Device mask classify (an HBM scan) on the 32768 x 29576 block mask,
    packed (121 MB) and dense (969 MB).  The wall time of mask_compile covers
    the host part too (metadata upload and a stream sync); the kernel's own
    time comes from a kernel trace."""
    import time
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


def _anc(parents, i):
    out = [i]
    while i != 0:
        i = int(parents[i])
        out.append(i)
    return out


def count_unmasked(w, name):
    import masked_flash_attention_mask_amd as ma
    from workloads.device import plan_kwargs
    import numpy as np
    kind, kw = plan_kwargs(w, name, host=True)
    plan = ma.mask_compile_host(kind, w.cu_seqlens_q, w.kv_lens, **kw)
    cls, words = plan.export()
    # FULL tiles: in-bounds area; PARTIAL tiles: popcount of the words.
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


if __name__ == "__main__":
    main()
