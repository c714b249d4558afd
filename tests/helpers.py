"""Shared plumbing for the GPU parity tests: device copies of a workload, the
library calls, the oracle's masks for the same inputs, and error metrics."""

import json
import os

import numpy as np
import torch

import masked_flash_attention_mask_amd as ma
from oracle import attention as OA
from workloads.device import device_inputs, plan_kwargs  # noqa: F401
from oracle import masks as OM

TOL_F32 = 1e-5      # fp32 inputs, fp32 accumulation
TOL_BF16 = 1.5e-2   # bf16 inputs, fp32 accumulation, fp32 output
# Backward (grad_err below): the kernels round P and dS to bf16 (unit
# roundoff u = 2^-9) before their products and accumulate in fp32, so each
# gradient element is off by about u times the RMS of its terms; 2^-5 = 16u
# leaves room for the max over a row against the row's RMS.  A wrong index,
# sign, scale or a dropped term moves a row by O(1) of its RMS.
TOL_GRAD = 2.0 ** -5


def parity_report(tag, **vals):
    """Appends one JSON line (the case and its measured errors) to the file
    that MASKATTN_PARITY_REPORT names, when it is set; does nothing
    otherwise.  The full-size cases call it so that one run of the GPU tests
    yields every configuration's error against the oracle."""
    path = os.environ.get("MASKATTN_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": tag, **{k: float(v) for k, v in vals.items()}}) + "\n")


def compile_plan(w, mask_name, tile_q=128, device_mask=True):
    kind, kw = plan_kwargs(w, mask_name, host=not device_mask)
    return ma.mask_compile(kind, w.cu_seqlens_q, w.kv_lens, tile_q=tile_q, **kw)


def run_prefill(w, dev_in, mask_name, tile_q=128, out_dtype=torch.float32, device_mask=True):
    plan = compile_plan(w, mask_name, tile_q, device_mask)
    out, lse = ma.attn_prefill_masked(plan, dev_in["q"], dev_in["k"], dev_in["v"], dev_in["pt"], w.scale,
                                      out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out, lse, plan


def oracle_masks(w, mask_name):
    mi = w.masks[mask_name]
    ql, kl = w.q_lens, w.kv_lens
    if mi.kind == "causal":
        return lambda b: OM.causal(int(ql[b]), int(kl[b]))
    if mi.kind == "window":
        return lambda b: OM.sliding_window(int(ql[b]), int(kl[b]), mi.window)
    if mi.kind == "prefix_lm":
        return lambda b: OM.prefix_lm(int(ql[b]), int(kl[b]), int(mi.prefix_len[b]))
    if mi.kind == "ranges":
        return lambda b: OM.ranges(int(ql[b]), int(kl[b]), mi.ranges[b])
    band = (lambda b: OM.window_band(int(ql[b]), int(kl[b]), mi.window)) if mi.window else None
    if mi.kind == "dense":
        lst = OM.dense_from_flat(mi.data, ql, kl)
        return (lambda b: lst[b] & band(b)) if band else (lambda b: lst[b])
    if mi.kind == "packed":
        lst = OM.packed_from_flat(mi.data, ql, kl)
        return (lambda b: lst[b] & band(b)) if band else (lambda b: lst[b])
    if mi.kind == "block_sparse":
        br, bc, indptr, indices = mi.bsr
        starts = np.concatenate([[0], np.cumsum([-(-int(q) // br) for q in ql])])

        def bsr(b):
            ip = indptr[starts[b]:starts[b + 1] + 1]
            m = OM.block_sparse(int(ql[b]), int(kl[b]), br, bc, ip, indices)
            return m & band(b) if band else m
        return bsr
    raise ValueError(mi.kind)


def oracle(w, mask_name, heads=None, rows=None):
    return OA.attention(w.q, w.k_cache, w.v_cache, w.page_table, w.cu_seqlens_q, w.kv_lens,
                        oracle_masks(w, mask_name), w.scale, heads=heads, rows=rows)


def max_abs_err(gpu, ref):
    g = gpu.float().cpu().numpy().astype(np.float64)
    sel = ~np.isnan(ref)
    assert not np.isnan(g[sel]).any(), "GPU output has NaN where the oracle has a value"
    return float(np.abs(g[sel] - ref[sel]).max()) if sel.any() else 0.0


def lse_err(gpu_lse, ref_lse):
    g = gpu_lse.cpu().numpy().astype(np.float64)
    sel = ~np.isnan(ref_lse)
    fin = sel & np.isfinite(ref_lse)
    assert np.array_equal(np.isneginf(g[sel]), np.isneginf(ref_lse[sel])), "fully masked rows differ"
    return float(np.abs(g[fin] - ref_lse[fin]).max()) if fin.any() else 0.0


def grad_err(gpu, ref):
    """Largest error of a gradient row (the last axis) relative to that row's
    reference RMS, plus a floor of 2^-8 of the whole tensor's RMS for rows
    whose exact gradient is (near) zero.  Rows the oracle left NaN (heads it
    did not compute) are skipped; every compared GPU value must be finite."""
    d = ref.shape[-1]
    g = gpu.float().cpu().numpy().astype(np.float64).reshape(-1, d)
    r = ref.reshape(-1, d)
    sel = ~np.isnan(r).any(axis=1)
    g, r = g[sel], r[sel]
    assert np.isfinite(g).all(), "GPU gradient has a non-finite value"
    rms_row = np.sqrt((r ** 2).mean(axis=1))
    floor = 2.0 ** -8 * np.sqrt((r ** 2).mean()) if r.size else 0.0
    if not r.size:
        return 0.0
    return float((np.abs(g - r).max(axis=1) / (rms_row + floor + 1e-30)).max())


def bf16_out_err(gpu_bf16, ref):
    """Error of a bf16 output against the oracle, less one bf16 rounding step
    of the reference value (the output rounding alone)."""
    g = gpu_bf16.float().cpu().numpy().astype(np.float64)
    sel = ~np.isnan(ref)
    r = ref[sel]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - 7)
    return float((np.abs(g[sel] - r) - ulp).max())


# ------------------------------------------------------------------- fp8 --
def fp8_dequantized(w, f8):
    """The workload with Q / K / V replaced by the exact values of their e4m3
    bytes times the descale factors (what the fp8 kernel computes with)."""
    import copy
    from oracle import fp8 as OF
    w2 = copy.copy(w)
    w2.q = OF.e4m3_decode(f8["q8"]) * f8["q_s"]
    w2.k_cache = OF.e4m3_decode(f8["k8"]) * f8["k_s"]
    w2.v_cache = OF.e4m3_decode(f8["v8"]) * f8["v_s"]
    return w2


def fp8_bound(q_rows, k, v, mask_rows, scale, o_ref):
    """Error bounds of the fp8 kernel for the given query rows of one head,
    returned as (per-element bound on O, per-row bound on LSE).

    The kernel's probabilities are rounded to e4m3: relative half-ulp 2^-4,
    absolute 2^-10 below the normal range, in units of the kernel's running
    reference maximum, which never exceeds the row's true maximum, so in units
    where the row's largest probability is 1 each rounding error is at most
    e_k = max(2^-4 p_k, 2^-10).  Then O moves by exactly
    sum_k eps_k (V_k - O) / sum_k p~_k; the bound is six standard deviations
    of that sum for independent errors (variance at most e_k^2 / 3), plus
    1e-3 for fp32 accumulation.  The row sum moves by at most sum_k e_k, which
    bounds the LSE error by that over sum_k p_k (with 5% slack) plus 1e-4."""
    s = scale * (q_rows @ k.T)
    s = np.where(mask_rows, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    has = np.isfinite(mx)
    p = np.where(mask_rows & has, np.exp(np.where(mask_rows & has, s - np.where(has, mx, 0.0), 0.0)), 0.0)
    e = np.where(mask_rows & has, np.maximum(2.0 ** -4 * p, 2.0 ** -10), 0.0)
    e2 = e ** 2
    # sum_k e_k^2 (V_kx - O_tx)^2, expanded into products
    var = (e2 @ v ** 2) - 2.0 * o_ref * (e2 @ v) + o_ref ** 2 * e2.sum(axis=1, keepdims=True)
    var = np.maximum(var, 0.0) / 3.0
    tot = np.maximum(p.sum(axis=1, keepdims=True), 1e-300)
    o_bound = 6.0 * np.sqrt(var) / tot + 1e-3
    lse_bound = 1.05 * e.sum(axis=1) / tot[:, 0] + 1e-4
    return o_bound, lse_bound


def repage(w, ps, seed):
    """The same workload with its K/V laid out in pages of ps keys, in a
    random page order (spare pages NaN)."""
    import copy
    c = copy.copy(w)
    rng = np.random.default_rng(seed)
    pages = [(int(k) + ps - 1) // ps for k in w.kv_lens]
    total = sum(pages) + 2
    perm = rng.permutation(total)
    c.k_cache = np.full((total, ps) + w.k_cache.shape[2:], np.nan, np.float32)
    c.v_cache = np.full_like(c.k_cache, np.nan)
    c.page_table = np.full((len(pages), max(pages)), perm[-1], np.int32)
    c.page_size = ps
    off = 0
    for b, kl in enumerate(w.kv_lens):
        j = np.arange(int(kl))
        src_p, src_s = w.page_table[b, j // w.page_size], j % w.page_size
        dst = perm[off + j // ps]
        c.k_cache[dst, j % ps] = w.k_cache[src_p, src_s]
        c.v_cache[dst, j % ps] = w.v_cache[src_p, src_s]
        c.page_table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    return c
