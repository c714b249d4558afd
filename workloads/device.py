"""Device copies of a workload and the mask arguments a caller would pass to
mask_compile (plumbing only; no arithmetic of the method)."""

import numpy as np


def device_inputs(w, dev="cuda"):
    import torch
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    return {
        "q": torch.from_numpy(w.q).to(dev).to(dt).contiguous(),
        "k": torch.from_numpy(w.k_cache).to(dev).to(dt).contiguous(),
        "v": torch.from_numpy(w.v_cache).to(dev).to(dt).contiguous(),
        "pt": torch.from_numpy(w.page_table).to(dev).contiguous(),
        "cu": torch.from_numpy(w.cu_seqlens_q).to(dev).contiguous(),
        "kv": torch.from_numpy(w.kv_lens).to(dev).contiguous(),
    }


def plan_kwargs(w, mask_name, host=False):
    """(kind, kwargs) for mask_compile; dense / packed masks go to the device
    unless host=True."""
    mi = w.masks[mask_name]
    kw = {}
    if mi.kind == "window":
        kw["window"] = mi.window
    elif mi.kind == "prefix_lm":
        kw["prefix_len"] = mi.prefix_len
    elif mi.kind == "ranges":
        kw["ranges"] = mi.ranges
    elif mi.kind == "block_sparse":
        kw["bsr"] = mi.bsr
        if mi.window:
            kw["window"] = mi.window
    elif mi.kind in ("dense", "packed"):
        if mi.window:
            kw["window"] = mi.window
        if host:
            kw["mask"] = mi.data
        else:
            import torch
            data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
            kw["mask"] = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    return mi.kind, kw
