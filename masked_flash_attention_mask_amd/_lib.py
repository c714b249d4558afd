"""ctypes binding of libmaskattn.so: argument marshalling only.

Every function here converts Python / torch arguments into the C ABI's plain
pointers and sizes and calls the library; none computes any part of the
attention or the mask.  The library must have been built (see build.py); a
missing library raises at import of this module, there is no fallback.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmaskattn.so")

MA_OK, MA_ERR_INVALID, MA_ERR_CONFLICT, MA_ERR_SIZE = 0, -1, -2, -3
MA_ERR_UNSUPPORTED, MA_ERR_PLAN_MISMATCH, MA_ERR_HIP, MA_ERR_NOMEM = -4, -5, -6, -7
RANGE_FULL, RANGE_CAUSAL, RANGE_INV_CAUSAL, RANGE_BI_CAUSAL, RANGE_CHUNK_CAUSAL = 0, 1, 2, 3, 4
KIND = {"causal": 0, "window": 1, "prefix_lm": 2, "ranges": 3, "dense": 4, "packed": 5, "block_sparse": 6}
F32, BF16 = 0, 1
TILE_SKIP, TILE_FULL, TILE_PARTIAL = 0, 1, 2

EXPORTS = ["mask_compile", "mask_compile_host", "mask_plan_upload", "mask_plan_destroy",
           "mask_plan_info_get", "mask_plan_export", "mask_plan_serialize", "attn_prefill_masked",
           "attn_prefill_masked_fp8", "attn_backward_workspace", "attn_backward_masked", "attn_verify_tree_workspace", "attn_verify_tree",
           "attn_verify_tree_noalloc",
           "attn_decode_workspace", "attn_decode", "attn_decode_kv8",
           "ma_status_string", "ma_last_error"]


class MaRange(ctypes.Structure):
    _fields_ = [("q_start", ctypes.c_int32), ("q_end", ctypes.c_int32), ("k_start", ctypes.c_int32),
                ("k_end", ctypes.c_int32), ("type", ctypes.c_int32), ("chunk_size", ctypes.c_int32)]


class MaMaskDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("cu_seqlens_q", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
                ("window", ctypes.c_int32), ("prefix_len", ctypes.c_void_p),
                ("ranges", ctypes.c_void_p), ("range_indptr", ctypes.c_void_p),
                ("mask", ctypes.c_void_p), ("mask_numel", ctypes.c_int64),
                ("mask_on_device", ctypes.c_int32), ("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("block_r", ctypes.c_int32), ("block_c", ctypes.c_int32),
                ("bsr_indptr", ctypes.c_void_p), ("bsr_indices", ctypes.c_void_p)]


class MaPlanInfo(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("num_qtiles", ctypes.c_int32), ("num_tiles", ctypes.c_int64),
                ("num_entries", ctypes.c_int64), ("num_word_blocks", ctypes.c_int64),
                ("total_q", ctypes.c_int64), ("device_bytes", ctypes.c_int64),
                ("on_device", ctypes.c_int32), ("host_valid", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with masked_flash_attention_mask_amd.build.build()")
    # torch brings its own HIP runtime.  Load it first so that the library's
    # libamdhip64 dependency resolves to that same runtime: two HIP runtimes
    # in one process do not share the device, and the second finds none.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "mask_compile": (i32, [vp, vp, pp]),
        "mask_compile_host": (i32, [vp, pp]),
        "mask_plan_upload": (i32, [vp, vp]),
        "mask_plan_destroy": (i32, [vp]),
        "mask_plan_info_get": (i32, [vp, vp]),
        "mask_plan_export": (i32, [vp, vp, vp]),
        "mask_plan_serialize": (i32, [vp, vp, ctypes.POINTER(sz)]),
        "attn_prefill_masked": (i32, [vp, vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, i32, i32, i32, f32,
                                      vp, vp, vp]),
        "attn_prefill_masked_fp8": (i32, [vp, vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, i32, f32, f32, f32, i32,
                                          f32, vp, vp, vp]),
        "attn_backward_workspace": (sz, [vp, i32]),
        "attn_backward_masked": (i32, [vp, vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, i32, vp, i32, vp, vp, f32,
                                       vp, vp, vp, vp, sz, vp]),
        "attn_verify_tree_workspace": (sz, [i32, i32, i32, i32, i32, i32]),
        "attn_verify_tree": (i32, [vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, i32, i32, i32,
                                   i32, vp, i64, i32, i32, f32, vp, sz, vp, vp, vp]),
        "attn_verify_tree_noalloc": (i32, [vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, i32, i32, i32,
                                           i32, vp, i64, i32, i32, f32, vp, vp, vp]),
        "attn_decode_workspace": (sz, [i32, i32, i32, i32, i32, i32]),
        "attn_decode": (i32, [vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                              vp, vp, i64, i32, i32, f32, vp, sz, vp, vp, vp]),
        "attn_decode_kv8": (i32, [vp, i64, i32, vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32,
                                  i32, vp, vp, i64, i32, f32, f32, f32, vp, sz, vp, vp, vp]),
        "ma_status_string": (ctypes.c_char_p, [i32]),
        "ma_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


class MaskAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = LIB.ma_last_error().decode() or LIB.ma_status_string(status).decode()
        super().__init__(f"{where}: {LIB.ma_status_string(status).decode()} ({status}): {msg}")


def check(status, where):
    if status != MA_OK:
        raise MaskAttnError(status, where)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(arr):
    return None if arr is None else arr.ctypes.data_as(ctypes.c_void_p)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Plan:
    """Owns one ma_plan handle."""

    def __init__(self, handle, keep):
        self.handle = handle
        self._keep = keep   # the host arrays the description pointed at

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h:
            LIB.mask_plan_destroy(h)

    def info(self):
        out = MaPlanInfo()
        check(LIB.mask_plan_info_get(self.handle, ctypes.byref(out)), "mask_plan_info_get")
        return out

    def export(self, words=True):
        """(classes uint8 [num_tiles], words uint64 [num_tiles, tile_q] or None)."""
        inf = self.info()
        cls = np.zeros(inf.num_tiles, dtype=np.uint8)
        w = np.zeros((inf.num_tiles, inf.tile_q * inf.tile_k // 64), dtype=np.uint64) if words else None
        check(LIB.mask_plan_export(self.handle, _ptr(cls), _ptr(w)), "mask_plan_export")
        return cls, w

    def serialize(self):
        n = ctypes.c_size_t(0)
        check(LIB.mask_plan_serialize(self.handle, None, ctypes.byref(n)), "mask_plan_serialize")
        buf = np.zeros(n.value, dtype=np.uint8)
        check(LIB.mask_plan_serialize(self.handle, _ptr(buf), ctypes.byref(n)), "mask_plan_serialize")
        return buf.tobytes()

    def upload(self, stream=None):
        check(LIB.mask_plan_upload(self.handle, _stream(stream)), "mask_plan_upload")


def make_desc(kind, cu_seqlens_q, kv_lens, window=0, prefix_len=None, ranges=None, mask=None,
              tile_q=128, tile_k=64, bsr=None):
    """Builds the C mask description; returns (desc, arrays to keep alive).
    bsr = (block_r, block_c, indptr, indices) for the block-sparse kind (the
    block rows of all sequences concatenated, column indices per sequence)."""
    cu = _i32(cu_seqlens_q)
    kv = _i32(kv_lens)
    keep = [cu, kv]
    d = MaMaskDesc()
    d.kind = KIND[kind] if isinstance(kind, str) else int(kind)
    d.batch = len(kv)
    d.cu_seqlens_q = _ptr(cu)
    d.kv_lens = _ptr(kv)
    d.window = int(window)
    d.tile_q = tile_q
    d.tile_k = tile_k
    if prefix_len is not None:
        pl = _i32(prefix_len)
        keep.append(pl)
        d.prefix_len = _ptr(pl)
    if ranges is not None:
        flat = [r for seq in ranges for r in seq]
        indptr = _i32(np.concatenate([[0], np.cumsum([len(s) for s in ranges])]))
        arr = (MaRange * max(1, len(flat)))(*[MaRange(*map(int, r)) for r in flat])
        keep += [indptr, arr]
        d.ranges = ctypes.cast(arr, ctypes.c_void_p)
        d.range_indptr = _ptr(indptr)
    if bsr is not None:
        br, bc, indptr, indices = bsr
        ip, ix = _i32(indptr), _i32(indices)
        keep += [ip, ix]
        d.block_r, d.block_c = int(br), int(bc)
        d.bsr_indptr = _ptr(ip)
        d.bsr_indices = _ptr(ix) if ix.size else None
    if mask is not None:
        if hasattr(mask, "is_cuda"):
            d.mask = ctypes.c_void_p(mask.data_ptr())
            d.mask_numel = mask.numel()
            d.mask_on_device = 1 if mask.is_cuda else 0
            keep.append(mask)
        else:
            m = np.ascontiguousarray(mask)
            keep.append(m)
            d.mask = _ptr(m)
            d.mask_numel = m.size
            d.mask_on_device = 0
    return d, keep


def mask_compile_host(kind, cu_seqlens_q, kv_lens, **kw):
    desc, keep = make_desc(kind, cu_seqlens_q, kv_lens, **kw)
    h = ctypes.c_void_p()
    check(LIB.mask_compile_host(ctypes.byref(desc), ctypes.byref(h)), "mask_compile_host")
    return Plan(h.value, keep)


def mask_compile(kind, cu_seqlens_q, kv_lens, stream=None, **kw):
    desc, keep = make_desc(kind, cu_seqlens_q, kv_lens, **kw)
    h = ctypes.c_void_p()
    check(LIB.mask_compile(ctypes.byref(desc), _stream(stream), ctypes.byref(h)), "mask_compile")
    return Plan(h.value, keep)


def _dtype_code(t):
    import torch
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t}")


def _cache_args(k_cache, v_cache):
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride():
        raise ValueError("k_cache and v_cache must share shape [pages, page_size, Hkv, d] and strides")
    if k_cache.stride(3) != 1:
        raise ValueError("the head dimension of the caches must be contiguous")
    strides = (ctypes.c_int64 * 3)(k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))
    return strides


def attn_prefill_masked(plan, q, k_cache, v_cache, page_table, scale, out=None, lse=None,
                        out_dtype=None, stream=None):
    """q [total_q, Hq, d]; caches [pages, page_size, Hkv, d]; page_table int32
    [batch, max_pages].  Returns (out, lse)."""
    import torch
    if not q.is_contiguous() or not page_table.is_contiguous() or page_table.dtype != torch.int32:
        raise ValueError("q must be contiguous and page_table a contiguous int32 tensor")
    total_q, hq, d = q.shape
    hkv, page_size = k_cache.shape[2], k_cache.shape[1]
    strides = _cache_args(k_cache, v_cache)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    st = LIB.attn_prefill_masked(
        plan.handle, q.data_ptr(), total_q, hq, k_cache.data_ptr(), v_cache.data_ptr(), hkv, d, page_size,
        strides, page_table.data_ptr(), page_table.shape[1], _dtype_code(q.dtype), _dtype_code(out.dtype),
        float(scale), out.data_ptr(), lse.data_ptr() if lse is not False else None, _stream(stream))
    check(st, "attn_prefill_masked")
    return out, lse


def attn_prefill_masked_fp8(plan, q8, k8, v8, page_table, scale, q_descale, k_descale, v_descale, out=None,
                            lse=None, out_dtype=None, stream=None):
    """fp8 (e4m3) prefill: q8 [total_q, Hq, d], k8 / v8 [pages, page_size, Hkv, d]
    as uint8 (or float8_e4m3fn) device tensors; per-tensor descale factors.
    Returns (out, lse); out is bf16 unless out_dtype says otherwise."""
    import torch
    if not q8.is_contiguous() or not page_table.is_contiguous() or page_table.dtype != torch.int32:
        raise ValueError("q must be contiguous and page_table a contiguous int32 tensor")
    for t in (q8, k8, v8):
        if t.element_size() != 1:
            raise ValueError("fp8 inputs must be one-byte tensors")
    total_q, hq, d = q8.shape
    hkv, page_size = k8.shape[2], k8.shape[1]
    strides = _cache_args(k8, v8)
    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype, device=q8.device)
    if lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q8.device)
    st = LIB.attn_prefill_masked_fp8(
        plan.handle, q8.data_ptr(), total_q, hq, k8.data_ptr(), v8.data_ptr(), hkv, d, page_size, strides,
        page_table.data_ptr(), page_table.shape[1], float(q_descale), float(k_descale), float(v_descale),
        _dtype_code(out.dtype), float(scale), out.data_ptr(), lse.data_ptr() if lse is not False else None,
        _stream(stream))
    check(st, "attn_prefill_masked_fp8")
    return out, lse


def attn_backward_workspace(plan, hq):
    return int(LIB.attn_backward_workspace(plan.handle, hq))


def attn_backward_masked(plan, q, k_cache, v_cache, page_table, out, lse, dout, scale, dq=None, dk_cache=None,
                         dv_cache=None, workspace=None, stream=None):
    """Gradients of attn_prefill_masked given its out and lse and the upstream
    gradient dout (bf16, like q).  Returns fp32 (dq [total_q, Hq, d],
    dk_cache, dv_cache); the caches take k_cache's shape and strides, and
    slots of no key are left as passed (zero when allocated here)."""
    import torch
    for t in (q, page_table, out, lse, dout):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("backward tensors must be contiguous device tensors")
    if dout.shape != q.shape or dout.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("out and dout must match q's shape (dout also its dtype)")
    total_q, hq, d = q.shape
    hkv, page_size = k_cache.shape[2], k_cache.shape[1]
    strides = _cache_args(k_cache, v_cache)
    if dq is None:
        dq = torch.empty((total_q, hq, d), dtype=torch.float32, device=q.device)
    grads = []
    for g in (dk_cache, dv_cache):
        if g is None:
            g = torch.zeros_like(k_cache, dtype=torch.float32)
        if g.dtype != torch.float32 or g.shape != k_cache.shape or g.stride() != k_cache.stride():
            raise ValueError("dk_cache and dv_cache must be fp32 with k_cache's shape and strides")
        grads.append(g)
    need = attn_backward_workspace(plan, hq)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.attn_backward_masked(
        plan.handle, q.data_ptr(), total_q, hq, k_cache.data_ptr(), v_cache.data_ptr(), hkv, d, page_size, strides,
        page_table.data_ptr(), page_table.shape[1], out.data_ptr(), _dtype_code(out.dtype), dout.data_ptr(),
        lse.data_ptr(), float(scale), dq.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(), ws_ptr, ws_bytes,
        _stream(stream))
    check(st, "attn_backward_masked")
    return dq, grads[0], grads[1]


def attn_verify_tree_workspace(batch, max_q, max_kv, hq, hkv, d):
    return int(LIB.attn_verify_tree_workspace(batch, max_q, max_kv, hq, hkv, d))


def attn_verify_tree(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, mask, mask_kind, max_q, max_kv,
                     scale, workspace=None, out=None, lse=None, out_dtype=None, stream=None):
    """Tree verify with lengths and mask on the device.  mask_kind: 'dense'
    (uint8 rows) or 'packed' (int64/uint64 words)."""
    import torch
    total_q, hq, d = q.shape
    hkv, page_size = k_cache.shape[2], k_cache.shape[1]
    batch = kv_lens.shape[0]
    strides = _cache_args(k_cache, v_cache)
    for t in (q, page_table, cu_seqlens_q, kv_lens, mask):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("verify tensors must be contiguous device tensors")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    need = attn_verify_tree_workspace(batch, max_q, max_kv, hq, hkv, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = LIB.attn_verify_tree(
        q.data_ptr(), total_q, hq, k_cache.data_ptr(), v_cache.data_ptr(), hkv, d, page_size, strides,
        page_table.data_ptr(), page_table.shape[1], cu_seqlens_q.data_ptr(), kv_lens.data_ptr(), batch,
        int(max_q), int(max_kv), KIND[mask_kind], mask.data_ptr(), mask.numel(), _dtype_code(q.dtype),
        _dtype_code(out.dtype), float(scale), ws_ptr, ws_bytes, out.data_ptr(),
        lse.data_ptr() if lse is not False else None, _stream(stream))
    check(st, "attn_verify_tree")
    return out, lse


def attn_verify_tree_noalloc(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, mask, mask_kind, max_q,
                             max_kv, scale, out=None, lse=None, out_dtype=None, stream=None):
    """attn_verify_tree on the library's own per-GPU scratch (no workspace
    argument; the library allocates nothing during the call)."""
    import torch
    total_q, hq, d = q.shape
    hkv, page_size = k_cache.shape[2], k_cache.shape[1]
    batch = kv_lens.shape[0]
    strides = _cache_args(k_cache, v_cache)
    for t in (q, page_table, cu_seqlens_q, kv_lens, mask):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("verify tensors must be contiguous device tensors")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    st = LIB.attn_verify_tree_noalloc(
        q.data_ptr(), total_q, hq, k_cache.data_ptr(), v_cache.data_ptr(), hkv, d, page_size, strides,
        page_table.data_ptr(), page_table.shape[1], cu_seqlens_q.data_ptr(), kv_lens.data_ptr(), batch,
        int(max_q), int(max_kv), KIND[mask_kind], mask.data_ptr(), mask.numel(), _dtype_code(q.dtype),
        _dtype_code(out.dtype), float(scale), out.data_ptr(), lse.data_ptr() if lse is not False else None,
        _stream(stream))
    check(st, "attn_verify_tree_noalloc")
    return out, lse


def attn_decode_workspace(batch, max_q, max_kv, hq, hkv, d):
    return int(LIB.attn_decode_workspace(batch, max_q, max_kv, hq, hkv, d))


def attn_decode(q, k_cache, v_cache, page_table, cu_seqlens_q, kv_lens, max_q, max_kv, scale, mask_kind="causal",
                window=0, prefix_len=None, mask=None, workspace=None, out=None, lse=None, out_dtype=None,
                stream=None):
    """Masked decode with lengths on the device.  mask_kind: 'causal',
    'window' (window >= 1), 'prefix_lm' (prefix_len: device int32 [batch]),
    'dense' (uint8 rows) or 'packed' (int64/uint64 words)."""
    import torch
    total_q, hq, d = q.shape
    hkv, page_size = k_cache.shape[2], k_cache.shape[1]
    batch = kv_lens.shape[0]
    strides = _cache_args(k_cache, v_cache)
    for t in (q, page_table, cu_seqlens_q, kv_lens) + tuple(x for x in (mask, prefix_len) if x is not None):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("decode tensors must be contiguous device tensors")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace(batch, max_q, max_kv, hq, hkv, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    kind = {"window": KIND["window"], "sliding_window": KIND["window"]}.get(mask_kind, KIND.get(mask_kind))
    if kind is None:
        raise ValueError(f"unknown mask kind {mask_kind!r}")
    st = LIB.attn_decode(
        q.data_ptr(), total_q, hq, k_cache.data_ptr(), v_cache.data_ptr(), hkv, d, page_size, strides,
        page_table.data_ptr(), page_table.shape[1], cu_seqlens_q.data_ptr(), kv_lens.data_ptr(), batch,
        int(max_q), int(max_kv), kind, int(window), prefix_len.data_ptr() if prefix_len is not None else None,
        mask.data_ptr() if mask is not None else None, mask.numel() if mask is not None else 0,
        _dtype_code(q.dtype), _dtype_code(out.dtype), float(scale), ws_ptr, ws_bytes, out.data_ptr(),
        lse.data_ptr() if lse is not False else None, _stream(stream))
    check(st, "attn_decode")
    return out, lse


def attn_decode_kv8(q, k8_cache, v8_cache, page_table, cu_seqlens_q, kv_lens, max_q, max_kv, scale, k_descale,
                    v_descale, mask_kind="causal", window=0, prefix_len=None, mask=None, workspace=None, out=None,
                    lse=None, out_dtype=None, stream=None):
    """attn_decode with e4m3 K/V caches (uint8 tensors of the cache shape,
    K = k_descale * decode(K8), likewise V) and bf16 queries."""
    import torch
    total_q, hq, d = q.shape
    hkv, page_size = k8_cache.shape[2], k8_cache.shape[1]
    batch = kv_lens.shape[0]
    if k8_cache.dtype != torch.uint8 or v8_cache.dtype != torch.uint8:
        raise ValueError("fp8 caches must be uint8 tensors of e4m3 bytes")
    strides = _cache_args(k8_cache, v8_cache)
    for t in (q, page_table, cu_seqlens_q, kv_lens) + tuple(x for x in (mask, prefix_len) if x is not None):
        if not t.is_contiguous() or not t.is_cuda:
            raise ValueError("decode tensors must be contiguous device tensors")
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((total_q, hq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace(batch, max_q, max_kv, hq, hkv, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    kind = {"window": KIND["window"], "sliding_window": KIND["window"]}.get(mask_kind, KIND.get(mask_kind))
    if kind is None:
        raise ValueError(f"unknown mask kind {mask_kind!r}")
    st = LIB.attn_decode_kv8(
        q.data_ptr(), total_q, hq, k8_cache.data_ptr(), v8_cache.data_ptr(), hkv, d, page_size, strides,
        page_table.data_ptr(), page_table.shape[1], cu_seqlens_q.data_ptr(), kv_lens.data_ptr(), batch,
        int(max_q), int(max_kv), kind, int(window), prefix_len.data_ptr() if prefix_len is not None else None,
        mask.data_ptr() if mask is not None else None, mask.numel() if mask is not None else 0,
        _dtype_code(out.dtype), float(scale), float(k_descale), float(v_descale), ws_ptr, ws_bytes,
        out.data_ptr(), lse.data_ptr() if lse is not False else None, _stream(stream))
    check(st, "attn_decode_kv8")
    return out, lse
