"""C ABI surface without a GPU: every declared symbol is exported, and every
argument check fires on the host before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

import masked_flash_attention_mask_amd as ma
from masked_flash_attention_mask_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "maskattn.h")


def test_header_symbols_exported():
    text = open(HEADER).read()
    names = re.findall(r"^(?:ma_status|size_t|const char \*)\s*\*?(\w+)\(", text, flags=re.M)
    assert len(names) >= 12
    assert sorted(names) == sorted(L.EXPORTS)
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _status(fn):
    with pytest.raises(ma.MaskAttnError) as e:
        fn()
    return e.value.status


def test_mask_validation_rules():
    cu, kv = [0, 8], [8]
    # a sliding window needs the causal kind (sglang-jax review comment)
    assert _status(lambda: ma.mask_compile_host("prefix_lm", cu, kv, window=4, prefix_len=[2])) == L.MA_ERR_CONFLICT
    assert _status(lambda: ma.mask_compile_host("causal", cu, kv, window=4)) == L.MA_ERR_CONFLICT
    # a custom mask together with causal is rejected (reference implementation rule)
    m = np.ones(64, np.uint8)
    assert _status(lambda: ma.mask_compile_host("causal", cu, kv, mask=m)) == L.MA_ERR_CONFLICT
    assert _status(lambda: ma.mask_compile_host("causal", cu, kv, ranges=[[]])) == L.MA_ERR_CONFLICT
    # custom mask smaller than its sequences (size check)
    assert _status(lambda: ma.mask_compile_host("dense", cu, kv, mask=m[:63])) == L.MA_ERR_SIZE
    assert _status(lambda: ma.mask_compile_host("packed", [0, 8, 10], [8, 70],
                                               mask=np.zeros(11, np.uint64))) == L.MA_ERR_SIZE
    ma.mask_compile_host("packed", [0, 8, 10], [8, 70], mask=np.zeros(12, np.uint64))
    # bounds and parameters
    assert _status(lambda: ma.mask_compile_host("window", cu, kv, window=0)) == L.MA_ERR_INVALID
    assert _status(lambda: ma.mask_compile_host("prefix_lm", cu, kv, prefix_len=[9])) == L.MA_ERR_INVALID
    assert _status(lambda: ma.mask_compile_host("ranges", cu, kv, ranges=[[(0, 9, 0, 8, 0, 0)]])) == L.MA_ERR_INVALID
    assert _status(lambda: ma.mask_compile_host("ranges", cu, kv, ranges=[[(0, 8, 0, 8, 4, 0)]])) == L.MA_ERR_INVALID
    assert _status(lambda: ma.mask_compile_host("ranges", cu, kv, ranges=[[(0, 8, 0, 8, 7, 0)]])) == L.MA_ERR_INVALID
    assert _status(lambda: ma.mask_compile_host("causal", [1, 8], kv)) == L.MA_ERR_INVALID
    assert _status(lambda: ma.mask_compile_host("causal", [0, 8, 4], [8, 8])) == L.MA_ERR_INVALID
    assert _status(lambda: ma.mask_compile_host("causal", cu, kv, tile_q=32)) == L.MA_ERR_UNSUPPORTED
    assert _status(lambda: ma.mask_compile_host("causal", cu, kv, tile_k=128)) == L.MA_ERR_UNSUPPORTED
    assert "window" in L.LIB.ma_last_error().decode() or True


def test_empty_and_degenerate_plans():
    # zero-length sequences and empty range lists compile
    p = ma.mask_compile_host("causal", [0, 0, 5], [0, 5])
    assert p.info().num_qtiles == 1
    p = ma.mask_compile_host("ranges", [0, 5], [7], ranges=[[]])
    cls, _ = p.export()
    assert (cls == ma.TILE_SKIP).all()
    data = np.frombuffer(p.serialize(), dtype=np.int32)
    assert data[4 + 2] == 0    # the q-tile has no tiles to visit


FAKE = ctypes.c_void_p(0x1000)


def _prefill(plan, total_q=8, hq=2, hkv=1, d=128, page=16, strides=(2048, 128, 128), maxp=1,
             in_dt=L.BF16, out_dt=L.BF16, scale=0.1, q=FAKE):
    st = (ctypes.c_int64 * 3)(*strides)
    return L.LIB.attn_prefill_masked(plan.handle if plan else None, q, total_q, hq, FAKE, FAKE, hkv, d, page,
                                     st, FAKE, maxp, in_dt, out_dt, scale, FAKE, None, None)


def test_prefill_validation_before_hip():
    plan = ma.mask_compile_host("causal", [0, 8], [8])
    assert _prefill(None) == L.MA_ERR_INVALID
    assert _prefill(plan, q=None) == L.MA_ERR_INVALID
    assert _prefill(plan, total_q=9) == L.MA_ERR_PLAN_MISMATCH
    assert _prefill(plan, hq=3, hkv=2) == L.MA_ERR_INVALID
    assert _prefill(plan, d=96) == L.MA_ERR_UNSUPPORTED
    assert _prefill(plan, d=256, in_dt=L.F32, out_dt=L.F32) == L.MA_ERR_UNSUPPORTED
    assert _prefill(plan, in_dt=L.F32, out_dt=L.BF16, d=64) == L.MA_ERR_UNSUPPORTED
    assert _prefill(plan, page=12) == L.MA_ERR_UNSUPPORTED
    assert _prefill(plan, page=4, maxp=1) == L.MA_ERR_INVALID       # 4 keys < kv_len 8
    assert _prefill(plan, scale=0.0) == L.MA_ERR_INVALID
    assert _prefill(plan, scale=float("nan")) == L.MA_ERR_INVALID
    assert _prefill(plan, strides=(2048, 128, 64)) == L.MA_ERR_INVALID   # head stride < d
    assert plan.info().on_device == 0       # nothing was uploaded


def _verify(kind=L.KIND["packed"], max_q=64, ws=None, ws_bytes=0, d=128, in_dt=L.BF16, batch=2, max_kv=4000,
            numel=1000):
    st = (ctypes.c_int64 * 3)(2048, 128, 128)
    return L.LIB.attn_verify_tree(FAKE, 128, 4, FAKE, FAKE, 1, d, 16, st, FAKE, 300, FAKE, FAKE, batch, max_q,
                                  max_kv, kind, FAKE, numel, in_dt, L.F32, 0.1, ws, ws_bytes, FAKE, None, None)


def test_verify_validation_before_hip():
    assert _verify(kind=L.KIND["causal"]) == L.MA_ERR_CONFLICT
    assert _verify(max_q=65) == L.MA_ERR_UNSUPPORTED
    assert _verify(d=96) == L.MA_ERR_UNSUPPORTED
    assert _verify(in_dt=L.F32) == L.MA_ERR_UNSUPPORTED
    need = ma.attn_verify_tree_workspace(2, 64, 4000, 4, 1, 128)
    assert need > 0
    assert _verify(ws=FAKE, ws_bytes=need - 1) == L.MA_ERR_SIZE
    assert ma.attn_verify_tree_workspace(0, 64, 4000, 4, 1, 128) == 0


def test_short_custom_mask_is_a_size_error():
    """Lengths are on the device, so the host checks the one bound it can: a
    dense or packed mask needs an element per query row (128 rows here);
    shorter masks are MA_ERR_SIZE before any HIP call, for tree verify and
    decode alike.  (Elements past mask_numel of a longer mask read as 0, i.e.
    masked; the GPU tests check that.)"""
    need = ma.attn_verify_tree_workspace(2, 64, 4000, 4, 1, 128)
    for kind in (L.KIND["packed"], L.KIND["dense"]):
        assert _verify(kind=kind, numel=127, ws=FAKE, ws_bytes=need) == L.MA_ERR_SIZE
        assert _verify(kind=kind, numel=0, ws=FAKE, ws_bytes=need) == L.MA_ERR_INVALID
    dneed = ma.attn_decode_workspace(2, 1, 4000, 4, 1, 128)
    for kind in (L.KIND["packed"], L.KIND["dense"]):
        assert _decode(kind=kind, mask=FAKE, numel=1, ws=FAKE, ws_bytes=dneed) == L.MA_ERR_SIZE   # 2 rows


def _decode(kind=L.KIND["causal"], window=0, prefix=None, mask=None, numel=0, max_q=1, ws=None, ws_bytes=0,
            d=128, in_dt=L.BF16, batch=2, max_kv=4000):
    st = (ctypes.c_int64 * 3)(2048, 128, 128)
    return L.LIB.attn_decode(FAKE, 2, 4, FAKE, FAKE, 1, d, 16, st, FAKE, 300, FAKE, FAKE, batch, max_q, max_kv,
                             kind, window, prefix, mask, numel, in_dt, L.F32, 0.1, ws, ws_bytes, FAKE, None, None)


def test_decode_validation_before_hip():
    need = ma.attn_decode_workspace(2, 1, 4000, 4, 1, 128)
    assert need > 0
    ok = dict(ws=FAKE, ws_bytes=need)
    assert _decode(kind=L.KIND["window"], window=0, **ok) == L.MA_ERR_INVALID
    assert _decode(kind=L.KIND["prefix_lm"], prefix=None, **ok) == L.MA_ERR_INVALID
    assert _decode(kind=L.KIND["dense"], mask=None, **ok) == L.MA_ERR_INVALID
    assert _decode(kind=L.KIND["ranges"], **ok) == L.MA_ERR_UNSUPPORTED
    assert _decode(kind=17, **ok) == L.MA_ERR_INVALID
    assert _decode(max_q=65, **ok) == L.MA_ERR_UNSUPPORTED
    assert _decode(d=96, **ok) == L.MA_ERR_UNSUPPORTED
    assert _decode(in_dt=L.F32, **ok) == L.MA_ERR_UNSUPPORTED
    assert _decode(ws=FAKE, ws_bytes=need - 1) == L.MA_ERR_SIZE
    assert ma.attn_decode_workspace(2, 65, 4000, 4, 1, 128) == 0
    # the same bound serves tree verify: a 64-row tree needs more than decode
    assert ma.attn_verify_tree_workspace(2, 64, 4000, 4, 1, 128) >= need


def _decode8(kind=L.KIND["causal"], window=0, ks=1.0, vs=1.0, page=16, d=128, ws=None, ws_bytes=0,
             strides=(2048, 128, 128)):
    st = (ctypes.c_int64 * 3)(*strides)
    maxp = (4000 + page - 1) // page
    return L.LIB.attn_decode_kv8(FAKE, 2, 4, FAKE, FAKE, 1, d, page, st, FAKE, maxp, FAKE, FAKE, 2, 1, 4000, kind,
                                 window, None, None, 0, L.F32, 0.1, ks, vs, ws, ws_bytes, FAKE, None, None)


def test_decode_kv8_validation_before_hip():
    need = ma.attn_decode_workspace(2, 1, 4000, 4, 1, 128)
    ok = dict(ws=FAKE, ws_bytes=need)
    assert _decode8(ks=0.0, **ok) == L.MA_ERR_INVALID
    assert _decode8(vs=-1.0, **ok) == L.MA_ERR_INVALID
    assert _decode8(ks=float("inf"), **ok) == L.MA_ERR_INVALID
    assert _decode8(vs=float("nan"), **ok) == L.MA_ERR_INVALID
    assert _decode8(page=4, **ok) == L.MA_ERR_UNSUPPORTED          # fewer than 1024 / d keys per page
    assert _decode8(d=64, page=8, **ok) == L.MA_ERR_UNSUPPORTED
    assert _decode8(strides=(1 << 32, 128, 128), **ok) == L.MA_ERR_UNSUPPORTED
    assert _decode8(kind=L.KIND["window"], window=0, **ok) == L.MA_ERR_INVALID
    assert _decode8(kind=L.KIND["ranges"], **ok) == L.MA_ERR_UNSUPPORTED
    assert _decode8(ws=FAKE, ws_bytes=need - 1) == L.MA_ERR_SIZE


def _backward(plan, d=128, out_dt=L.BF16, total_q=8, ws=FAKE, ws_bytes=1 << 20, dout=FAKE, lse=FAKE, maxp=300):
    st = (ctypes.c_int64 * 3)(2048, 128, 128)
    return L.LIB.attn_backward_masked(plan.handle if plan else None, FAKE, total_q, 4, FAKE, FAKE, 1, d, 16, st,
                                      FAKE, maxp, FAKE, out_dt, dout, lse, 0.1, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_backward_validation_before_hip():
    plan = ma.mask_compile_host("causal", [0, 8], [8])
    need = ma.attn_backward_workspace(plan, 4)
    assert need == 2 * 8 * 4 * 4
    assert _backward(None) == L.MA_ERR_INVALID
    assert _backward(plan, dout=None) == L.MA_ERR_INVALID
    assert _backward(plan, lse=None) == L.MA_ERR_INVALID
    assert _backward(plan, total_q=9) == L.MA_ERR_PLAN_MISMATCH
    assert _backward(plan, d=96) == L.MA_ERR_UNSUPPORTED
    assert _backward(plan, out_dt=7) == L.MA_ERR_UNSUPPORTED
    assert _backward(plan, ws_bytes=need - 1) == L.MA_ERR_SIZE
    assert _backward(plan, ws=None) == L.MA_ERR_SIZE
    assert plan.info().on_device == 0       # nothing was uploaded


def test_status_strings():
    for s in range(-7, 1):
        assert L.LIB.ma_status_string(s).decode()


def test_single_hip_runtime_in_process():
    """Importing the package alone maps exactly one HIP runtime: the library's
    libamdhip64 dependency resolves to the one torch loads (two runtimes in
    one process do not share the device)."""
    import subprocess
    import sys
    code = ("import os, masked_flash_attention_mask_amd\n"
            "m = open(f'/proc/{os.getpid()}/maps').read()\n"
            "print(sorted({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root, timeout=300)
    assert r.returncode == 0, r.stderr
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs


def test_verify_noalloc_refuses_bounds_beyond_its_scratch():
    """The allocation-free tree verify holds 64 MiB of scratch per GPU:
    bounds that need more are MA_ERR_SIZE before any HIP call; bad arguments
    fail as for attn_verify_tree."""
    need = ma.attn_verify_tree_workspace(64, 64, 1 << 20, 32, 8, 128)
    assert need > 64 << 20
    st = (ctypes.c_int64 * 3)(2048, 128, 128)
    f = FAKE
    args = lambda kind, numel: (f, 64 * 64, 32, f, f, 8, 128, 16, st, f, 65536, f, f, 64, 64, 1 << 20, kind, f,
                                numel, L.BF16, L.F32, 0.1, f, None, None)
    assert L.LIB.attn_verify_tree_noalloc(*args(L.KIND["packed"], 1 << 30)) == L.MA_ERR_SIZE
    assert "scratch" in L.LIB.ma_last_error().decode()
    assert L.LIB.attn_verify_tree_noalloc(*args(L.KIND["causal"], 1 << 30)) == L.MA_ERR_CONFLICT
    assert L.LIB.attn_verify_tree_noalloc(*args(L.KIND["packed"], 100)) == L.MA_ERR_SIZE   # < one word per row
