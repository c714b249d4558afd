"""GPU parity of masked decode over e4m3 (fp8) K/V caches against the fp64
oracle run on the exactly decoded caches (K = k_descale * decode(K8),
likewise V; bf16 queries): every mask kind, d 64 / 128 / 256, GQA and MHA,
ragged contexts that split, and the decode benchmark batch."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import TOL_BF16, device_inputs, lse_err, max_abs_err, oracle, repage
from oracle import fp8 as OF
from test_gpu_decode import KV_LENS, Q_LENS, _workload

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _kv8(w):
    """Device e4m3 caches and descale factors of a workload, and the
    workload with its caches replaced by their exact decoded values."""
    import copy
    f8 = W.fp8_inputs(w)
    wd = copy.copy(w)
    wd.k_cache = OF.e4m3_decode(f8["k8"]) * f8["k_s"]
    wd.v_cache = OF.e4m3_decode(f8["v8"]) * f8["v_s"]
    dev8 = {"k8": torch.from_numpy(np.ascontiguousarray(f8["k8"])).cuda(),
            "v8": torch.from_numpy(np.ascontiguousarray(f8["v8"])).cuda()}
    return f8, wd, dev8


def _decode8(w, dev, dev8, f8, name, max_q, max_kv, out_dtype=torch.float32):
    mi = w.masks[name]
    kw = {}
    if mi.kind == "window":
        kw["window"] = mi.window
    elif mi.kind == "prefix_lm":
        kw["prefix_len"] = torch.from_numpy(mi.prefix_len).cuda()
    elif mi.kind in ("dense", "packed"):
        data = mi.data if mi.kind == "dense" else mi.data.view(np.int64)
        kw["mask"] = torch.from_numpy(np.ascontiguousarray(data)).cuda()
    out, lse = ma.attn_decode_kv8(dev["q"], dev8["k8"], dev8["v8"], dev["pt"], dev["cu"], dev["kv"], max_q, max_kv,
                                  w.scale, f8["k_s"], f8["v_s"], mask_kind=mi.kind, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("d,hq,hkv", [(64, 8, 2), (128, 8, 2), (128, 4, 4), (256, 4, 1)])
def test_decode_kv8_mask_kinds(d, hq, hkv):
    w = _workload(900 + d + hq, d, hq, hkv)
    dev = device_inputs(w)
    f8, wd, dev8 = _kv8(w)
    for name in ("causal", "window", "wide_window", "prefix", "dense", "packed"):
        _say("decode kv8", d, hq, hkv, name)
        out, lse = _decode8(w, dev, dev8, f8, name, max(Q_LENS), max(KV_LENS))
        ref_o, ref_l = oracle(wd, name)
        err = max_abs_err(out, ref_o)
        assert err <= TOL_BF16, (name, err)
        assert lse_err(lse, ref_l) <= 1e-2, name


@pytest.mark.parametrize("d", [64, 128])
def test_decode_kv8_page_sizes(d):
    """e4m3 caches in pages of the smallest allowed size (1024 / d keys) up
    to 256 keys: every positional mask matches the oracle on the decoded
    caches, and the output does not depend on the page size."""
    w = _workload(804, d, 8, 2)
    names = ("causal", "window", "prefix")
    first = {}
    for ps in (1024 // d, 64, 256):
        wp = repage(w, ps, 910 + ps)
        dev = device_inputs(wp)
        f8, wd, dev8 = _kv8(wp)
        for n in names:
            _say("decode kv8 pages", d, ps, n)
            o, lse = _decode8(wp, dev, dev8, f8, n, max(Q_LENS), max(KV_LENS))
            ref_o, ref_l = oracle(wd, n)
            assert max_abs_err(o, ref_o) <= TOL_BF16, (ps, n)
            assert lse_err(lse, ref_l) <= 1e-2, (ps, n)
            if n in first:
                assert torch.equal(o, first[n][0]) and torch.equal(lse, first[n][1]), (ps, n)
            else:
                first[n] = (o, lse)


def test_decode_kv8_bf16_output_and_determinism():
    w = _workload(951, 128, 8, 2)
    dev = device_inputs(w)
    f8, wd, dev8 = _kv8(w)
    o1, l1 = _decode8(w, dev, dev8, f8, "dense", max(Q_LENS), max(KV_LENS), out_dtype=torch.bfloat16)
    o2, l2 = _decode8(w, dev, dev8, f8, "dense", max(Q_LENS), max(KV_LENS), out_dtype=torch.bfloat16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    of, lf = _decode8(w, dev, dev8, f8, "dense", max(Q_LENS), max(KV_LENS))
    assert torch.equal(l1, lf)
    assert (o1.float() - of).abs().max().item() <= 2.0 ** -8 * of.abs().max().item() + 1e-6


def test_decode_kv8_benchmark_batch():
    """16 sequences of 4k-16k keys, 32 / 8 heads, d 128, 1 query each, causal
    and a 4096-key window, all heads against the oracle."""
    w = W.decode(q_len=1)
    dev = device_inputs(w)
    f8, wd, dev8 = _kv8(w)
    for name in ("causal", "window"):
        _say("decode kv8 benchmark batch", name)
        out, lse = _decode8(w, dev, dev8, f8, name, 1, int(w.kv_lens.max()))
        ref_o, ref_l = oracle(wd, name)
        assert max_abs_err(out, ref_o) <= TOL_BF16, name
        assert lse_err(lse, ref_l) <= 1e-2, name
