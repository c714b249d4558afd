"""GPU parity of the further mask inputs: block-sparse masks (block-row CSR)
and a sliding window intersected with custom (dense / packed, classified on
the device) and block-sparse masks, against the fp64 oracle; device
classification with a window against the host compiler; a block-sparse mask
against the equal dense mask, bit for bit."""

import numpy as np
import pytest
import torch

import masked_flash_attention_mask_amd as ma
import workloads as W
from helpers import TOL_BF16, compile_plan, device_inputs, lse_err, max_abs_err, oracle, oracle_masks, run_prefill

pytestmark = pytest.mark.gpu

MASKS = ("bsr64x64", "bsr128x128", "bsr16x48", "bsr64x64_window", "dense_window", "packed_window")


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("tile_q", [128, 64])
def test_mask_inputs_prefill(tile_q):
    w = W.mask_inputs()
    dev = device_inputs(w)
    for name in MASKS:
        _say("mask input", name, tile_q)
        out, lse, _ = run_prefill(w, dev, name, tile_q=tile_q)
        ref_o, ref_l = oracle(w, name)
        assert max_abs_err(out, ref_o) <= TOL_BF16, name
        assert lse_err(lse, ref_l) <= 1e-2, name


@pytest.mark.parametrize("tile_q", [128, 64])
def test_device_classify_with_window_matches_host(tile_q):
    w = W.mask_inputs()
    for name in ("dense_window", "packed_window"):
        _say("classify window", name, tile_q)
        dp = compile_plan(w, name, tile_q=tile_q, device_mask=True)
        hp = compile_plan(w, name, tile_q=tile_q, device_mask=False)
        c1, w1 = dp.export()
        c2, w2 = hp.export()
        assert np.array_equal(c1, c2) and np.array_equal(w1, w2), name


def test_block_sparse_equals_dense_bits():
    """A block-sparse description and the dense mask with the same bits give
    the same plan, hence bit-identical outputs."""
    w = W.mask_inputs()
    dev = device_inputs(w)
    om = oracle_masks(w, "bsr16x48")
    flat = np.concatenate([om(b).astype(np.uint8).reshape(-1) for b in range(w.batch)])
    w.masks["bsr16x48_dense"] = W.MaskInput("dense", data=flat)
    o1, l1, _ = run_prefill(w, dev, "bsr16x48")
    o2, l2, _ = run_prefill(w, dev, "bsr16x48_dense")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
