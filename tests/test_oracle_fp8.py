"""Pins for oracle.fp8 (CPU only): torch's float8_e4m3fn decoder over all 256
codes, and the format's closed forms."""

import numpy as np
import torch

from oracle import fp8 as F


def test_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])


def test_closed_forms():
    d = F.e4m3_decode
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x40) == 2.0 and d(0x30) == 0.5
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0            # largest finite
    assert d(0x08) == 2.0 ** -6 and d(0x01) == 2.0 ** -9      # smallest normal, smallest subnormal
    assert d(0x00) == 0.0 and d(0x80) == 0.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    pos = d(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                         # codes 0..0x7E increase strictly
    # spacing: 8 values per binade, 2^(e-10) apart; subnormals 2^-9 apart
    assert np.allclose(np.diff(pos[:9]), 2.0 ** -9)
    assert np.allclose(np.diff(pos[0x38:0x41]), 2.0 ** -3)
