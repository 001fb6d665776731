"""The input generators' bf16 rounding (numpy) against torch's own
fp32 -> bf16 conversion, over random and special values."""

import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(1)
    bits = r.integers(0, 1 << 32, 200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x7F800001,
                        0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000,
                        0x3F808000, 0x3F818000, 0x3F80FFFF, 0x00000001, 0x807FFFFF], np.uint32)
    bits = np.concatenate([special, bits])
    x32 = bits.view(np.float32)
    want = torch.from_numpy(x32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    with np.errstate(invalid="ignore"):          # signalling NaN patterns
        got = workloads.to_bf16_bits(x32.astype(np.float64))
    nan = np.isnan(x32)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == 0x7FC0) and np.all((want[nan] & 0x7FFF) > 0x7F80)
