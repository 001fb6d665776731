"""GPU parity where a launch's tile count leaves a partial group of the
XCD-aware tile order (groups of 8C consecutive workgroups take 8C
consecutive tiles; a trailing partial group keeps the plain order), so
that both parts of the map and the seam between them carry data.

Sizes (bf16): 2053 * 4096 + 123 elements are 2054 tiles of the per-tensor
cast and of the dequant (one group of 2048 plus 6 for the cast's C = 256; 8
groups of 256 plus 6 for the dequant's C = 32) and 1027 tiles of amax (4
groups of 256 plus 3); the MX matrix of 2040 x 4128 is 2056 tiles of the
row-block cast (one group of 2048 plus 8)."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, bulk
import workloads
from tests._gpu import assert_counts, codes_like, dev_bf16, host_u8, host_u16, state_with_k

pytestmark = pytest.mark.gpu


def _bf16_input(n, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal(n) * np.exp2(r.integers(-12, 12, n // 4096 + 1)).repeat(4096)[:n]
    x[n // 2] = np.inf
    x[n - 1] = np.nan
    bits = workloads.to_bf16_bits(x)
    return dev_bf16(bits), bulk.bf16_bits_to_f64(bits)


def test_amax_cast_and_dequant_past_the_last_full_group():
    n = 2053 * 4096 + 123
    xd, x64 = _bf16_input(n, 11)
    am = nc.new_counts(1)
    nc.nc_amax([xd], am)
    codes = codes_like(n)
    out = nc.new_counts(1)
    nc.nc_cast_tensor([xd], [codes], "e4m3", state_with_k([-5]), out)
    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    nc.nc_dequant([codes], [y], "e4m3", st=state_with_k([-5]))
    torch.cuda.synchronize()
    wc, wn = bulk.cast_tensor_f64(E4M3, x64, -5)
    c = host_u8(codes)
    bad = np.flatnonzero(c != wc)
    assert bad.size == 0, (bad[:5], bad.size)
    assert_counts(nc.counts_list(out)[0], wn)
    assert nc.counts_list(am)[0]["amax"] == wn["amax"]
    assert np.array_equal(host_u16(y), bulk.dequant_bf16_f64(E4M3, wc, -5))


def test_mx_row_blocks_past_the_last_full_group():
    rows, cols = 2040, 4128
    xd, x64 = _bf16_input(rows * cols, 12)
    codes = codes_like(rows * cols)
    scales = torch.empty(rows * cols // 32, dtype=torch.uint8, device="cuda")
    out = nc.new_counts(1)
    nc.nc_cast_mx([xd], [codes], [scales], [cols], "e4m3", "ocp", out)
    torch.cuda.synchronize()
    wc, ws, wn = bulk.cast_mx_f64(E4M3, x64, cols, "ocp")
    assert np.array_equal(host_u8(scales), ws)
    bad = np.flatnonzero(host_u8(codes) != wc)
    assert bad.size == 0, (bad[:5], bad.size)
    assert_counts(nc.counts_list(out)[0], wn)
