"""GPU parity over batches of 64 tensors, the most one launch takes, with
empty tensors at both ends of the groups of eight that the per-workgroup
tensor lookup scans and a run of empty tensors across two groups: each
kernel that launches over a batch, every tensor's results against the
oracle."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, E5M2, bulk
import workloads
from tests._gpu import assert_counts, codes_like, dev_bf16, dev_f32, host_u8, host_u16, state_with_k

pytestmark = pytest.mark.gpu
T = 64
EMPTY = {0, 7, 8, 15, 16, 17, 18, 19, 20, 21, 22, 23, 24, 25, 31, 55, 56, 63}


def _sizes(seed, unit, hi):
    r = np.random.default_rng(seed)
    return [0 if j in EMPTY else unit * int(r.integers(1, hi)) for j in range(T)]


def _inputs(sizes, seed, dtype):
    r = np.random.default_rng(seed)
    xd, x64 = [], []
    for m in sizes:
        x = (r.standard_normal(m) * 10.0 ** r.uniform(-3, 3)).astype(np.float32)
        if m > 100:
            x[m // 3] = np.inf
        if dtype == "bf16":
            bits = workloads.to_bf16_bits(x.astype(np.float64))
            xd.append(dev_bf16(bits))
            x64.append(bulk.bf16_bits_to_f64(bits))
        else:
            xd.append(dev_f32(x))
            x64.append(x.astype(np.float64))
    return xd, x64


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_amax_and_per_tensor_cast(dtype):
    sizes = _sizes(1, 1, 9000)
    xd, x64 = _inputs(sizes, 2, dtype)
    ks = [int(v) for v in np.random.default_rng(3).integers(-5, 15, T)]
    am = nc.new_counts(T)
    nc.nc_amax(xd, am)
    codes = [codes_like(m) for m in sizes]
    out = nc.new_counts(T)
    nc.nc_cast_tensor(xd, codes, "e4m3", state_with_k(ks), out)
    torch.cuda.synchronize()
    ga, gc = nc.counts_list(am), nc.counts_list(out)
    for j, x in enumerate(x64):
        wc, wn = bulk.cast_tensor_f64(E4M3, x, ks[j])
        assert np.array_equal(host_u8(codes[j]), wc), j
        assert_counts(gc[j], wn)
        assert ga[j]["amax"] == wn["amax"] and ga[j]["n_nonfinite"] == wn["n_nonfinite"], j
        assert ga[j]["n_finite"] == wn["n_finite"], j


def test_per_tensor_dequant():
    sizes = _sizes(4, 1, 12000)
    r = np.random.default_rng(5)
    codes = [r.integers(0, 256, m).astype(np.uint8) for m in sizes]
    ks = [int(v) for v in r.integers(-20, 20, T)]
    ys = [torch.full((m,), -3.0, dtype=torch.bfloat16, device="cuda") for m in sizes]
    nc.nc_dequant([torch.from_numpy(c).cuda() for c in codes], ys, "e5m2", st=state_with_k(ks))
    torch.cuda.synchronize()
    for j, c in enumerate(codes):
        assert np.array_equal(host_u16(ys[j]), bulk.dequant_bf16_f64(E5M2, c, ks[j])), j


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mx_row_blocks(dtype):
    cols = 96
    sizes = _sizes(6, cols, 80)
    xd, x64 = _inputs(sizes, 7, dtype)
    codes = [codes_like(m) for m in sizes]
    scales = [torch.empty(m // 32, dtype=torch.uint8, device="cuda") for m in sizes]
    out = nc.new_counts(T)
    nc.nc_cast_mx(xd, codes, scales, [cols] * T, "e4m3", "ocp", out)
    torch.cuda.synchronize()
    got = nc.counts_list(out)
    for j, x in enumerate(x64):
        wc, ws, wn = bulk.cast_mx_f64(E4M3, x, cols, "ocp")
        assert np.array_equal(host_u8(codes[j]), wc) and np.array_equal(host_u8(scales[j]), ws), j
        assert_counts(got[j], wn)


def test_mx_column_block_dequant():
    r = np.random.default_rng(8)
    shapes = [(0, 32) if j in EMPTY else (32 * int(r.integers(1, 4)), int(r.choice([32, 64, 96, 160])))
              for j in range(T)]
    codes = [r.integers(0, 256, rows * cols).astype(np.uint8) for rows, cols in shapes]
    scales = [r.integers(0, 255, rows * cols // 32).astype(np.uint8) for rows, cols in shapes]
    ys = [torch.full((rows * cols,), -3.0, dtype=torch.bfloat16, device="cuda") for rows, cols in shapes]
    nc.nc_dequant([torch.from_numpy(c).cuda() for c in codes], ys, "e4m3",
                  scales=[torch.from_numpy(s).cuda() for s in scales], cols=[c for _, c in shapes], axis="cols")
    torch.cuda.synchronize()
    for j, ((rows, cols), c, s) in enumerate(zip(shapes, codes, scales)):
        K = -bulk.mx_element_exponents(s.astype(np.int64) - 127, rows * cols, cols, "cols")
        assert np.array_equal(host_u16(ys[j]), bulk.dequant_bf16_f64(E4M3, c, K)), j
