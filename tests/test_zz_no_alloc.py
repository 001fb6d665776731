"""nc_cast_tensor_static (the per-tensor cast with the library's static
scratch in place of a workspace) against nc_cast_tensor (same inputs, a
workspace of its own): codes, counts and statistics bit for bit, on two
calls in a row -- a batch of three fp32 tensors with a loss-scale unscale,
then one smaller bf16 tensor -- and the oracle's codes on the second.  A
batch past the scratch's limit is refused before anything is enqueued."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, E5M2, bulk
from tests._gpu import dev_bf16, dev_f32, host_u8, state_with_k

pytestmark = pytest.mark.gpu


def _both(xs, fmt, ks, ls=None):
    """Run both entry points on the same inputs; return their outputs."""
    n = [x.numel() for x in xs]
    res = []
    for static in (True, False):
        codes = [torch.full((m,), 0xA5, dtype=torch.uint8, device="cuda") for m in n]
        out = nc.new_counts(len(xs))
        stats = nc.new_stats(len(xs))
        st = state_with_k(ks)
        if static:
            nc.nc_cast_tensor_static(xs, codes, fmt, st, out, ls=ls, stats=stats)
        else:
            nc.nc_cast_tensor(xs, codes, fmt, st, out, ls=ls, stats=stats)
        torch.cuda.synchronize()
        res.append(([host_u8(c) for c in codes], out.cpu(), stats.cpu()))
    return res


def test_static_scratch_matches_workspace_call_twice():
    rng = np.random.default_rng(77)
    # first call: three fp32 tensors (several tiles and ragged tails), unscale by 2^-3
    sizes = [100003, 8192 + 77, 5]
    host = [(rng.standard_normal(m) * 10.0 ** rng.uniform(-2, 3, m)).astype(np.float32) for m in sizes]
    host[0][17] = np.inf
    host[1][3] = np.nan
    xs = [dev_f32(h) for h in host]
    ls = nc.new_loss_scale(3)
    ks = [2, -1, 9]
    a, b = _both(xs, "e5m2", ks, ls=ls)
    for ca, cb in zip(a[0], b[0]):
        assert np.array_equal(ca, cb)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    for i, h in enumerate(host):                 # the static call's codes against the oracle (E5M2 at k - s)
        assert np.array_equal(a[0][i], bulk.cast_f64(E5M2, h.astype(np.float64), ks[i] - 3)[0]), i
    # second call, smaller: one bf16 tensor of 4097 elements
    bits = rng.integers(0, 1 << 16, 4097).astype(np.uint16)
    xb = dev_bf16(bits)
    a, b = _both([xb], "e4m3", [5])
    assert np.array_equal(a[0][0], b[0][0])
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert np.array_equal(a[0][0], bulk.cast_f64(E4M3, bulk.bf16_bits_to_f64(bits), 5)[0])


def test_static_scratch_refuses_a_batch_past_its_limit():
    # 2^28 + 2^20 fp32 elements need more than 8 MiB of slots at the
    # workspace's tile size: refused with NC_E_SCRATCH, nothing launched
    # (the buffers are real, so even a launch would stay in bounds)
    n = (1 << 28) + (1 << 20)
    x = torch.zeros(n, dtype=torch.float32, device="cuda")
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    desc, cnt = nc.tensors([x], [codes])
    assert nc.workspace_bytes(desc, cnt) > nc._lib.NC_STATIC_SCRATCH_BYTES
    out = nc.new_counts(1)
    with pytest.raises(nc.NarrowcastError) as e:
        nc.nc_cast_tensor_static([x], [codes], "e4m3", state_with_k([0]), out)
    assert e.value.status == nc._lib.NC_E_SCRATCH
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0
    del x, codes
    torch.cuda.empty_cache()
