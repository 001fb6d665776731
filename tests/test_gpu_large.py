"""One tensor past 2^31 elements: 32,769 rows of 65,536 bf16 values, each
row every bf16 pattern once (2,147,549,184 elements, 4.3 GB).  Every output
is then periodic by rows, so every output is checked -- each row against
the oracle's row -- and every count is 32,769 times one row's: amax, the
per-tensor cast, the MX cast (row blocks), both dequants, and the
stochastic-rounding cast sampled past element 2^31 (its draws are not
periodic).  Offsets past 2^31 reach every kernel's 64-bit indexing."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
from oracle import E4M3, bulk, rng
from tests._gpu import state_with_k

pytestmark = pytest.mark.gpu
ROWS, COLS = 32769, 65536


def _rows_equal(got: torch.Tensor, row: np.ndarray) -> bool:
    want = torch.from_numpy(np.ascontiguousarray(row)).cuda()
    return bool((got.view(ROWS, -1) == want).all())


def test_one_tensor_past_2p31():
    n = ROWS * COLS
    assert n > 1 << 31
    bits = np.arange(COLS, dtype=np.uint32).astype(np.uint16)
    v = bulk.bf16_bits_to_f64(bits)
    fin = np.isfinite(v)
    x = torch.from_numpy(bits.view(np.int16)).cuda().repeat(ROWS).view(torch.bfloat16)
    desc, cnt = nc.tensors([x], [None])
    ws = nc.new_workspace(desc, cnt)

    am = nc.new_counts(1)
    nc.nc_amax([x], am, ws=ws)
    torch.cuda.synchronize()
    a = nc.counts_list(am)[0]
    assert a["n_finite"] == ROWS * int(fin.sum()) and a["n_nonfinite"] == ROWS * int((~fin).sum())
    assert a["amax"] == float(np.max(np.abs(v[fin])))

    k = 0
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = nc.new_counts(1)
    nc.nc_cast_tensor([x], [codes], "e4m3", state_with_k([k]), out, ws=ws)
    torch.cuda.synchronize()
    wc, clip, uf, nf = bulk.cast_f64(E4M3, v, k)
    assert _rows_equal(codes, wc)
    c = nc.counts_list(out)[0]
    assert (c["n_clip"], c["n_underflow"], c["n_nonfinite"]) == \
        (ROWS * int(clip.sum()), ROWS * int(uf.sum()), ROWS * int(nf.sum()))

    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    nc.nc_dequant([codes], [y], "e4m3", st=state_with_k([k]))
    torch.cuda.synchronize()
    assert _rows_equal(y.view(torch.int16), bulk.dequant_bf16_f64(E4M3, wc, k).view(np.int16))

    # stochastic rounding: draws differ per element; 2^16 samples past 2^31
    seed, offset = 99, 5
    out = nc.new_counts(1)
    nc.nc_cast_tensor_sr([x], [codes], "e4m3", state_with_k([k]), out, seed, offset, ws=ws)
    torch.cuda.synchronize()
    idx = np.sort(np.random.default_rng(3).integers((1 << 31) - (1 << 20), n, 1 << 16))
    got = codes[torch.from_numpy(idx).cuda()].cpu().numpy()
    want = bulk.cast_sr_f64(E4M3, v[idx % COLS], k, rng.sr_uniforms_at(seed, offset, 0, idx))[0]
    assert np.array_equal(got, want)

    scales = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    out = nc.new_counts(1)
    nc.nc_cast_mx([x], [codes], [scales], [COLS], "e4m3", "ocp", out, ws=ws)
    torch.cuda.synchronize()
    mc, ms, mn = bulk.cast_mx_f64(E4M3, v, COLS, "ocp")
    assert _rows_equal(codes, mc) and _rows_equal(scales, ms)
    c = nc.counts_list(out)[0]
    for f in ("n_finite", "n_clip", "n_underflow", "n_nonfinite"):
        assert c[f] == ROWS * mn[f], f
    nc.nc_dequant([codes], [y], "e4m3", scales=[scales], cols=[COLS])
    torch.cuda.synchronize()
    K = np.repeat(127 - ms.astype(np.int64), 32)
    assert _rows_equal(y.view(torch.int16), bulk.dequant_bf16_f64(E4M3, mc, K).view(np.int16))


def test_column_blocks_past_2p31():
    """Column blocks on 32,800 rows of the same 65,536-pattern row
    (2,149,580,800 elements): each 32-row band of a column holds one value 32
    times, so every band of codes and every row of scale bytes is the same
    and checked in full against the oracle's band; dequant likewise."""
    rows = 32800
    n = rows * COLS
    assert n > 1 << 31 and rows % 32 == 0
    bits = np.arange(COLS, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).cuda().repeat(rows).view(torch.bfloat16)
    band = np.tile(bits, 32)
    vb = bulk.bf16_bits_to_f64(band)
    mc, ms, mn = bulk.cast_mx_f64(E4M3, vb, COLS, "ocp", axis="cols")
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    scales = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    desc, cnt = nc.tensors([x], [codes])
    ws = nc.new_workspace(desc, cnt)
    out = nc.new_counts(1)
    nc.nc_cast_mx([x], [codes], [scales], [COLS], "e4m3", "ocp", out, ws=ws, axis="cols")
    torch.cuda.synchronize()
    bands = rows // 32
    assert bool((codes.view(bands, -1) == torch.from_numpy(mc).cuda()).all())
    assert bool((scales.view(bands, -1) == torch.from_numpy(ms).cuda()).all())
    c = nc.counts_list(out)[0]
    for f in ("n_finite", "n_clip", "n_underflow", "n_nonfinite"):
        assert c[f] == bands * mn[f], f
    y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    nc.nc_dequant([codes], [y], "e4m3", scales=[scales], cols=[COLS], axis="cols")
    torch.cuda.synchronize()
    K = -bulk.mx_element_exponents(ms.astype(np.int64) - 127, mc.size, COLS, "cols")
    want = torch.from_numpy(bulk.dequant_bf16_f64(E4M3, mc, K).view(np.int16)).cuda()
    assert bool((y.view(torch.int16).view(bands, -1) == want).all())
