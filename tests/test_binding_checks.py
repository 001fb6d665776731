"""The Python binding refuses, before any pointer is taken or anything is
launched, buffers that do not match what the kernels will read or write:
short or long code buffers, wrong scale byte counts, mixed input dtypes,
undersized count, statistics, state, history and loss-scale buffers,
dequant outputs of the wrong size.  Host tensors are enough to reach every
check (the first step past them asks for device memory), so these run
without a GPU."""

import pytest
import torch

import scaled_fp8_casting_amd as nc


def f32(n):
    return torch.zeros(n, dtype=torch.float32)


def bf16(n):
    return torch.zeros(n, dtype=torch.bfloat16)


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


def counts(rows):
    return torch.zeros((rows, 5), dtype=torch.int64)


def stats(rows):
    return torch.zeros((rows, 6), dtype=torch.float64)


def state(rows):
    return torch.zeros((rows, 6), dtype=torch.int32)


def test_code_buffer_sizes():
    with pytest.raises(ValueError, match="codes\\[0\\]: 99 elements for 100"):
        nc.nc_cast_tensor([f32(100)], [u8(99)], "e4m3", state(1), counts(1))
    with pytest.raises(ValueError, match="codes\\[1\\]: 101 elements for 100"):
        nc.nc_cast_tensor([f32(64), f32(100)], [u8(64), u8(101)], "e4m3", state(2), counts(2))
    with pytest.raises(ValueError, match="codes\\[0\\]: dtype"):
        nc.nc_cast_tensor([f32(8)], [torch.zeros(8, dtype=torch.int8)], "e4m3", state(1), counts(1))


def test_mixed_input_dtypes():
    with pytest.raises(ValueError, match="one dtype per call"):
        nc.nc_cast_tensor([f32(64), bf16(64)], [u8(64), u8(64)], "e4m3", state(2), counts(2))
    with pytest.raises(ValueError, match="one dtype per call"):
        nc.nc_amax([bf16(64), f32(64)], counts(2))
    with pytest.raises(TypeError):
        nc.nc_amax([torch.zeros(8, dtype=torch.float16)], counts(1))


def test_mx_scale_sizes():
    with pytest.raises(ValueError, match="scales\\[0\\]: 3 bytes for 4 blocks"):
        nc.nc_cast_mx([bf16(128)], [u8(128)], [u8(3)], [128], "e4m3", "ocp", counts(1))
    with pytest.raises(ValueError, match="scales\\[0\\]: 5 bytes for 4 blocks"):
        nc.nc_dequant([u8(128)], [bf16(128)], "e4m3", scales=[u8(5)], cols=[128])
    with pytest.raises(ValueError, match="cols: 2 entries for 1 tensors"):
        nc.nc_cast_mx([bf16(128)], [u8(128)], [u8(4)], [128, 128], "e4m3", "ocp", counts(1))


def test_count_stat_state_buffers():
    with pytest.raises(ValueError, match="out: shape \\(1, 5\\)"):
        nc.nc_cast_tensor([f32(8), f32(8)], [u8(8), u8(8)], "e4m3", state(2), counts(1))
    with pytest.raises(ValueError, match="st: shape \\(1, 6\\)"):
        nc.nc_cast_tensor([f32(8), f32(8)], [u8(8), u8(8)], "e4m3", state(1), counts(2))
    with pytest.raises(ValueError, match="stats: shape \\(1, 6\\)"):
        nc.nc_cast_mx([bf16(64), bf16(64)], [u8(64), u8(64)], [u8(2), u8(2)], [64, 64], "e4m3", "ocp",
                      counts(2), stats=stats(1))
    with pytest.raises(ValueError, match="out: dtype torch.int32"):
        nc.nc_amax([f32(8)], torch.zeros((1, 5), dtype=torch.int32))
    with pytest.raises(ValueError, match="ls: 1 elements"):
        nc.nc_cast_tensor([f32(8)], [u8(8)], "e4m3", state(1), counts(1), ls=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="out: dtype torch.int64, expected torch.float64"):
        nc.nc_cast_stats([f32(8), f32(8)], [u8(8), u8(8)], "e4m3", counts(2), st=state(2))
    with pytest.raises(ValueError, match="out: shape \\(1, 6\\)"):
        nc.nc_cast_stats([f32(8), f32(8)], [u8(8), u8(8)], "e4m3", stats(1), st=state(2))
    with pytest.raises(ValueError, match="ws: dtype"):
        nc.nc_cast_tensor([f32(8)], [u8(8)], "e4m3", state(1), counts(1), ws=f32(64))


def test_scale_update_buffers():
    pol = nc.policy("e4m3", "max_window", 16)
    with pytest.raises(ValueError, match="hist: 16 elements, at least 32"):
        nc.nc_scale_update(pol, state(2), counts(2), torch.zeros((1, 16), dtype=torch.float32))
    with pytest.raises(ValueError, match="in_counts: shape \\(1, 5\\)"):
        nc.nc_scale_update(pol, state(2), counts(1), torch.zeros((2, 16), dtype=torch.float32))


def test_dequant_outputs():
    with pytest.raises(ValueError, match="ys\\[0\\]: 63 elements for 64 codes"):
        nc.nc_dequant([u8(64)], [bf16(63)], "e4m3", st=state(1))
    with pytest.raises(TypeError):
        nc.nc_dequant([u8(64)], [f32(64)], "e4m3", st=state(1))
    with pytest.raises(ValueError, match="ys: 2 entries for 1 tensors"):
        nc.nc_dequant([u8(64)], [bf16(64), bf16(64)], "e4m3", st=state(1))


def test_update_monitor_buffers():
    with pytest.raises(ValueError, match="flags\\[0\\]: 7 elements, at least 8"):
        nc.nc_swamp_watch([f32(8)], [f32(8)], "bf16", counts(1), flags=[u8(7)])
    with pytest.raises(ValueError, match="one update"):
        nc.nc_swamp_watch([f32(8)], [f32(8), f32(8)], "bf16", counts(1))
    with pytest.raises(ValueError, match="out: shape \\(1, 5\\)"):
        nc.nc_swamp_watch([f32(8), f32(8)], [f32(8), f32(8)], "bf16", counts(1))


def test_well_formed_calls_reach_the_device_check():
    """A call whose buffers all fit passes every size check and stops only at
    the first pointer, which must be device memory (there is no CPU path)."""
    with pytest.raises(ValueError, match="device tensor expected"):
        nc.nc_cast_tensor([f32(8)], [u8(8)], "e4m3", state(1), counts(1), ws=u8(4096))
    with pytest.raises(ValueError, match="device tensor expected"):
        nc.nc_cast_mx([bf16(64)], [u8(64)], [u8(2)], [64], "e4m3", "ocp", counts(1), ws=u8(4096))
