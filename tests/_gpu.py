"""Helpers for the GPU parity tests: host arrays in, device tensors through
the C-ABI binding, host arrays back.  Inputs always originate on the host
(numpy, from ``workloads``); expected values come from ``oracle`` only."""

import numpy as np
import torch

import scaled_fp8_casting_amd as nc

DEV = "cuda"


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).to(DEV).view(torch.bfloat16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint8)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def state_with_k(ks) -> torch.Tensor:
    st = nc.new_state(len(ks))
    st[:, 0] = torch.tensor(list(ks), dtype=torch.int32)
    st[:, 2] = 1
    return st


def codes_like(n: int) -> torch.Tensor:
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def assert_counts(got: dict, want: dict, keys=("n_finite", "n_clip", "n_underflow", "n_nonfinite")):
    for k in keys:
        assert got[k] == want[k], (k, got[k], want[k])
    assert got["amax"] == want["amax"], ("amax", got["amax"], want["amax"])


def stats_close(got, want):
    """|gpu - exact| <= 1e-6 |exact| + 1e-12 A, with A a bound on the sum of
    the terms' magnitudes (the binary64 accumulation error is far below
    1e-12 A for the chain lengths used)."""
    g = dict(zip(nc.STAT_FIELDS, got))
    A = {
        "sum_e": want["sum_abs_e"], "sum_abs_e": want["sum_abs_e"], "sum_e2": want["sum_e2"],
        "sum_dir_e": want["sum_abs_e"], "sum_xe": (want["sum_x2"] * want["sum_e2"]) ** 0.5,
        "sum_x2": want["sum_x2"],
    }
    for k in nc.STAT_FIELDS:
        tol = 1e-6 * abs(want[k]) + 1e-12 * A[k]
        assert abs(g[k] - want[k]) <= tol, (k, g[k], want[k], tol)
