"""Seeded synthetic inputs shaped like the workloads the pages describe.

This module generates inputs only.  It holds none of the cast's arithmetic
and is shared by the tests (which hand the same arrays to the HIP path and to
the oracle) and by the benchmark.  Every generator is deterministic in its
seed.  Rounding to the input dtype (fp64 -> fp32 -> bf16, nearest even) is
done by numpy.

Workloads (standard deviations are the second argument of N(0, s)):

* ``per_tensor_small``: 65,536 fp32 values ~ N(0, 1), seed 101.
* ``tanh_activations``: a rows x cols bf16 matrix of tanh(N(0, 1.5)) -- tanh
  outputs pile up just below 1.0, where the OCP block rule clips most
  ([Drift, "What the measurements said"]).  Seed 102.
* ``gradient_steps``: 64 fp32 gradient tensors of 2^12 .. 2^22 elements with
  per-tensor magnitudes 10^U[-10, 2], fresh N(0, 1) values each step and
  100x spikes on 5% of steps ([MaxWin, "Key Contributions"]: a spike beyond
  the delayed estimate saturates).  Seed 103.
* ``heavy_tailed_rows``: 2^30 bf16 values, 262,144 rows of 4096, row r =
  10^(v_r) * t_3 with v_r ~ U(-3, 3) ([E3, "Worked solution"]: one global
  scale cannot serve a layer a thousand times smaller).  Seed 105.
* ``LlamaGrads``: fp32 gradients shaped like a 7B decoder (per layer four
  4096x4096 and three 4096x11008 tensors, plus a 32000x4096 embedding), S *
  N(0, 1e-6) with S = 2^16 (loss-scaled, [MP-card, item (1)]), drawn on the
  device from a seeded generator each step; 1e-7 of all elements are then
  set to +Inf or NaN (even odds) at positions drawn on the host from seed
  104 and the step.
* ``UpdateStep``: fp32 master weights and one optimizer update for the
  update/step-ratio monitor ([E3, "Worked solution"]; [SP, "Master weights
  and the optimizer step"]: weights of order 1 meet updates far below their
  step late in training).  rows of 4096: w ~ N(0, 0.02) (an initialisation
  spread), d = lr * g * 10^(u_r) with lr = 1e-4, g ~ N(0, 1) and a per-row
  u_r ~ U(-3, 1), so the update/step ratio spans several binades either side
  of one.  Drawn on the device from a seeded generator (seed 106).
"""

import numpy as np
import torch


def to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (nearest even at each step, overflow to Inf, NaN
    -> 0x7FC0), as uint16 bits.  numpy only: no torch CPU kernel runs here, so
    no thread pool is started in a process that later forks workers (nor in
    the workers)."""
    b = np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32).view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    r[(b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)] = 0x7FC0
    return r


def per_tensor_small(n: int = 65536, seed: int = 101) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(n).astype(np.float32)


def tanh_activations(rows: int = 4096, cols: int = 4096, seed: int = 102) -> np.ndarray:
    z = np.random.default_rng(seed).normal(0.0, 1.5, rows * cols)
    return to_bf16_bits(np.tanh(z)).reshape(rows, cols)


class GradientSteps:
    """64 fp32 tensors per step; tensor i has 2^(12 + (i mod 11)) elements
    and log10-magnitude u_i ~ U[-10, 2], drawn once.  Step t draws fresh
    N(0, 1) values from seed + 1000 t.  Exactly round(5% of steps) spike steps
    are drawn from steps 1 .. steps-1; on each, one uniformly drawn tensor is
    multiplied by 100."""

    def __init__(self, n_tensors: int = 64, steps: int = 32, seed: int = 103,
                 log2_min: int = 12, n_sizes: int = 11):
        rng = np.random.default_rng(seed)
        self.seed = seed
        self.sizes = [1 << (log2_min + (i % n_sizes)) for i in range(n_tensors)]
        self.log10_mag = rng.uniform(-10.0, 2.0, n_tensors)
        n_spikes = int(round(0.05 * steps))
        self.spike_steps = sorted(rng.choice(np.arange(1, steps), n_spikes, replace=False).tolist())
        self.spike_tensor = {t: int(rng.integers(0, n_tensors)) for t in self.spike_steps}
        self.steps = steps

    def step(self, t: int):
        rng = np.random.default_rng(self.seed + 1000 * t)
        out = []
        for i, n in enumerate(self.sizes):
            mag = 10.0 ** self.log10_mag[i]
            if self.spike_tensor.get(t) == i:
                mag *= 100.0
            out.append((mag * rng.standard_normal(n)).astype(np.float32))
        return out


def heavy_tailed_rows(row0: int, nrows: int, cols: int = 4096, seed: int = 105,
                      chunk_rows: int = 1024) -> np.ndarray:
    """Rows [row0, row0 + nrows) of the heavy-tailed bf16 matrix, as uint16
    bits of shape (nrows, cols).  Rows are generated in chunks of
    ``chunk_rows`` with one child seed per chunk, so any chunk can be
    regenerated on its own (row0 and nrows must be multiples of it)."""
    assert row0 % chunk_rows == 0 and nrows % chunk_rows == 0
    out = np.empty((nrows, cols), dtype=np.uint16)
    for c in range(nrows // chunk_rows):
        chunk = row0 // chunk_rows + c
        rng = np.random.default_rng([seed, chunk])
        v = rng.uniform(-3.0, 3.0, chunk_rows)
        t = rng.standard_t(3, (chunk_rows, cols))
        out[c * chunk_rows:(c + 1) * chunk_rows] = to_bf16_bits(t * (10.0 ** v)[:, None])
    return out


def random_fp32_bits(n: int, seed: int) -> np.ndarray:
    """Uniform 32-bit patterns (all classes: subnormals, Inf, NaN)."""
    return np.random.default_rng(seed).integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)


def mixed_magnitude_fp32(n: int, seed: int, log2_lo: int = -140, log2_hi: int = 127) -> np.ndarray:
    """Signed fp32 values with log-uniform magnitudes over [2^lo, 2^hi)."""
    rng = np.random.default_rng(seed)
    e = rng.uniform(log2_lo, log2_hi, n)
    s = rng.choice([-1.0, 1.0], n)
    with np.errstate(over="ignore"):
        return (s * np.exp2(e)).astype(np.float32)


def _ht_chunk(args):
    row0, nrows, cols, seed = args
    return row0, heavy_tailed_rows(row0, nrows, cols, seed)


def heavy_tailed_parallel(nrows: int = 262144, cols: int = 4096, seed: int = 105,
                          procs: int = 8, chunk_rows: int = 1024, context: str = "fork") -> np.ndarray:
    """``heavy_tailed_rows(0, nrows)`` generated by a process pool (same
    values: each chunk has its own child seed).  context: the
    multiprocessing start method ("spawn" from a process that already uses
    the GPU)."""
    import multiprocessing as mp
    assert nrows % chunk_rows == 0, "nrows must be a multiple of chunk_rows"
    out = np.empty((nrows, cols), dtype=np.uint16)
    jobs = [(r, chunk_rows, cols, seed) for r in range(0, nrows, chunk_rows)]
    if procs <= 1:
        for j in jobs:
            r, a = _ht_chunk(j)
            out[r:r + chunk_rows] = a
        return out
    with mp.get_context(context).Pool(procs) as pool:
        for r, a in pool.imap_unordered(_ht_chunk, jobs):
            out[r:r + chunk_rows] = a
    return out


class LlamaGrads:
    """Device-resident loss-scaled gradients of a Llama-7B-shaped model (see
    the module docstring).  ``layers`` scales the model down for tests; the
    embedding is always included.  ``fill(t)`` overwrites the buffers with
    step t's values and returns the injected positions as (tensor, offset,
    is_nan) arrays."""

    S_LOG2 = 16
    SIGMA = 1e-6

    def __init__(self, layers: int = 32, seed: int = 104, device: str = "cuda"):
        shapes = []
        for _ in range(layers):
            shapes += [(4096, 4096)] * 4 + [(4096, 11008)] * 3
        shapes.append((32000, 4096))
        self.shapes = shapes
        self.sizes = [r * c for r, c in shapes]
        self.starts = np.concatenate([[0], np.cumsum(self.sizes)])
        self.total = int(self.starts[-1])
        self.seed = seed
        self.device = device
        self.bufs = [torch.empty(n, dtype=torch.float32, device=device) for n in self.sizes]
        self.n_inject = int(round(1e-7 * self.total))

    def fill(self, t: int):
        g = torch.Generator(device=self.device)
        g.manual_seed(self.seed * 1000003 + t)
        std = float(2 ** self.S_LOG2) * self.SIGMA
        for b in self.bufs:
            b.normal_(0.0, std, generator=g)
        rng = np.random.default_rng([self.seed, t])
        pos = np.unique(rng.integers(0, self.total, self.n_inject))
        while pos.size < self.n_inject:
            pos = np.unique(np.concatenate([pos, rng.integers(0, self.total, self.n_inject - pos.size)]))
        is_nan = rng.integers(0, 2, pos.size).astype(bool)
        tensor = np.searchsorted(self.starts, pos, side="right") - 1
        offset = pos - self.starts[tensor]
        for i in np.unique(tensor):
            m = tensor == i
            idx = torch.from_numpy(offset[m]).to(self.device)
            val = torch.from_numpy(np.where(is_nan[m], np.nan, np.inf).astype(np.float32)).to(self.device)
            self.bufs[i].index_copy_(0, idx, val)
        return tensor, offset, is_nan


class UpdateStep:
    """Device-resident fp32 weights ``w`` and updates ``d`` (see the module
    docstring), rows x 4096."""

    COLS = 4096
    SIGMA_W = 0.02
    LR = 1e-4

    def __init__(self, rows: int, seed: int = 106, device: str = "cuda"):
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        n = rows * self.COLS
        self.w = torch.empty(n, dtype=torch.float32, device=device).normal_(0.0, self.SIGMA_W, generator=g)
        self.d = torch.empty(n, dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
        u = torch.empty(rows, 1, dtype=torch.float32, device=device).uniform_(-3.0, 1.0, generator=g)
        self.d.view(rows, self.COLS).mul_(torch.pow(10.0, u) * self.LR)
        self.n = n

