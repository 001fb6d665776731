"""Checkpoint and resume of the scaling state.  The only state of the path
is plain device memory -- the per-tensor scale states, the amax history ring
and the loss scale -- so a checkpoint is a copy to the host and a resume a
copy back into fresh buffers.  Twelve delayed-scaling steps straight must
equal six steps, a save, a restore into new buffers and six more, bit for
bit (codes, counts, states, history, loss scale), with non-finite steps that
skip and a loss scale that halves and grows."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
import workloads

pytestmark = pytest.mark.gpu
STEPS, HALF, W = 12, 6, 4


def _inputs():
    gen = workloads.GradientSteps(n_tensors=16, steps=STEPS, seed=103, log2_min=10, n_sizes=6)
    steps = []
    for t in range(STEPS):
        xs = [x * np.float32(2.0 ** 8) for x in gen.step(t)]       # loss-scaled by S = 2^8
        if t in (3, 8):
            xs[2][5] = np.inf if t == 3 else np.nan                  # a non-finite gradient: the step is skipped
        steps.append(xs)
    return gen.sizes, steps


class _Run:
    def __init__(self, sizes):
        T = len(sizes)
        self.codes = [torch.empty(m, dtype=torch.uint8, device="cuda") for m in sizes]
        self.xs = [torch.empty(m, dtype=torch.float32, device="cuda") for m in sizes]
        desc, cnt = nc.tensors(self.xs, self.codes)
        self.ws = nc.new_workspace(desc, cnt)
        self.st, self.hist, self.ls = nc.new_state(T), nc.new_history(T, W), nc.new_loss_scale(8)
        self.pol = nc.policy("e5m2", "max_window", W, hysteresis=True, interval=2, skip_on_nonfinite=True,
                             ls_enable=True, ls_growth_interval=3, ls_log2_min=0, ls_log2_max=16)

    def step(self, t, xs):
        for d, x in zip(self.xs, xs):
            d.copy_(torch.from_numpy(x))
        T = len(xs)
        if t == 0:                                     # no history yet: current scaling from this step's amax
            am = nc.new_counts(T)
            nc.nc_amax(self.xs, am, ls=self.ls, ws=self.ws)
            nc.nc_scale_update(nc.policy("e5m2", "current", W), self.st, am)
        out = nc.new_counts(T)
        nc.nc_cast_tensor(self.xs, self.codes, "e5m2", self.st, out, ls=self.ls, ws=self.ws)
        nc.nc_scale_update(self.pol, self.st, out, self.hist, self.ls)
        torch.cuda.synchronize()
        return [c.cpu().clone() for c in self.codes] + [t_.cpu().clone() for t_ in (out, self.st, self.hist, self.ls)]

    def save(self):
        return [t_.cpu().clone() for t_ in (self.st, self.hist, self.ls)]

    def restore(self, saved):
        for d, s in zip((self.st, self.hist, self.ls), saved):
            d.copy_(s.cuda())


def test_checkpoint_resume_bitwise():
    sizes, steps = _inputs()
    a = _Run(sizes)
    straight = [a.step(t, steps[t]) for t in range(STEPS)]
    b = _Run(sizes)
    for t in range(HALF):
        b.step(t, steps[t])
    saved = b.save()
    del b
    torch.cuda.empty_cache()
    c = _Run(sizes)                                   # fresh buffers, state restored from the host copy
    c.restore(saved)
    for t in range(HALF, STEPS):
        got = c.step(t, steps[t])
        for i, (u, v) in enumerate(zip(got, straight[t])):
            assert torch.equal(u, v), (t, i)
    # the run exercised what it claims: skipped steps and a moving loss scale
    ls_track = [int(s[-1][0]) for s in straight]
    assert len(set(ls_track)) > 1, ls_track
