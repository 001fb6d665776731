"""Calls on a side stream, and captured in a HIP graph: the library launches
only on the stream it is given and allocates nothing, so a captured
sequence replays with fresh inputs.  Every replay is compared with the same
calls run eagerly."""

import numpy as np
import pytest
import torch

import scaled_fp8_casting_amd as nc
import workloads

pytestmark = pytest.mark.gpu


def _data(seed, n):
    r = np.random.default_rng(seed)
    x = (r.standard_t(3, n) * 10.0 ** r.uniform(-2, 2, n)).astype(np.float64)
    return torch.from_numpy(workloads.to_bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)


class _Step:
    """amax -> current-scaling update -> per-tensor and MX casts ->
    dequant, on fixed buffers."""

    def __init__(self, n, cols):
        self.x = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        self.cols = cols
        self.codes = torch.empty(n, dtype=torch.uint8, device="cuda")
        self.mx = torch.empty(n, dtype=torch.uint8, device="cuda")
        self.sc = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
        self.y = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        desc, cnt = nc.tensors([self.x], [self.codes])
        self.ws = nc.new_workspace(desc, cnt)
        self.am, self.c1, self.c2 = nc.new_counts(1), nc.new_counts(1), nc.new_counts(1)
        self.st = nc.new_state(1)
        self.pol = nc.policy("e4m3", "current", hysteresis=False)

    def run(self, stream=None):
        for c in (self.am, self.c1, self.c2):
            c.zero_()                                    # a fill kernel, not a memset node
        nc.nc_amax([self.x], self.am, ws=self.ws, stream=stream)
        nc.nc_scale_update(self.pol, self.st, self.am, stream=stream)
        nc.nc_cast_tensor([self.x], [self.codes], "e4m3", self.st, self.c1, ws=self.ws, stream=stream)
        nc.nc_cast_mx([self.x], [self.mx], [self.sc], [self.cols], "e4m3", "ocp", self.c2, ws=self.ws,
                      stream=stream)
        nc.nc_dequant([self.codes], [self.y], "e4m3", st=self.st, stream=stream)

    def outputs(self):
        return [t.clone() for t in (self.codes, self.mx, self.sc, self.y.view(torch.int16), self.am, self.c1,
                                    self.c2, self.st)]


def test_side_stream():
    n, cols = 3 * 8192 + 4096, 1024
    a, b = _Step(n, cols), _Step(n, cols)
    x = _data(1, n)
    a.x.copy_(x)
    b.x.copy_(x)
    a.run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b.run(stream=s)
    s.synchronize()
    for u, v in zip(a.outputs(), b.outputs()):
        assert torch.equal(u, v)


def test_graph_capture_and_replay():
    n, cols = 5 * 8192 + 2048, 2048
    g_step, e_step = _Step(n, cols), _Step(n, cols)
    g_step.x.copy_(_data(2, n))
    # warm up on a side stream, as capture requires
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g_step.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_step.run()
    for rep in range(4):
        x = _data(10 + rep, n)
        g_step.x.copy_(x)
        graph.replay()
        torch.cuda.synchronize()
        got = g_step.outputs()
        e_step.x.copy_(x)                                 # the same calls, eagerly, in between replays
        e_step.run()
        torch.cuda.synchronize()
        for i, (u, v) in enumerate(zip(got, e_step.outputs())):
            assert torch.equal(u, v), (rep, i)
