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


class _Rest:
    """The other entry points on fixed buffers: delayed scaling with a
    history window, the per-tensor cast with fused statistics, the
    stochastic-rounding cast, the separate statistics passes, MX with blocks
    down the columns (cast, dequant, statistics), and the update/step monitor
    with its window (with and without flag bytes)."""

    def __init__(self, n, cols):
        dev = "cuda"
        self.x = torch.empty(n, dtype=torch.bfloat16, device=dev)
        self.w = torch.empty(n, dtype=torch.float32, device=dev)
        self.d = torch.empty(n, dtype=torch.float32, device=dev)
        self.cols = cols
        self.codes, self.sr, self.colc = (torch.empty(n, dtype=torch.uint8, device=dev) for _ in range(3))
        self.sc = torch.empty(n // 32, dtype=torch.uint8, device=dev)
        self.y = torch.empty(n, dtype=torch.bfloat16, device=dev)
        self.flags = torch.empty(n, dtype=torch.uint8, device=dev)
        desc, cnt = nc.tensors([self.x], [self.codes])
        self.ws = nc.new_workspace(desc, cnt)
        self.sws = nc.new_swamp_workspace([self.w], [self.d])
        self.st, self.hist = nc.new_state(1), nc.new_history(1, 4)
        self.c = [nc.new_counts(1) for _ in range(4)]
        self.s = [nc.new_stats(1) for _ in range(4)]
        self.sw = [nc.new_swamp_counts(1) for _ in range(2)]
        self.swst = nc.new_swamp_state(1)
        self.pol = nc.policy("e4m3", "max_window", 4)
        self.spol = nc.swamp_policy(window=2, num=1, den=4)
        self.step = 0

    def run(self):
        for t in self.c + self.s + self.sw:
            t.zero_()                                    # fill kernels, not memset nodes
        x, c = [self.x], self.c
        nc.nc_cast_tensor(x, [self.codes], "e4m3", self.st, c[0], stats=self.s[0], ws=self.ws)
        nc.nc_scale_update(self.pol, self.st, c[0], self.hist)
        nc.nc_cast_tensor_sr(x, [self.sr], "e4m3", self.st, c[1], 77, 5, ws=self.ws)
        nc.nc_cast_stats(x, [self.codes], "e4m3", self.s[1], self.ws, st=self.st)
        nc.nc_cast_mx(x, [self.colc], [self.sc], [self.cols], "e5m2", "ceil", c[2], ws=self.ws, axis="cols")
        nc.nc_dequant([self.colc], [self.y], "e5m2", scales=[self.sc], cols=[self.cols], axis="cols")
        nc.nc_cast_stats(x, [self.colc], "e5m2", self.s[2], self.ws, scales=[self.sc], cols=[self.cols],
                         axis="cols")
        nc.nc_swamp_watch([self.w], [self.d], "bf16", self.sw[0], workspace=self.sws)
        nc.nc_swamp_watch([self.w], [self.d], "fp16", self.sw[1], flags=[self.flags], workspace=self.sws)
        nc.nc_swamp_window(self.spol, self.swst, self.sw[0])

    def outputs(self):
        ts = [self.codes, self.sr, self.colc, self.sc, self.y.view(torch.int16), self.flags, self.st, self.hist,
              self.swst] + self.c + self.s + self.sw
        return [t.clone() for t in ts]


def _fill_rest(r, seed, n):
    r.x.copy_(_data(seed, n))
    g = np.random.default_rng(seed)
    w = g.normal(0.0, 0.02, n).astype(np.float32)
    d = (1e-4 * g.standard_normal(n) * 10.0 ** g.uniform(-3, 1, n)).astype(np.float32)
    r.w.copy_(torch.from_numpy(w))
    r.d.copy_(torch.from_numpy(d))


def test_graph_capture_and_replay_other_entry_points():
    """Replays 0-3 of the captured sequence against the same calls run
    eagerly in between; the scale, history and window states evolve across
    replays on both sides alike."""
    cols = 1056
    n = 96 * cols                                        # 96 rows: three 32-row bands; ragged row tiles
    g_rest, e_rest = _Rest(n, cols), _Rest(n, cols)
    _fill_rest(g_rest, 20, n)
    _fill_rest(e_rest, 20, n)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g_rest.run()
    torch.cuda.current_stream().wait_stream(s)
    e_rest.run()                                         # the warm-up step, eagerly on the other side too
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_rest.run()
    for rep in range(4):
        _fill_rest(g_rest, 30 + rep, n)
        graph.replay()
        torch.cuda.synchronize()
        got = g_rest.outputs()
        _fill_rest(e_rest, 30 + rep, n)
        e_rest.run()
        torch.cuda.synchronize()
        for i, (u, v) in enumerate(zip(got, e_rest.outputs())):
            assert torch.equal(u, v), (rep, i)


def test_two_streams_at_once():
    """Two different steps enqueued on two streams with no ordering between
    them (each with its own workspace and outputs) give what each gives on
    its own: the library keeps no state between calls."""
    n, cols = 6 * 8192 + 1024, 1024
    a, b, a1, b1 = (_Step(n, cols) for _ in range(4))
    xa, xb = _data(40, n), _data(41, n)
    for s_, x in ((a, xa), (b, xb), (a1, xa), (b1, xb)):
        s_.x.copy_(x)
    a1.run()
    b1.run()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):                                   # several rounds, so the two overlap on the device
        with torch.cuda.stream(s1):
            a.run(stream=s1)
        with torch.cuda.stream(s2):
            b.run(stream=s2)
    torch.cuda.synchronize()
    for u, v in zip(a.outputs(), a1.outputs()):
        assert torch.equal(u, v)
    for u, v in zip(b.outputs(), b1.outputs()):
        assert torch.equal(u, v)
