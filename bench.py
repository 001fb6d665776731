"""Throughput of the scaled FP8 cast on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows R] [--no-cpu]
                    [--no-llama] [--no-configs] [--cpu-rows R] [--copy-probe]

Workload: a heavy-tailed bf16 tensor of 2^30 elements (262,144 rows of 4096;
row r = 10^v_r * Student-t(3), v_r ~ U(-3, 3)), resident in HBM before the
timed region.  One step is one pass of the whole cast path over it:

  1. nc_amax          per-tensor amax pass                     (read 2 B/elem)
  2. nc_scale_update  current scaling -> k                      (O(1))
  3. nc_cast_tensor   per-tensor E4M3 cast + counts + amax      (2 + 1)
  4. nc_cast_mx       MXFP8 E4M3, OCP rule, + counts            (2 + 1 + 1/32)
  5. nc_dequant       per-tensor codes -> bf16                  (1 + 2)
  6. nc_dequant       MX codes -> bf16                          (1 + 1/32 + 2)
  7. nc_cast_stats    error/bias statistics, per-tensor         (2 + 1)
  8. nc_cast_stats    error/bias statistics, MX                 (2 + 1 + 1/32)

Beside the step (not part of it) the same JSON line reports the casts with
fused statistics, the stochastic-rounding cast, the MX cast, dequant and
statistics with blocks down the columns, the update/step-ratio monitor on
2^30 fp32 weights and updates (counts only, and with a flag byte per
element), torch's device copy of the cast's byte count, and one
delayed-scaling step of loss-scaled Llama-7B-shaped fp32 gradients (225
tensors, 6.6G elements, fused 2^-16 unscale).  `step_fused_stats` times the
same step with the statistics fused into the two casts (steps 1-6 with
statistics, no passes 7-8): the same outputs in fewer bytes.  Under "configs" it times the
three smaller workloads on their own (last-level cache flushed before each
rep): 65,536 fp32 elements under current scaling (microseconds, launch-bound),
the 4096 x 4096 tanh bf16 matrix to MXFP8 under the OCP, +1 and ceil rules, and one
delayed E5M2 scaling step over 64 fp32 gradient tensors.

Prints one JSON line.  `value` is elements per second through the whole step
(Gelem/s); `roofline` is the dominant kernel's algorithmic bytes per launch
over its mean launch time (HIP events on the launch stream, inside the timed
region) against 8 TB/s; `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
COLS = 4096


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The first steps after start-up run at a lower shader clock (the power
    # manager ramps it; some kernels ran 10-40% slower in the first one or
    # two steps), so the default warm-up covers them; step_series in the
    # output shows every step either way.
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--rows", type=int, default=262144, help="rows of 4096 (default 2^30 elements)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-llama", action="store_true",
                    help="skip the Llama-shaped unscale+cast measured beside the step")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the three smaller workloads timed after the step")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the workload the CPU oracle baseline runs on")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed region, copy 1 GiB device-to-device three times with a plain "
                         "torch copy kernel (the reference point for HBM byte counters)")
    ap.add_argument("--procs", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--input-cache", metavar="PATH",
                    help="raw uint16 file of the workload: read if present (and of the right size), "
                         "else generated and written there")
    ap.add_argument("--make-input", action="store_true",
                    help="only write --input-cache and exit (no GPU use); a profiled run that reads "
                         "the cache then starts no worker processes")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 --pmc counter files and exit")
    return ap.parse_args()


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_fp8_casting_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# rocprofv3 kernel names of each call's main kernel (format E4M3 = 0, bf16 = 1)
KERNEL_SIG = {"amax": "k_amax<1>", "cast_tensor": "k_cast_pt<0, 1, false>",
              "cast_mx": "k_cast_mx<0, 1, 0, false>", "dequant_pt": "k_dequant<0, false>",
              "dequant_mx": "k_dequant<0, true>", "stats_pt": "k_stats<0, 1, false>",
              "stats_mx": "k_stats<0, 1, true>",
              "cast_tensor+stats": "k_cast_pt<0, 1, true>", "cast_mx+stats": "k_cast_mx<0, 1, 0, true>",
              "cast_mx_cols": "k_cast_mx_col<0, 1, 0, false>", "dequant_mx_cols": "k_dequant_col<0>",
              "stats_mx_cols": "k_stats_col<0, 1>", "cast_tensor_sr": "k_cast_sr<0, 1>",
              "swamp_watch": "k_swamp<0, false>", "swamp_watch_flags": "k_swamp<0, true>"}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def traffic_for(call: str, src_hash: str):
    """HBM bytes per launch of a call's kernel from the committed rocprofv3
    counter runs, if they were taken on the current kernel sources; else None."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        t = json.load(f)
    if t.get("source_hash") != src_hash:
        return None
    k = t.get("kernels", {}).get(KERNEL_SIG.get(call, ""))
    return None if k is None else k.get("hbm_bytes_per_launch")


def write_traffic(fetch_csv: str, write_csv: str):
    """profiles/traffic.json from two rocprofv3 --pmc runs of this script with
    --copy-probe (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter
    is scaled by bytes / reading for the plain 1 GiB device copies of the
    probe (the rocclr copy kernel; that run does no other large copy), then
    averaged per kernel."""
    import csv
    from collections import defaultdict
    probe_kib = float(1 << 20)
    out = {"source_hash": source_hash(), "kernels": {}, "scale": {}}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = defaultdict(list)
        copy = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                name = r["Kernel_Name"]
                if name == "__amd_rocclr_copyBuffer":
                    copy.append(v)
                for sig in KERNEL_SIG.values():
                    if sig in name:
                        vals[sig].append(v)
        # the probe's copies (the run's other copies are small uploads)
        copy = [c for c in copy if c > 0.1 * probe_kib]
        if not copy:
            raise SystemExit(f"{path}: no 1 GiB copy dispatches (run with --copy-probe)")
        factor = probe_kib / (sum(copy) / len(copy))
        out["scale"][counter] = {"copy_kib": round(sum(copy) / len(copy), 1), "bytes_per_count_kib": factor}
        per[counter] = {sig: 1024.0 * factor * sum(v) / len(v) for sig, v in vals.items()}
    for sig in KERNEL_SIG.values():
        if sig in per["FETCH_SIZE"] and sig in per["WRITE_SIZE"]:
            rd, wr = round(per["FETCH_SIZE"][sig]), round(per["WRITE_SIZE"][sig])
            out["kernels"][sig] = {"read_bytes": rd, "write_bytes": wr, "hbm_bytes_per_launch": rd + wr}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(rows: int, procs: int):
    """The oracle (tier 1, vectorised exact binary64) over the same step on
    `rows` rows of the workload, row chunks spread over a process pool; and
    tier 0 (exact rationals, one core) on the 65,536-element current-scaling
    workload.  The workers are started with "spawn": this process has used
    the GPU, and a forked child would inherit its HIP state."""
    import multiprocessing as mp
    import workloads
    bits = workloads.heavy_tailed_parallel(rows, COLS, procs=procs, context="spawn")
    chunk = -(-rows // procs)
    jobs = [bits[r:r + chunk] for r in range(0, rows, chunk)]
    workers = min(procs, len(jobs))
    print(f"[bench] CPU oracle: input ready, {workers} workers", file=sys.stderr, flush=True)
    # the per-tensor scale needs the global amax first (as on the GPU); each
    # phase has a time limit, so a stuck worker cannot hold the bench
    with mp.get_context("spawn").Pool(workers) as pool:
        pool.map_async(_cpu_ready, range(workers)).get(timeout=120)   # start-up (imports) untimed
        t0 = time.perf_counter()
        amaxes = pool.map_async(_cpu_amax, jobs).get(timeout=120)
        k = _scale_k(max(amaxes))
        print(f"[bench] CPU oracle: amax pass done ({time.perf_counter() - t0:.1f} s)", file=sys.stderr,
              flush=True)
        pool.map_async(_cpu_step, [(j, k) for j in jobs]).get(timeout=150)
        dt = time.perf_counter() - t0
    n = rows * COLS
    t0_s, t0_n = _cpu_tier0_small()
    return dict(value=n / dt / 1e9, unit="Gelem/s", cores=workers, host_cpus=os.cpu_count(), kind="oracle",
                sample=f"{rows} rows x {COLS} of the same workload ({n} elements), whole step, "
                       f"{workers} worker processes on a host reporting {os.cpu_count()} CPUs, {dt:.1f} s, "
                       f"{_cpu_model()}",
                tier0_single_core=dict(workload=f"{t0_n} fp32 ~ N(0,1), current per-tensor E4M3 scaling "
                                                f"(amax, scale, cast) in exact rationals, one core",
                                       seconds=round(t0_s, 2), gelem_s=t0_n / t0_s / 1e9))


def _cpu_ready(_):
    from oracle import bulk  # noqa: F401  (the workers' imports, before the clock starts)
    return os.getpid()


def _cpu_tier0_small():
    """Tier 0 (Fractions) on the 65,536-element current-scaling workload, one core."""
    import workloads
    from oracle import E4M3
    from oracle import cast as t0
    from oracle.formats import Val
    x = workloads.per_tensor_small()
    t = time.perf_counter()
    vals = [Val.of(float(v)) for v in x]
    k = t0.scale_exponent(E4M3, t0.amax(vals))
    t0.cast_tensor(E4M3, vals, k)
    return time.perf_counter() - t, x.size


def mp_timeout():
    import multiprocessing as mp
    return mp.TimeoutError


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "cpu model unknown"


def _cpu_amax(b):
    from oracle import bulk
    return bulk.amax_f64(bulk.bf16_bits_to_f64(b.ravel()))


def _scale_k(a):
    from fractions import Fraction
    from oracle import E4M3
    from oracle.cast import scale_exponent
    return scale_exponent(E4M3, Fraction(a))


def _cpu_step(args):
    b, k = args
    from oracle import E4M3
    from oracle import bulk
    x = bulk.bf16_bits_to_f64(b.ravel())
    c_pt, clip, uf, nf = bulk.cast_f64(E4M3, x, k)
    c_mx, sc, _ = bulk.cast_mx_f64(E4M3, x, COLS, "ocp")
    K_mx = np.repeat(127 - sc.astype(np.int64), 32)
    bulk.dequant_bf16_f64(E4M3, c_pt, k)
    bulk.dequant_bf16_f64(E4M3, c_mx, K_mx)
    bulk.stats_f64(E4M3, x, c_pt, k)
    bulk.stats_f64(E4M3, x, c_mx, K_mx)
    return int(np.count_nonzero(clip))


def llama_unscale_cast(nc, torch, workloads):
    """Loss-scaled fp32 gradients of a Llama-7B-shaped model (225 tensors,
    6,607,077,376 elements, S = 2^16, 1e-7 of them Inf/NaN): one delayed-
    scaling step, i.e. a single nc_cast_tensor call over all tensors with the
    2^-16 unscale fused (scales from a current-scaling pass, untimed)."""
    g = workloads.LlamaGrads(layers=32)
    g.fill(0)
    T = len(g.bufs)
    codes = [torch.empty(m, dtype=torch.uint8, device="cuda") for m in g.sizes]
    desc, cnt = nc.tensors(g.bufs, codes)
    ws = nc.new_workspace(desc, cnt)
    ls = nc.new_loss_scale(g.S_LOG2)
    st = nc.new_state(T)
    am = nc.new_counts(T)
    nc.nc_amax(g.bufs, am, ls=ls, ws=ws)
    nc.nc_scale_update(nc.policy("e4m3", "current", hysteresis=False), st, am)
    out = nc.new_counts(T)
    fn = lambda: nc.nc_cast_tensor(g.bufs, codes, "e4m3", st, out, ls=ls, ws=ws)
    fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    n = g.total
    nbytes = 5 * n
    gbps = nbytes / (ms * 1e-3) / 1e9
    nonfinite = int(sum(c["n_nonfinite"] for c in nc.counts_list(out))) // (len(ev) + 1)
    del g, codes, ws
    torch.cuda.empty_cache()
    return dict(ms=round(ms, 4), gbps=round(gbps, 1), frac=round(gbps / HBM_PEAK_GBPS, 4),
                gelem_s=round(n / (ms * 1e-3) / 1e9, 2), elements=n, tensors=T,
                nonfinite_per_step=nonfinite)


def _timed(torch, fn, reps, flush=None):
    """Median of reps event-timed calls of fn on the current stream (ms);
    flush(), if given, runs untimed before each call."""
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def _captured(torch, fn):
    """fn's launches captured once into a HIP graph (after one warm run on a
    side stream, as graph capture wants); returns the graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def small_configs(nc, torch, workloads):
    """The three smaller workloads, timed on their own: a 65,536-element fp32
    vector under current per-tensor E4M3 scaling (amax, scale update, cast:
    launch-bound, so microseconds, not bandwidth); the 4096 x 4096 tanh bf16
    matrix cast to MXFP8 E4M3 under the OCP, +1 and ceil rules; and one step of
    delayed per-tensor E5M2 scaling over 64 fp32 gradient tensors (2^12 to
    2^22 elements) with a 16-step window.  Their working sets fit the GPU's
    last-level cache, so a 1 GiB buffer is read before every timed rep
    (untimed; a read leaves no dirty lines to write back during the rep) and
    each rep starts from HBM.  These sizes are launch-bound, so each is timed
    as eager calls and as one replay of the same calls captured in a HIP
    graph.  Medians of 20 reps."""
    dev = "cuda"
    print("[bench] smaller workloads", file=sys.stderr, flush=True)
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    flush = lambda: scratch.sum(dtype=torch.int64)
    res = {}

    def both(fn, reps=20):
        eager = _timed(torch, fn, reps, flush)
        g = _captured(torch, fn)
        graph = _timed(torch, g.replay, reps, flush)
        return eager, graph
    # 65,536 fp32 ~ N(0, 1): amax -> current scale -> cast
    x = torch.from_numpy(workloads.per_tensor_small()).to(dev)
    codes = torch.empty(x.numel(), dtype=torch.uint8, device=dev)
    desc, cnt = nc.tensors([x], [codes])
    ws = nc.new_workspace(desc, cnt)
    st, am, out = nc.new_state(1), nc.new_counts(1), nc.new_counts(1)
    pol = nc.policy("e4m3", "current", hysteresis=False)

    def c1():
        nc.nc_amax([x], am, ws=ws)
        nc.nc_scale_update(pol, st, am)
        nc.nc_cast_tensor([x], [codes], "e4m3", st, out, ws=ws)
    c1()
    ms, msg = both(c1)
    res["per_tensor_65536_fp32"] = dict(us=round(ms * 1e3, 1), us_graph=round(msg * 1e3, 1), elements=x.numel(),
                                        launches=3,
                                        note="amax + scale update + cast (each under 64 workgroups, so their "
                                             "counts go straight to the output: no slot pass), launch-bound")
    # 4096 x 4096 tanh(N(0, 1.5)) bf16, MXFP8 E4M3 per rule
    xb = torch.from_numpy(workloads.tanh_activations().reshape(-1).view(np.int16)).to(dev).view(torch.bfloat16)
    n = xb.numel()
    codes = torch.empty(n, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 32, dtype=torch.uint8, device=dev)
    desc, cnt = nc.tensors([xb], [codes])
    ws = nc.new_workspace(desc, cnt)
    for rule in ("ocp", "plus1", "ceil"):
        # what the cast does to this tensor under the rule, from one untimed
        # call with the statistics: clipped fraction, mean signed error, the
        # error along each element's own sign, the fraction kept along itself
        out, sts = nc.new_counts(1), nc.new_stats(1)
        nc.nc_cast_mx([xb], [codes], [scales], [4096], "e4m3", rule, out, stats=sts, ws=ws)
        torch.cuda.synchronize()
        c = nc.counts_list(out)[0]
        sm = dict(zip(nc.STAT_FIELDS, sts[0].cpu().tolist()))
        nf = c["n_finite"]
        out = nc.new_counts(1)
        fn = lambda: nc.nc_cast_mx([xb], [codes], [scales], [4096], "e4m3", rule, out, ws=ws)
        ms, msg = both(fn)
        nbytes = 3 * n + n // 32
        res[f"mx_tanh_4096x4096_{rule}"] = dict(
            us=round(ms * 1e3, 1), gbps=round(nbytes / (ms * 1e-3) / 1e9, 1),
            frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), us_graph=round(msg * 1e3, 1),
            clip_frac=round(c["n_clip"] / n, 5), mean_signed_error=sm["sum_e"] / nf,
            sign_aligned_bias=sm["sum_dir_e"] / nf, kept_fraction=1.0 + sm["sum_xe"] / sm["sum_x2"],
            rel_rms_error=(sm["sum_e2"] / sm["sum_x2"]) ** 0.5)
    # 64 fp32 tensors, delayed E5M2 scaling with a 16-step window: one batched
    # cast (counts and next amax fused) and one scale update per step
    gen = workloads.GradientSteps(steps=4)
    T = len(gen.sizes)
    xs = [torch.from_numpy(v).to(dev) for v in gen.step(0)]
    codes = [torch.empty(m, dtype=torch.uint8, device=dev) for m in gen.sizes]
    desc, cnt = nc.tensors(xs, codes)
    ws = nc.new_workspace(desc, cnt)
    st, hist, am = nc.new_state(T), nc.new_history(T, 16), nc.new_counts(T)
    nc.nc_amax(xs, am, ws=ws)
    nc.nc_scale_update(nc.policy("e5m2", "current", 16), st, am)
    pol = nc.policy("e5m2", "max_window", 16)
    out = nc.new_counts(T)

    def c3():
        out.zero_()
        nc.nc_cast_tensor(xs, codes, "e5m2", st, out, ws=ws)
        nc.nc_scale_update(pol, st, out, hist)
    c3()
    g = _captured(torch, c3)
    ms, msg = [], []
    for t in range(1, gen.steps):          # fresh values every step, uploaded untimed
        for d, v in zip(xs, gen.step(t)):
            d.copy_(torch.from_numpy(v))
        ms.append(_timed(torch, c3, 5, flush))
        msg.append(_timed(torch, g.replay, 5, flush))
    ms, msg = float(np.median(ms)), float(np.median(msg))
    ne = sum(gen.sizes)
    res["delayed_64_tensors_fp32"] = dict(
        us=round(ms * 1e3, 1), gbps=round(5 * ne / (ms * 1e-3) / 1e9, 1),
        frac=round(5 * ne / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), us_graph=round(msg * 1e3, 1),
        elements=ne, tensors=T,
        note="per step: counter zeroing, one batched cast, one scale update")
    del scratch, g
    torch.cuda.empty_cache()
    return res


def fused_step(a, torch, nc, bufs, t, sep):
    """The step's outputs with the statistics fused into the two casts instead
    of two separate statistics passes: amax, scale update, both casts with
    statistics, both dequants.  Timed like the step (after two untimed
    steps); its statistics are compared with `sep`, those of the separate
    passes in the last timed step (same input, same scale)."""
    n = t["x"].numel()

    def step():
        for b in ("am", "cpt", "cmx", "spt", "smx"):
            bufs[b].zero_()
        nc.nc_amax([t["x"]], bufs["am"], ws=t["ws"])
        nc.nc_scale_update(t["pol"], bufs["st"], bufs["am"])
        nc.nc_cast_tensor([t["x"]], [t["codes_pt"]], "e4m3", bufs["st"], bufs["cpt"], stats=bufs["spt"],
                          ws=t["ws"])
        nc.nc_cast_mx([t["x"]], [t["codes_mx"]], [t["scales"]], [COLS], "e4m3", "ocp", bufs["cmx"],
                      stats=bufs["smx"], ws=t["ws"])
        nc.nc_dequant([t["codes_pt"]], [t["y_pt"]], "e4m3", st=bufs["st"])
        nc.nc_dequant([t["codes_mx"]], [t["y_mx"]], "e4m3", scales=[t["scales"]], cols=[COLS])

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    k = max(1, min(a.steps, 10))
    t0 = time.perf_counter()
    for _ in range(k):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / k
    rel = max(float(((f - s).abs() / s.abs().clamp_min(1e-300)).max())
              for f, s in zip((bufs["spt"], bufs["smx"]), sep))
    nbytes = 2 * n + 3 * n + (3 * n + n // 32) + 3 * n + (3 * n + n // 32)
    return dict(ms_per_step=round(ms, 4), gelem_s=round(n / (ms * 1e-3) / 1e9, 3), steps=k,
                step_bytes=nbytes, frac_of_peak=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                stats_max_rel_diff_vs_passes=rel,
                calls="amax, scale update, cast_tensor + statistics, cast_mx + statistics, dequant x2")


def main():
    a = parse()
    if a.write_traffic:
        write_traffic(*a.write_traffic)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {a.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import scaled_fp8_casting_amd as nc
    import workloads

    if not a.make_input and not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    rows = a.rows
    n = rows * COLS
    t = time.time()
    cache = a.input_cache
    if cache and os.path.exists(cache) and os.path.getsize(cache) == 2 * n:
        print(f"[bench] loading {rows}x{COLS} bf16 from {cache}", file=sys.stderr, flush=True)
        host = np.fromfile(cache, dtype=np.uint16).reshape(rows, COLS)
    else:
        print(f"[bench] generating {rows}x{COLS} bf16 on {a.procs} processes", file=sys.stderr, flush=True)
        host = workloads.heavy_tailed_parallel(rows, COLS, procs=a.procs)
        if cache:
            host.tofile(cache)
    if a.make_input:
        print(f"[bench] wrote {cache}", file=sys.stderr, flush=True)
        return
    print(f"[bench] input ready in {time.time() - t:.1f}s; uploading", file=sys.stderr, flush=True)
    x = torch.from_numpy(host.view(np.int16).reshape(-1)).cuda().view(torch.bfloat16)
    del host
    dev = "cuda"
    codes_pt = torch.empty(n, dtype=torch.uint8, device=dev)
    codes_mx = torch.empty(n, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 32, dtype=torch.uint8, device=dev)
    y_pt = torch.empty(n, dtype=torch.bfloat16, device=dev)
    y_mx = torch.empty(n, dtype=torch.bfloat16, device=dev)
    desc, cnt = nc.tensors([x], [codes_pt])
    ws = nc.new_workspace(desc, cnt)
    pol = nc.policy("e4m3", "current", hysteresis=False)
    bufs = dict(am=nc.new_counts(1), cpt=nc.new_counts(1), cmx=nc.new_counts(1),
                spt=nc.new_stats(1), smx=nc.new_stats(1), st=nc.new_state(1))

    names = ["amax", "scale_update", "cast_tensor", "cast_mx", "dequant_pt", "dequant_mx",
             "stats_pt", "stats_mx"]
    alg_bytes = {"amax": 2 * n, "scale_update": 0, "cast_tensor": 3 * n, "cast_mx": 3 * n + n // 32,
                 "dequant_pt": 3 * n, "dequant_mx": 3 * n + n // 32, "stats_pt": 3 * n,
                 "stats_mx": 3 * n + n // 32}
    kernel_of = {"amax": "k_amax", "cast_tensor": "k_cast_pt", "cast_mx": "k_cast_mx",
                 "dequant_pt": "k_dequant", "dequant_mx": "k_dequant", "stats_pt": "k_stats",
                 "stats_mx": "k_stats"}

    def step(ev=None):
        for b in ("am", "cpt", "cmx", "spt", "smx"):
            bufs[b].zero_()
        calls = [
            lambda: nc.nc_amax([x], bufs["am"], ws=ws),
            lambda: nc.nc_scale_update(pol, bufs["st"], bufs["am"]),
            lambda: nc.nc_cast_tensor([x], [codes_pt], "e4m3", bufs["st"], bufs["cpt"], ws=ws),
            lambda: nc.nc_cast_mx([x], [codes_mx], [scales], [COLS], "e4m3", "ocp", bufs["cmx"], ws=ws),
            lambda: nc.nc_dequant([codes_pt], [y_pt], "e4m3", st=bufs["st"]),
            lambda: nc.nc_dequant([codes_mx], [y_mx], "e4m3", scales=[scales], cols=[COLS]),
            lambda: nc.nc_cast_stats([x], [codes_pt], "e4m3", bufs["spt"], ws, st=bufs["st"]),
            lambda: nc.nc_cast_stats([x], [codes_mx], "e4m3", bufs["smx"], ws, scales=[scales], cols=[COLS]),
        ]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i][0].record()
            c()
            if ev is not None:
                ev[i][1].record()

    wev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in names] for _ in range(a.warmup)]
    for w in range(a.warmup):
        step(wev[w])
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {a.steps} steps", file=sys.stderr, flush=True)
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in names] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / a.steps
    sep_stats = [bufs["spt"].clone(), bufs["smx"].clone()]   # the last step's statistics passes
    per = {nm: float(np.mean([evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(a.steps)]))
           for i, nm in enumerate(names)}
    kernels = {}
    for nm in names:
        gbps = alg_bytes[nm] / (per[nm] * 1e-3) / 1e9 if alg_bytes[nm] else None
        kernels[nm] = dict(ms=round(per[nm], 4), gbps=None if gbps is None else round(gbps, 1),
                           frac=None if gbps is None else round(gbps / HBM_PEAK_GBPS, 4),
                           gelem_s=round(n / (per[nm] * 1e-3) / 1e9, 2) if alg_bytes[nm] else None)
    # per-step sums of the calls' event times, warm-up steps first (no extra
    # synchronisation: the events were recorded around every call anyway)
    def call_ms(ev_step, i):
        return ev_step[i][0].elapsed_time(ev_step[i][1])
    i_mx = names.index("cast_mx")
    series = {"warmup_ms": [round(sum(call_ms(e, i) for i in range(len(names))), 4) for e in wev],
              "timed_ms": [round(sum(call_ms(e, i) for i in range(len(names))), 4) for e in evs],
              "cast_mx_warmup_ms": [round(call_ms(e, i_mx), 4) for e in wev],
              "cast_mx_timed_ms": [round(call_ms(e, i_mx), 4) for e in evs]}
    dom = max((nm for nm in names if alg_bytes[nm]), key=lambda nm: per[nm])
    ach = alg_bytes[dom] / (per[dom] * 1e-3) / 1e9
    src = source_hash()
    step_bytes = sum(alg_bytes.values())
    cc = nc.counts_list(bufs["cpt"])[0]
    cm = nc.counts_list(bufs["cmx"])[0]
    out = {
        "metric": "scaled FP8 cast Gelem/s and achieved HBM GB/s (% of peak), per-tensor + MX",
        "value": round(n / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gelem/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "heavy-tailed bf16 2^30 (262144x4096, 10^U(-3,3) * t3 rows): amax, "
                               "current-scaling E4M3 cast, MXFP8 E4M3 OCP cast, dequant x2, stats x2",
                   "elements": n, "rows": rows, "cols": COLS, "parallelism": "single GPU"},
        "hbm": {"step_bytes": step_bytes, "achieved_GBps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                "frac_of_peak": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": kernel_of[dom], "call": dom, "achieved": round(ach, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                     "bytes_per_launch": alg_bytes[dom],
                     "traffic": traffic_for(dom, src)},
        "results": {"k": int(bufs["st"][0, 0]), "amax": nc.counts_list(bufs["am"])[0]["amax"],
                    "pt_clip": cc["n_clip"], "pt_underflow_frac": round(cc["n_underflow"] / n, 5),
                    "mx_clip_frac": round(cm["n_clip"] / n, 5)},
        "source_hash": src,
        "step_series": series,
    }
    # Beside the step (not part of it): the casts with their statistics fused
    # (one pass instead of cast + separate statistics pass), and torch's own
    # device copy of the cast's byte count (context only: a copy kernel that
    # is not tuned for HBM, so it bounds nothing here).
    fused_pt, fused_mx = nc.new_stats(1), nc.new_stats(1)
    extras = {
        "cast_tensor+stats": (lambda: nc.nc_cast_tensor([x], [codes_pt], "e4m3", bufs["st"], bufs["cpt"],
                                                        stats=fused_pt, ws=ws), 3 * n),
        "cast_mx+stats": (lambda: nc.nc_cast_mx([x], [codes_mx], [scales], [COLS], "e4m3", "ocp", bufs["cmx"],
                                                stats=fused_mx, ws=ws), 3 * n + n // 32),
        # stochastic rounding (Philox4x32-10 draws, one 32-bit uniform per element)
        "cast_tensor_sr": (lambda: nc.nc_cast_tensor_sr([x], [codes_pt], "e4m3", bufs["st"], bufs["cpt"], 2024, 7,
                                                        ws=ws), 3 * n),
        # MX with blocks of 32 rows of a column (the transposed operand's layout)
        "cast_mx_cols": (lambda: nc.nc_cast_mx([x], [codes_mx], [scales], [COLS], "e4m3", "ocp", bufs["cmx"],
                                               ws=ws, axis="cols"), 3 * n + n // 32),
        "dequant_mx_cols": (lambda: nc.nc_dequant([codes_mx], [y_mx], "e4m3", scales=[scales], cols=[COLS],
                                                  axis="cols"), 3 * n + n // 32),
        "stats_mx_cols": (lambda: nc.nc_cast_stats([x], [codes_mx], "e4m3", bufs["smx"], ws, scales=[scales],
                                                   cols=[COLS], axis="cols"), 3 * n + n // 32),
    }
    if not a.copy_probe:     # (a counter run keeps the probe's copies the only large ones)
        cp_src = torch.empty(3 * n // 2, dtype=torch.uint8, device=dev).fill_(1)
        cp_dst = torch.empty_like(cp_src)
        extras["torch_copy"] = (lambda: cp_dst.copy_(cp_src), 3 * n)
    out["beside_step"] = {}
    for nm, (fn, nbytes) in extras.items():
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
        gbps = nbytes / (ms * 1e-3) / 1e9
        out["beside_step"][nm] = dict(ms=round(ms, 4), gbps=round(gbps, 1), frac=round(gbps / HBM_PEAK_GBPS, 4),
                                      gelem_s=round(n / (ms * 1e-3) / 1e9, 2), traffic=traffic_for(nm, src))
    extras.clear()
    out["step_fused_stats"] = fused_step(a, torch, nc, bufs, dict(
        x=x, codes_pt=codes_pt, codes_mx=codes_mx, scales=scales, y_pt=y_pt, y_mx=y_mx, ws=ws, pol=pol),
        sep_stats)
    # the update/step-ratio monitor on its own workload: 2^30 fp32 weights and
    # updates (8 GiB read), bf16 weight copies, counts only
    del y_pt, y_mx
    torch.cuda.empty_cache()
    upd = workloads.UpdateStep(rows=rows)
    sw_out = nc.new_swamp_counts(1)
    sw_ws = nc.new_swamp_workspace([upd.w], [upd.d])
    fn = lambda: nc.nc_swamp_watch([upd.w], [upd.d], "bf16", sw_out, workspace=sw_ws)
    fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    gbps = 8 * n / (ms * 1e-3) / 1e9
    sc = nc.swamp_counts_list(sw_out)[0]
    out["beside_step"]["swamp_watch"] = dict(
        ms=round(ms, 4), gbps=round(gbps, 1), frac=round(gbps / HBM_PEAK_GBPS, 4),
        gelem_s=round(n / (ms * 1e-3) / 1e9, 2), traffic=traffic_for("swamp_watch", src),
        workload="UpdateStep 2^30 fp32 w, d (w ~ N(0, 0.02), d = 1e-4 g 10^U(-3,1) per row); bf16 copies",
        below_frac=round(sc["n_below"] / max(sc["n_considered"], 1), 4),
        noop_frac=round(sc["n_noop"] / max(sc["n_considered"], 1), 4))
    # the same with a flag byte per element written (9 B/elem)
    flags = torch.empty(n, dtype=torch.uint8, device=dev)
    fn = lambda: nc.nc_swamp_watch([upd.w], [upd.d], "bf16", sw_out, flags=[flags], workspace=sw_ws)
    fn()
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    gbps = 9 * n / (ms * 1e-3) / 1e9
    out["beside_step"]["swamp_watch_flags"] = dict(
        ms=round(ms, 4), gbps=round(gbps, 1), frac=round(gbps / HBM_PEAK_GBPS, 4),
        gelem_s=round(n / (ms * 1e-3) / 1e9, 2), traffic=traffic_for("swamp_watch_flags", src))
    del upd, sw_ws, flags
    torch.cuda.empty_cache()
    if not a.no_llama:
        out["beside_step"]["llama_unscale_cast"] = llama_unscale_cast(nc, torch, workloads)
    if not a.no_configs:
        out["configs"] = small_configs(nc, torch, workloads)
    if a.copy_probe:
        src_b = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst_b = torch.empty_like(src_b)
        for _ in range(3):
            dst_b.copy_(src_b)
        torch.cuda.synchronize()
        del src_b, dst_b
    if not a.no_cpu:
        print(f"[bench] CPU oracle baseline on {a.cpu_rows} rows", file=sys.stderr, flush=True)
        try:
            out["cpu_baseline"] = cpu_baseline(a.cpu_rows, a.procs)
        except mp_timeout():
            print("[bench] CPU oracle baseline timed out", file=sys.stderr, flush=True)
            out["cpu_baseline"] = None
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
