"""scaled_fp8_casting_amd: the scaled FP8 cast on MI355X (gfx950).

A thin Python binding over libnarrowcast's C-ABI (include/narrowcast.h).
Functions carry the C names and only marshal arguments: torch tensors
provide device memory and the current HIP stream; every step of the cast
runs in the library's HIP kernels.  There is no CPU fallback: calls raise if
the library is not built or a tensor is not on the GPU.

Device buffers used by the calls, as torch tensors:

* counts: int64 [count, 5] -- n_finite, n_clip, n_underflow, n_nonfinite,
  then amax (fp32 bits in the low 32 bits of the fifth word);
* stats:  float64 [count, 6] -- sum e, |e|, e^2, sign(x) e, x e, x^2;
* state:  int32 [count, 6] -- k, a_ref bits, has_ref, n_hist, head, step;
* hist:   float32 [count, window];
* loss scale: int32 [2] -- s_log2, clean_steps.
"""

import ctypes
import struct
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import (NC_BF16, NC_E4M3, NC_E5M2, NC_EST_CURRENT, NC_EST_EMA, NC_EST_MAX_WINDOW,  # noqa: F401
                   NC_EST_MOST_RECENT, NC_F32, NC_MX_CEIL, NC_MX_OCP, NC_MX_PLUS1, NC_W_BF16, NC_W_FP16,
                   NcPolicy, NcSwampPolicy, NcTensor, NcUpdateTensor)

COUNT_FIELDS = ("n_finite", "n_clip", "n_underflow", "n_nonfinite")
STAT_FIELDS = ("sum_e", "sum_abs_e", "sum_e2", "sum_dir_e", "sum_xe", "sum_x2")
STATE_FIELDS = ("k", "a_ref_bits", "has_ref", "n_hist", "head", "step")

FMT = {"e4m3": NC_E4M3, "e5m2": NC_E5M2}
MX_RULE = {"ocp": NC_MX_OCP, "plus1": NC_MX_PLUS1, "ceil": NC_MX_CEIL}
MX_AXIS = {"rows": 0, "cols": 1}
EST = {"current": NC_EST_CURRENT, "most_recent": NC_EST_MOST_RECENT, "max_window": NC_EST_MAX_WINDOW,
       "ema": NC_EST_EMA}


class NarrowcastError(RuntimeError):
    def __init__(self, status: int, call: str):
        msg = _lib.load().nc_status_string(status).decode()
        super().__init__(f"{call}: status {status}: {msg}")
        self.status = status


def _check(status: int, call: str):
    if status != 0:
        raise NarrowcastError(status, call)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return NC_F32
    if t.dtype == torch.bfloat16:
        return NC_BF16
    raise TypeError(f"input dtype {t.dtype} (float32 or bfloat16 expected)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected (no CPU path)")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, rows: int, width: Optional[int] = None):
    """Raise ValueError unless t is a contiguous `dtype` tensor holding at least
    `rows` rows of `width` elements (or `rows` elements when width is None):
    the kernels write (or read) that many, so a smaller buffer would be
    overrun on the GPU."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: contiguous tensor expected")
    if width is None:
        if t.numel() < rows:
            raise ValueError(f"{name}: {t.numel()} elements, at least {rows} needed")
    elif t.dim() != 2 or t.shape[1] != width or t.shape[0] < rows:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected ({rows}, {width}) or more rows")


def tensors(xs: Sequence[Optional[torch.Tensor]], codes: Sequence[Optional[torch.Tensor]],
            cols: Optional[Sequence[int]] = None, scales: Optional[Sequence[torch.Tensor]] = None,
            n: Optional[Sequence[int]] = None, axis: str = "rows"):
    """A host array of nc_tensor descriptors (contiguous device tensors).

    Before any pointer is taken, the sizes are checked against what the
    kernels will touch: every input has the first input's dtype (fp32 or
    bf16), every code buffer is uint8 with exactly as many elements as its
    input, every scale buffer uint8 with one byte per 32 elements, and the
    per-tensor lists have one entry per tensor.  A mismatch raises
    ValueError."""
    count = len(codes)
    for name, lst in (("xs", xs), ("cols", cols), ("scales", scales), ("n", n)):
        if lst is not None and len(lst) != count:
            raise ValueError(f"{name}: {len(lst)} entries for {count} tensors")
    if axis not in MX_AXIS:
        raise ValueError(f"axis {axis!r}")
    dt0 = None
    if xs is not None and count:
        dt0 = xs[0].dtype
        _dtype_code(xs[0])
    ns = []
    for i in range(count):
        x = xs[i] if xs is not None else None
        c = codes[i]
        if x is not None and x.dtype != dt0:
            raise ValueError(f"xs[{i}]: dtype {x.dtype}, but xs[0] is {dt0} (one dtype per call)")
        for t in (x, c):
            if t is not None and not t.is_contiguous():
                raise ValueError("contiguous tensors expected")
        ni = n[i] if n is not None else (x.numel() if x is not None else c.numel())
        if x is not None and x.numel() != ni:
            raise ValueError(f"xs[{i}]: {x.numel()} elements, n = {ni}")
        if c is not None:
            if c.dtype != torch.uint8:
                raise ValueError(f"codes[{i}]: dtype {c.dtype}, expected torch.uint8")
            if c.numel() != ni:
                raise ValueError(f"codes[{i}]: {c.numel()} elements for {ni} inputs")
        if scales is not None:
            sc = scales[i]
            if sc.dtype != torch.uint8 or not sc.is_contiguous():
                raise ValueError(f"scales[{i}]: contiguous torch.uint8 expected")
            if sc.numel() != ni // 32:
                raise ValueError(f"scales[{i}]: {sc.numel()} bytes for {ni // 32} blocks of 32")
        ns.append(ni)
    arr = (NcTensor * max(count, 1))()
    for i in range(count):
        x = xs[i] if xs is not None else None
        c = codes[i]
        arr[i].x = _ptr(x) if x is not None and x.numel() else None
        arr[i].codes = _ptr(c) if c is not None and c.numel() else None
        arr[i].n = ns[i]
        arr[i].cols = cols[i] if cols is not None else 0
        arr[i].scales = _ptr(scales[i]) if scales is not None and scales[i].numel() else None
        arr[i].mx_axis = MX_AXIS[axis]
    return arr, count


# -- device buffers ---------------------------------------------------------

def new_counts(count: int, device="cuda") -> torch.Tensor:
    return torch.zeros((count, 5), dtype=torch.int64, device=device)


def new_stats(count: int, device="cuda") -> torch.Tensor:
    return torch.zeros((count, 6), dtype=torch.float64, device=device)


def new_state(count: int, device="cuda") -> torch.Tensor:
    return torch.zeros((count, 6), dtype=torch.int32, device=device)


def new_history(count: int, window: int, device="cuda") -> torch.Tensor:
    return torch.zeros((count, window), dtype=torch.float32, device=device)


def new_loss_scale(s_log2: int, device="cuda") -> torch.Tensor:
    return torch.tensor([s_log2, 0], dtype=torch.int32, device=device)


def policy(fmt="e4m3", est="max_window", window=16, margin=0, hysteresis=True, interval=1,
           skip_on_nonfinite=False, ls_enable=False, ls_growth_interval=2000, ls_log2_min=0,
           ls_log2_max=24, ema_alpha=0.0625) -> NcPolicy:
    return NcPolicy(FMT[fmt] if isinstance(fmt, str) else fmt, EST[est] if isinstance(est, str) else est,
                    window, margin, int(hysteresis), interval, int(skip_on_nonfinite), int(ls_enable),
                    ls_growth_interval, ls_log2_min, ls_log2_max, ema_alpha)


def counts_list(counts: torch.Tensor):
    """Host view of a counts tensor: one dict per tensor (amax as a float)."""
    rows = counts.cpu().tolist()
    out = []
    for r in rows:
        d = dict(zip(COUNT_FIELDS, r[:4]))
        d["amax_bits"] = r[4] & 0xFFFFFFFF
        d["amax"] = struct.unpack("<f", struct.pack("<I", d["amax_bits"]))[0]
        out.append(d)
    return out


def workspace_bytes(desc, count: int) -> int:
    return int(_lib.load().nc_workspace_bytes(desc, count))


def new_workspace(desc, count: int, device="cuda") -> torch.Tensor:
    """Device workspace for the calls that reduce (amax, casts, statistics);
    torch's allocator returns 256-byte aligned memory."""
    return torch.empty(max(workspace_bytes(desc, count), 16), dtype=torch.uint8, device=device)


def _check_cast_outputs(count, st, out, ls, stats, ws):
    _need(st, "st", torch.int32, count, 6)
    _need(out, "out", torch.int64, count, 5)
    _need(ls, "ls", torch.int32, 2)
    _need(stats, "stats", torch.float64, count, 6)
    _need(ws, "ws", torch.uint8, 0)


def _ws(ws, desc, count):
    return new_workspace(desc, count) if ws is None else ws


# -- the C-ABI calls ----------------------------------------------------------

def nc_amax(xs: Sequence[torch.Tensor], out: torch.Tensor, ls: Optional[torch.Tensor] = None,
            ws: Optional[torch.Tensor] = None, stream=None):
    _need(out, "out", torch.int64, len(xs), 5)
    _need(ls, "ls", torch.int32, 2)
    _need(ws, "ws", torch.uint8, 0)
    desc, count = tensors(xs, [None] * len(xs))
    dt = _dtype_code(xs[0]) if xs else NC_F32
    ws = _ws(ws, desc, count)
    _check(_lib.load().nc_amax(desc, count, dt, _ptr(ls), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
           "nc_amax")


def nc_scale_update(pol: NcPolicy, st: torch.Tensor, in_counts: torch.Tensor,
                    hist: Optional[torch.Tensor] = None, ls: Optional[torch.Tensor] = None,
                    stream=None):
    count = st.shape[0]
    _need(st, "st", torch.int32, count, 6)
    _need(in_counts, "in_counts", torch.int64, count, 5)
    _need(hist, "hist", torch.float32, count * pol.window)
    _need(ls, "ls", torch.int32, 2)
    _check(_lib.load().nc_scale_update(ctypes.byref(pol), count, _ptr(st), _ptr(hist),
                                       _ptr(in_counts), _ptr(ls), _stream(stream)), "nc_scale_update")


def nc_cast_tensor(xs: Sequence[torch.Tensor], codes: Sequence[torch.Tensor], fmt, st: torch.Tensor,
                   out: torch.Tensor, ls: Optional[torch.Tensor] = None,
                   stats: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                   stream=None):
    _check_cast_outputs(len(codes), st, out, ls, stats, ws)
    desc, count = tensors(xs, codes)
    dt = _dtype_code(xs[0]) if xs else NC_F32
    f = FMT[fmt] if isinstance(fmt, str) else fmt
    ws = _ws(ws, desc, count)
    _check(_lib.load().nc_cast_tensor(desc, count, dt, f, _ptr(st), _ptr(ls), _ptr(out), _ptr(stats),
                                      _ptr(ws), ws.numel(), _stream(stream)), "nc_cast_tensor")


def nc_cast_tensor_static(xs: Sequence[torch.Tensor], codes: Sequence[torch.Tensor], fmt, st: torch.Tensor,
                          out: torch.Tensor, ls: Optional[torch.Tensor] = None,
                          stats: Optional[torch.Tensor] = None, stream=None):
    """nc_cast_tensor without a workspace: the library's static per-GPU
    scratch serves instead, so nothing is allocated (for callers that cannot
    allocate).  Calls that overlap on one GPU race on that scratch."""
    _check_cast_outputs(len(codes), st, out, ls, stats, None)
    desc, count = tensors(xs, codes)
    dt = _dtype_code(xs[0]) if xs else NC_F32
    f = FMT[fmt] if isinstance(fmt, str) else fmt
    _check(_lib.load().nc_cast_tensor_static(desc, count, dt, f, _ptr(st), _ptr(ls), _ptr(out), _ptr(stats),
                                             _stream(stream)), "nc_cast_tensor_static")


def nc_cast_tensor_sr(xs: Sequence[torch.Tensor], codes: Sequence[torch.Tensor], fmt, st: torch.Tensor,
                      out: torch.Tensor, seed: int, offset: int, ls: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None):
    _check_cast_outputs(len(codes), st, out, ls, None, ws)
    desc, count = tensors(xs, codes)
    dt = _dtype_code(xs[0]) if xs else NC_F32
    f = FMT[fmt] if isinstance(fmt, str) else fmt
    ws = _ws(ws, desc, count)
    _check(_lib.load().nc_cast_tensor_sr(desc, count, dt, f, _ptr(st), _ptr(ls), seed & (2 ** 64 - 1),
                                         offset & (2 ** 64 - 1), _ptr(out), _ptr(ws), ws.numel(),
                                         _stream(stream)), "nc_cast_tensor_sr")


def nc_cast_mx(xs: Sequence[torch.Tensor], codes: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
               cols: Sequence[int], fmt, rule, out: torch.Tensor, stats: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, stream=None, axis: str = "rows"):
    _check_cast_outputs(len(codes), None, out, None, stats, ws)
    desc, count = tensors(xs, codes, cols=cols, scales=scales, axis=axis)
    dt = _dtype_code(xs[0]) if xs else NC_BF16
    f = FMT[fmt] if isinstance(fmt, str) else fmt
    r = MX_RULE[rule] if isinstance(rule, str) else rule
    ws = _ws(ws, desc, count)
    _check(_lib.load().nc_cast_mx(desc, count, dt, f, r, _ptr(out), _ptr(stats), _ptr(ws), ws.numel(),
                                  _stream(stream)), "nc_cast_mx")


def nc_dequant(codes: Sequence[torch.Tensor], ys: Sequence[torch.Tensor], fmt,
               st: Optional[torch.Tensor] = None, scales: Optional[Sequence[torch.Tensor]] = None,
               cols: Optional[Sequence[int]] = None, stream=None, axis: str = "rows"):
    count = len(codes)
    if len(ys) != count:
        raise ValueError(f"ys: {len(ys)} entries for {count} tensors")
    for i, y in enumerate(ys):
        if y.dtype != torch.bfloat16 or not y.is_contiguous():
            raise TypeError("dequant output must be contiguous bfloat16")
        if y.numel() != codes[i].numel():
            raise ValueError(f"ys[{i}]: {y.numel()} elements for {codes[i].numel()} codes")
    _need(st, "st", torch.int32, count, 6)
    desc, count = tensors(None, codes, cols=cols, scales=scales, axis=axis)
    f = FMT[fmt] if isinstance(fmt, str) else fmt
    yp = (ctypes.c_void_p * max(count, 1))(*[_ptr(y) if y.numel() else None for y in ys])
    _check(_lib.load().nc_dequant(desc, count, f, _ptr(st), yp, NC_BF16, _stream(stream)), "nc_dequant")


def nc_cast_stats(xs: Sequence[torch.Tensor], codes: Sequence[torch.Tensor], fmt, out: torch.Tensor,
                  ws: Optional[torch.Tensor] = None, st: Optional[torch.Tensor] = None,
                  ls: Optional[torch.Tensor] = None,
                  scales: Optional[Sequence[torch.Tensor]] = None, cols: Optional[Sequence[int]] = None,
                  stream=None, axis: str = "rows"):
    _need(out, "out", torch.float64, len(codes), 6)
    _need(st, "st", torch.int32, len(codes), 6)
    _need(ls, "ls", torch.int32, 2)
    _need(ws, "ws", torch.uint8, 0)
    desc, count = tensors(xs, codes, cols=cols, scales=scales, axis=axis)
    dt = _dtype_code(xs[0]) if xs else NC_F32
    f = FMT[fmt] if isinstance(fmt, str) else fmt
    ws = _ws(ws, desc, count)
    _check(_lib.load().nc_cast_stats(desc, count, dt, f, _ptr(st), _ptr(ls), _ptr(out), _ptr(ws),
                                     ws.numel(), _stream(stream)), "nc_cast_stats")


# -- the update/step-ratio ("swamping") monitor -------------------------------

WFMT = {"bf16": NC_W_BF16, "fp16": NC_W_FP16}
SWAMP_FIELDS = ("n_considered", "n_zero", "n_below", "n_noop", "n_excluded")


def update_tensors(ws: Sequence[torch.Tensor], ds: Sequence[torch.Tensor],
                   flags: Optional[Sequence[Optional[torch.Tensor]]] = None):
    """A host array of nc_update_tensor descriptors (contiguous fp32 device tensors)."""
    count = len(ws)
    if len(ds) != count or (flags is not None and len(flags) != count):
        raise ValueError("one update (and flag buffer) per weight tensor")
    for i in range(count):
        w, d = ws[i], ds[i]
        for t in (w, d):
            if t.dtype != torch.float32 or not t.is_contiguous():
                raise TypeError("weights and updates must be contiguous float32")
        if w.numel() != d.numel():
            raise ValueError("a weight tensor and its update differ in size")
        if flags is not None and flags[i] is not None:
            _need(flags[i], f"flags[{i}]", torch.uint8, w.numel())
            if flags[i].numel() != w.numel():
                raise ValueError(f"flags[{i}]: {flags[i].numel()} bytes for {w.numel()} elements")
    arr = (NcUpdateTensor * max(count, 1))()
    for i in range(count):
        w, d = ws[i], ds[i]
        arr[i].w = _ptr(w) if w.numel() else None
        arr[i].d = _ptr(d) if d.numel() else None
        f = flags[i] if flags is not None else None
        arr[i].flags = _ptr(f) if f is not None and f.numel() else None
        arr[i].n = w.numel()
    return arr, count


def new_swamp_counts(count: int, device="cuda") -> torch.Tensor:
    return torch.zeros((count, 5), dtype=torch.int64, device=device)


def new_swamp_state(count: int, device="cuda") -> torch.Tensor:
    return torch.zeros((count, 4), dtype=torch.int32, device=device)


def swamp_policy(window=8, num=1, den=2) -> NcSwampPolicy:
    return NcSwampPolicy(window, num, den, 0)


def swamp_counts_list(counts: torch.Tensor):
    return [dict(zip(SWAMP_FIELDS, r)) for r in counts.cpu().tolist()]


def new_swamp_workspace(ws: Sequence[torch.Tensor], ds: Sequence[torch.Tensor], device="cuda") -> torch.Tensor:
    desc, count = update_tensors(ws, ds)
    return torch.empty(max(int(_lib.load().nc_swamp_workspace_bytes(desc, count)), 16), dtype=torch.uint8,
                       device=device)


def nc_swamp_watch(ws: Sequence[torch.Tensor], ds: Sequence[torch.Tensor], wfmt, out: torch.Tensor,
                   flags: Optional[Sequence[Optional[torch.Tensor]]] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None):
    _need(out, "out", torch.int64, len(ws), 5)
    _need(workspace, "workspace", torch.uint8, 0)
    desc, count = update_tensors(ws, ds, flags)
    lib = _lib.load()
    if workspace is None:
        workspace = new_swamp_workspace(ws, ds)
    f = WFMT[wfmt] if isinstance(wfmt, str) else wfmt
    _check(lib.nc_swamp_watch(desc, count, f, _ptr(out), _ptr(workspace), workspace.numel(), _stream(stream)),
           "nc_swamp_watch")


def nc_swamp_window(pol: NcSwampPolicy, st: torch.Tensor, in_counts: torch.Tensor, stream=None):
    _need(st, "st", torch.int32, st.shape[0], 4)
    _need(in_counts, "in_counts", torch.int64, st.shape[0], 5)
    _check(_lib.load().nc_swamp_window(ctypes.byref(pol), st.shape[0], _ptr(st), _ptr(in_counts),
                                       _stream(stream)), "nc_swamp_window")
