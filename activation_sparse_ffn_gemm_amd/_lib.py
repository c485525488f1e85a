"""ctypes binding of libtwell.so: argument marshalling only.

Torch tensors supply device memory (``data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``); every step of the layer runs in
the library's HIP kernels. There is no fallback: if the library is missing
the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtwell.so")

TWELL_F32, TWELL_BF16 = 0, 1
TILE_C = 128
DEV_TILE_OVERFLOW, DEV_OVF_CAPACITY, DEV_BAD_INDEX = 1, 2, 4

# every extern "C" symbol include/twell.h declares
EXPORTS = ("twell_gate_pack", "twell_gate_workspace_bytes", "twell_ffn_fwd", "twell_fwd_workspace_bytes", "twell_decode_fwd",
           "twell_decode_workspace_bytes", "twell_to_hybrid", "hybrid_ffn_fwd",
           "hybrid_fwd_workspace_bytes", "hybrid_ffn_bwd", "hybrid_bwd_workspace_bytes",
           "twell_status_str", "twell_decode_fwd_noalloc")
STATIC_SCRATCH_BYTES = 12 << 20  # twell_decode_fwd_noalloc's scratch per GPU
DECODE_T = 64  # most tokens twell_decode_fwd takes (few-token kernels up to here)

c_i32, c_sz, c_p = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p


class TwellC(ctypes.Structure):
    _fields_ = [("T", c_i32), ("d_ff", c_i32), ("width", c_i32), ("dtype", ctypes.c_int),
                ("count", c_p), ("col", c_p), ("val", c_p)]


TIMING_MAX = 24


class TimingC(ctypes.Structure):
    _fields_ = [("events", c_p * (TIMING_MAX + 1)), ("n_events", c_i32), ("n_used", c_i32),
                ("names", ctypes.c_char_p * TIMING_MAX)]


class KernelTimer:
    """Per-kernel HIP-event timing of library calls on the current stream.

    ``timer.arg()`` gives the struct to pass to one call; after the stream is
    synchronised, ``timer.collect()`` returns [(kernel name, ms), ...] of the
    last call and ``timer.add(totals)`` accumulates them into a dict.
    """

    def __init__(self):
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(TIMING_MAX + 1)]
        for e in self.ev:  # materialise the underlying events
            e.record()
        torch.cuda.synchronize()
        self.c = TimingC()
        for k, e in enumerate(self.ev):
            self.c.events[k] = e.cuda_event
        self.c.n_events = TIMING_MAX + 1

    def arg(self):
        return ctypes.byref(self.c)

    def collect(self):
        out = []
        for k in range(self.c.n_used - 1):
            out.append((self.c.names[k].decode(), self.ev[k].elapsed_time(self.ev[k + 1])))
        return out

    def add(self, totals: dict):
        for name, ms in self.collect():
            totals[name] = totals.get(name, 0.0) + ms


class HybridC(ctypes.Structure):
    _fields_ = [("T", c_i32), ("d_ff", c_i32), ("K", c_i32), ("max_ovf", c_i32),
                ("dtype", ctypes.c_int), ("row_nnz", c_p), ("row_slot", c_p), ("ell_col", c_p),
                ("ell_val", c_p), ("ovf_rows", c_p), ("dense", c_p), ("n_ovf", c_p)]


_lib = None


class TwellError(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libtwell.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise TwellError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                         "(the HIP library is the only implementation; there is no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, S = c_p, c_i32, c_sz
    L.twell_gate_pack.argtypes = [ctypes.c_int, P, P, I, I, ctypes.POINTER(TwellC), P, S, P, P,
                                  P]
    L.twell_gate_workspace_bytes.argtypes = [ctypes.c_int, I, I, I]
    L.twell_gate_workspace_bytes.restype = S
    L.twell_ffn_fwd.argtypes = [ctypes.c_int, P, ctypes.POINTER(TwellC), P, P, I, P, P, S, P, P,
                                P]
    L.twell_fwd_workspace_bytes.argtypes = [ctypes.c_int, I, I, I, I]
    L.twell_fwd_workspace_bytes.restype = S
    L.twell_decode_fwd.argtypes = [ctypes.c_int, P, P, P, P, I, ctypes.POINTER(TwellC), P, P,
                                   S, P, P, P]
    L.twell_decode_fwd_noalloc.argtypes = [ctypes.c_int, P, P, P, P, I,
                                           ctypes.POINTER(TwellC), P, P, P, P]
    L.twell_decode_workspace_bytes.argtypes = [ctypes.c_int, I, I, I, I]
    L.twell_decode_workspace_bytes.restype = S
    L.twell_to_hybrid.argtypes = [ctypes.POINTER(TwellC), ctypes.POINTER(HybridC), P, P, P]
    L.hybrid_ffn_bwd.argtypes = [ctypes.c_int, P, P, ctypes.POINTER(HybridC), P, P, P, I,
                                 ctypes.c_float, P, P, P, P, P, S, P, P, P]
    L.hybrid_ffn_fwd.argtypes = [ctypes.c_int, P, ctypes.POINTER(HybridC), P, P, I, P, P, S, P,
                                 P, P]
    L.hybrid_fwd_workspace_bytes.argtypes = [ctypes.c_int, I, I, I, I, I]
    L.hybrid_fwd_workspace_bytes.restype = S
    L.hybrid_bwd_workspace_bytes.argtypes = [ctypes.c_int, I, I, I, I, I]
    L.hybrid_bwd_workspace_bytes.restype = S
    L.twell_status_str.argtypes = [ctypes.c_int]
    L.twell_status_str.restype = ctypes.c_char_p
    for f in ("twell_gate_pack", "twell_ffn_fwd", "twell_decode_fwd", "twell_to_hybrid",
              "hybrid_ffn_fwd", "hybrid_ffn_bwd", "twell_decode_fwd_noalloc"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != 0:
        raise TwellError(f"{what}: {load().twell_status_str(rc).decode()} (status {rc})")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TWELL_BF16
    if t.dtype == torch.float32:
        return TWELL_F32
    raise TwellError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else c_p(t.data_ptr())


# ---- argument checks: the C-ABI sees only pointers, so every tensor's shape,
# dtype, layout and device is checked here, before any call reaches the GPU
def _req(t, name, shape, dtype, device=None):
    """t must be a contiguous tensor of `shape` and `dtype` (on `device` if
    given); raises TwellError otherwise."""
    if not isinstance(t, torch.Tensor):
        raise TwellError(f"{name}: expected a tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise TwellError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TwellError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise TwellError(f"{name}: must be contiguous (row-major), e.g. not a transposed view")
    if device is not None and t.device != torch.device(device):
        raise TwellError(f"{name}: on {t.device}, expected {device}")


def _ws_form(workspace):
    if workspace is not None and (not isinstance(workspace, torch.Tensor)
                                  or workspace.dtype != torch.uint8 or workspace.dim() != 1
                                  or not workspace.is_contiguous()):
        raise TwellError("workspace: expected a contiguous 1-D uint8 tensor")


def _on_gpu(*named):
    """Every given tensor lives on one GPU; returns that device. (The
    workspace's form is checked first: it is the one argument whose shape the
    other checks do not cover.)"""
    for name, t in named:
        if name == "workspace":
            _ws_form(t)
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise TwellError(f"{name}: on {t.device}; the library runs on the GPU only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise TwellError(f"{name}: on {t.device}, other arguments on {dev}")
    return dev


def _ws(workspace, need, device):
    """The caller's workspace, checked, or a new one of `need` bytes."""
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device) if need else None
    _ws_form(workspace)
    if workspace.numel() < need:
        raise TwellError(f"workspace: {workspace.numel()} bytes, need {need}")
    return workspace


def _status(status, device):
    if status is not None:
        _req(status, "status", (1,), torch.int32)
    return status


def _check_weights(d_ff, d_model, dtype, **w):
    for name, t in w.items():
        _req(t, name, (d_ff, d_model), dtype)


def _check_twell(tw, T, dtype):
    if not isinstance(tw, Twell):
        raise TwellError("expected a Twell")
    nt = tw.count.shape[1] if tw.count.dim() == 2 else -1
    if tw.count.dim() != 2 or tw.col.dim() != 3:
        raise TwellError("twell: count must be [T][d_ff/128], col/val [T][d_ff/128][width]")
    W = tw.col.shape[2]
    _req(tw.count, "twell.count", (T, nt), torch.int32)
    _req(tw.col, "twell.col", (T, nt, W), torch.int16)
    _req(tw.val, "twell.val", (T, nt, W), dtype)


def _check_hybrid(hy, T, dtype):
    if not isinstance(hy, Hybrid):
        raise TwellError("expected a Hybrid")
    if hy.ell_col.dim() != 2 or hy.dense.dim() != 2:
        raise TwellError("hybrid: ell_col/ell_val must be [T][K], dense [max_ovf][d_ff]")
    K, mo, dff = hy.ell_col.shape[1], hy.dense.shape[0], hy.dense.shape[1]
    _req(hy.row_nnz, "hybrid.row_nnz", (T,), torch.int32)
    _req(hy.row_slot, "hybrid.row_slot", (T,), torch.int32)
    _req(hy.ell_col, "hybrid.ell_col", (T, K), torch.int16)
    _req(hy.ell_val, "hybrid.ell_val", (T, K), dtype)
    _req(hy.ovf_rows, "hybrid.ovf_rows", (mo,), torch.int32)
    _req(hy.dense, "hybrid.dense", (mo, dff), dtype)
    _req(hy.n_ovf, "hybrid.n_ovf", (1,), torch.int32)


def _twell_tensors(tw):
    return [("twell.count", tw.count), ("twell.col", tw.col), ("twell.val", tw.val)]


def _hybrid_tensors(hy):
    return [("hybrid.row_nnz", hy.row_nnz), ("hybrid.row_slot", hy.row_slot),
            ("hybrid.ell_col", hy.ell_col), ("hybrid.ell_val", hy.ell_val),
            ("hybrid.ovf_rows", hy.ovf_rows), ("hybrid.dense", hy.dense),
            ("hybrid.n_ovf", hy.n_ovf)]


def _x2(x, name="x"):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise TwellError(f"{name}: expected a [T][d_model] tensor")
    _dt(x)
    return x.shape


def _stream(device) -> c_p:
    return c_p(torch.cuda.current_stream(device).cuda_stream)


@dataclass
class Twell:
    """TwELL arrays (device tensors) of h = ReLU(x W_g)."""

    count: torch.Tensor  # [T][d_ff/128] int32
    col: torch.Tensor    # [T][d_ff/128][width] int16
    val: torch.Tensor    # [T][d_ff/128][width] dtype

    @property
    def T(self):
        return self.count.shape[0]

    @property
    def d_ff(self):
        return self.count.shape[1] * TILE_C

    @property
    def width(self):
        return self.col.shape[2]

    def c(self) -> TwellC:
        return TwellC(self.T, self.d_ff, self.width, _dt(self.val), self.count.data_ptr(),
                      self.col.data_ptr(), self.val.data_ptr())


@dataclass
class Hybrid:
    """Hybrid ELL + dense-backup arrays (device tensors)."""

    row_nnz: torch.Tensor   # [T] int32
    row_slot: torch.Tensor  # [T] int32
    ell_col: torch.Tensor   # [T][K] int16
    ell_val: torch.Tensor   # [T][K] dtype
    ovf_rows: torch.Tensor  # [max_ovf] int32
    dense: torch.Tensor     # [max_ovf][d_ff] dtype
    n_ovf: torch.Tensor     # [1] int32

    @property
    def T(self):
        return self.row_nnz.shape[0]

    @property
    def K(self):
        return self.ell_col.shape[1]

    @property
    def max_ovf(self):
        return self.dense.shape[0]

    @property
    def d_ff(self):
        return self.dense.shape[1]

    def c(self) -> HybridC:
        return HybridC(self.T, self.d_ff, self.K, self.max_ovf, _dt(self.ell_val),
                       self.row_nnz.data_ptr(), self.row_slot.data_ptr(),
                       self.ell_col.data_ptr(), self.ell_val.data_ptr(),
                       self.ovf_rows.data_ptr(), self.dense.data_ptr(), self.n_ovf.data_ptr())


def empty_twell(T, d_ff, width, dtype, device) -> Twell:
    nt = d_ff // TILE_C
    return Twell(torch.empty((T, nt), dtype=torch.int32, device=device),
                 torch.empty((T, nt, width), dtype=torch.int16, device=device),
                 torch.empty((T, nt, width), dtype=dtype, device=device))


def empty_hybrid(T, d_ff, K, max_ovf, dtype, device) -> Hybrid:
    return Hybrid(torch.empty(T, dtype=torch.int32, device=device),
                  torch.empty(T, dtype=torch.int32, device=device),
                  torch.empty((T, K), dtype=torch.int16, device=device),
                  torch.empty((T, K), dtype=dtype, device=device),
                  torch.empty(max_ovf, dtype=torch.int32, device=device),
                  torch.empty((max_ovf, d_ff), dtype=dtype, device=device),
                  torch.zeros(1, dtype=torch.int32, device=device))


def _timing(t):
    return None if t is None else t.arg()


def gate_workspace_bytes(dtype, T, d_model, d_ff) -> int:
    return int(load().twell_gate_workspace_bytes(dtype, T, d_model, d_ff))


def gate_pack(x, wg_t, width=TILE_C, out: Twell | None = None, status=None,
              timing: KernelTimer | None = None, workspace=None) -> Twell:
    T, dm = _x2(x)
    _req(x, "x", (T, dm), x.dtype)
    if not isinstance(wg_t, torch.Tensor) or wg_t.dim() != 2:
        raise TwellError("wg_t: expected a [d_ff][d_model] tensor")
    d_ff = wg_t.shape[0]
    _req(wg_t, "wg_t", (d_ff, dm), x.dtype)
    if out is None:
        out = empty_twell(T, d_ff, width, x.dtype, x.device)
    _check_twell(out, T, x.dtype)
    if out.d_ff != d_ff:
        raise TwellError(f"out: d_ff {out.d_ff}, wg_t has {d_ff} rows")
    dev = _on_gpu(("x", x), ("wg_t", wg_t), *_twell_tensors(out), ("status", status),
                  ("workspace", workspace))
    _status(status, dev)
    need = gate_workspace_bytes(_dt(x), T, dm, d_ff)
    workspace = _ws(workspace, need, dev)
    nbytes = 0 if workspace is None else workspace.numel()
    c = out.c()
    _check(load().twell_gate_pack(_dt(x), _ptr(x), _ptr(wg_t), T, dm, ctypes.byref(c),
                                  _ptr(workspace), nbytes, _ptr(status), _timing(timing),
                                  _stream(x.device)), "twell_gate_pack")
    return out


def fwd_workspace_bytes(dtype, T, d_model, d_ff, width) -> int:
    return int(load().twell_fwd_workspace_bytes(dtype, T, d_model, d_ff, width))


def ffn_fwd(x, tw: Twell, wu_t, wd, y=None, workspace=None, status=None,
            timing: KernelTimer | None = None):
    T, dm = _x2(x)
    _req(x, "x", (T, dm), x.dtype)
    _check_twell(tw, T, x.dtype)
    _check_weights(tw.d_ff, dm, x.dtype, wu_t=wu_t, wd=wd)
    if y is None:
        y = torch.empty((T, dm), dtype=torch.float32, device=x.device)
    _req(y, "y", (T, dm), torch.float32)
    dev = _on_gpu(("x", x), *_twell_tensors(tw), ("wu_t", wu_t), ("wd", wd), ("y", y),
                  ("status", status), ("workspace", workspace))
    _status(status, dev)
    need = fwd_workspace_bytes(_dt(x), T, dm, tw.d_ff, tw.width)
    workspace = _ws(workspace, need, dev)
    nbytes = 0 if workspace is None else workspace.numel()
    c = tw.c()
    _check(load().twell_ffn_fwd(_dt(x), _ptr(x), ctypes.byref(c), _ptr(wu_t), _ptr(wd), dm,
                                _ptr(y), _ptr(workspace), nbytes, _ptr(status),
                                _timing(timing), _stream(x.device)), "twell_ffn_fwd")
    return y


def decode_workspace_bytes(dtype, T, d_model, d_ff, width) -> int:
    return int(load().twell_decode_workspace_bytes(dtype, T, d_model, d_ff, width))


def decode_fwd(x, wg_t, wu_t, wd, width=TILE_C, out: Twell | None = None, y=None,
               workspace=None, status=None, timing: KernelTimer | None = None):
    """The whole layer for T <= DECODE_T tokens in one call (three launches
    on the current stream); returns (TwELL of h, y float32)."""
    T, dm = _x2(x)
    _req(x, "x", (T, dm), x.dtype)
    if not isinstance(wg_t, torch.Tensor) or wg_t.dim() != 2:
        raise TwellError("wg_t: expected a [d_ff][d_model] tensor")
    d_ff = wg_t.shape[0]
    _check_weights(d_ff, dm, x.dtype, wg_t=wg_t, wu_t=wu_t, wd=wd)
    if T > DECODE_T:
        raise TwellError(f"decode_fwd takes at most {DECODE_T} tokens, got {T}")
    if out is None:
        out = empty_twell(T, d_ff, width, x.dtype, x.device)
    _check_twell(out, T, x.dtype)
    if out.d_ff != d_ff:
        raise TwellError(f"out: d_ff {out.d_ff}, wg_t has {d_ff} rows")
    if y is None:
        y = torch.empty((T, dm), dtype=torch.float32, device=x.device)
    _req(y, "y", (T, dm), torch.float32)
    dev = _on_gpu(("x", x), ("wg_t", wg_t), ("wu_t", wu_t), ("wd", wd), *_twell_tensors(out),
                  ("y", y), ("status", status), ("workspace", workspace))
    _status(status, dev)
    need = decode_workspace_bytes(_dt(x), T, dm, d_ff, out.width)
    workspace = _ws(workspace, need, dev)
    nbytes = 0 if workspace is None else workspace.numel()
    c = out.c()
    _check(load().twell_decode_fwd(_dt(x), _ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), dm,
                                   ctypes.byref(c), _ptr(y), _ptr(workspace), nbytes,
                                   _ptr(status), _timing(timing), _stream(x.device)),
           "twell_decode_fwd")
    return out, y


def decode_fwd_noalloc(x, wg_t, wu_t, wd, out: Twell, y, status=None,
                       timing: KernelTimer | None = None):
    """decode_fwd for callers that cannot allocate: the caller passes the
    outputs (out, y), the library's static per-GPU scratch replaces the
    workspace, and nothing is allocated. Overlapping calls on one GPU race."""
    T, dm = _x2(x)
    _req(x, "x", (T, dm), x.dtype)
    if not isinstance(wg_t, torch.Tensor) or wg_t.dim() != 2:
        raise TwellError("wg_t: expected a [d_ff][d_model] tensor")
    d_ff = wg_t.shape[0]
    _check_weights(d_ff, dm, x.dtype, wg_t=wg_t, wu_t=wu_t, wd=wd)
    if T > DECODE_T:
        raise TwellError(f"decode_fwd_noalloc takes at most {DECODE_T} tokens, got {T}")
    _check_twell(out, T, x.dtype)
    if out.d_ff != d_ff:
        raise TwellError(f"out: d_ff {out.d_ff}, wg_t has {d_ff} rows")
    _req(y, "y", (T, dm), torch.float32)
    dev = _on_gpu(("x", x), ("wg_t", wg_t), ("wu_t", wu_t), ("wd", wd), *_twell_tensors(out),
                  ("y", y), ("status", status))
    _status(status, dev)
    c = out.c()
    _check(load().twell_decode_fwd_noalloc(_dt(x), _ptr(x), _ptr(wg_t), _ptr(wu_t), _ptr(wd), dm,
                                           ctypes.byref(c), _ptr(y), _ptr(status),
                                           _timing(timing), _stream(x.device)),
           "twell_decode_fwd_noalloc")
    return out, y


def to_hybrid(tw: Twell, K, max_ovf, out: Hybrid | None = None, status=None,
              timing: KernelTimer | None = None) -> Hybrid:
    if not isinstance(tw, Twell):
        raise TwellError("expected a Twell")
    _check_twell(tw, tw.T, tw.val.dtype)
    _dt(tw.val)
    if out is None:
        out = empty_hybrid(tw.T, tw.d_ff, K, max_ovf, tw.val.dtype, tw.val.device)
    _check_hybrid(out, tw.T, tw.val.dtype)
    if (out.K, out.max_ovf, out.d_ff) != (K, max_ovf, tw.d_ff):
        raise TwellError(f"out: (K, max_ovf, d_ff) = {(out.K, out.max_ovf, out.d_ff)}, "
                         f"expected {(K, max_ovf, tw.d_ff)}")
    dev = _on_gpu(*_twell_tensors(tw), *_hybrid_tensors(out), ("status", status))
    _status(status, dev)
    ct, ch = tw.c(), out.c()
    _check(load().twell_to_hybrid(ctypes.byref(ct), ctypes.byref(ch), _ptr(status),
                                  _timing(timing), _stream(tw.val.device)), "twell_to_hybrid")
    return out


def hybrid_fwd_workspace_bytes(dtype, T, d_model, d_ff, K, max_ovf) -> int:
    return int(load().hybrid_fwd_workspace_bytes(dtype, T, d_model, d_ff, K, max_ovf))


def hybrid_fwd(x, hy: Hybrid, wu_t, wd, y=None, workspace=None, status=None,
               timing: KernelTimer | None = None):
    """Training forward over a hybrid; returns y (float32)."""
    T, dm = _x2(x)
    _req(x, "x", (T, dm), x.dtype)
    _check_hybrid(hy, T, x.dtype)
    _check_weights(hy.d_ff, dm, x.dtype, wu_t=wu_t, wd=wd)
    if y is None:
        y = torch.empty((T, dm), dtype=torch.float32, device=x.device)
    _req(y, "y", (T, dm), torch.float32)
    dev = _on_gpu(("x", x), *_hybrid_tensors(hy), ("wu_t", wu_t), ("wd", wd), ("y", y),
                  ("status", status), ("workspace", workspace))
    _status(status, dev)
    need = hybrid_fwd_workspace_bytes(_dt(x), T, dm, hy.d_ff, hy.K, hy.max_ovf)
    workspace = _ws(workspace, need, dev)
    nbytes = 0 if workspace is None else workspace.numel()
    ch = hy.c()
    _check(load().hybrid_ffn_fwd(_dt(x), _ptr(x), ctypes.byref(ch), _ptr(wu_t), _ptr(wd), dm,
                                 _ptr(y), _ptr(workspace), nbytes, _ptr(status), _timing(timing),
                                 _stream(x.device)), "hybrid_ffn_fwd")
    return y


def bwd_workspace_bytes(dtype, T, d_model, d_ff, K, max_ovf) -> int:
    return int(load().hybrid_bwd_workspace_bytes(dtype, T, d_model, d_ff, K, max_ovf))


def ffn_bwd(x, dy, hy: Hybrid, wg_t, wu_t, wd, out=None, workspace=None, status=None,
            timing: KernelTimer | None = None, l1: float = 0.0):
    """Returns (dx, dwg_t, dwu_t, dwd), all float32; l1 weights an activation
    penalty l1 * sum(h) whose gradient is included."""
    T, dm = _x2(x)
    _req(x, "x", (T, dm), x.dtype)
    _req(dy, "dy", (T, dm), x.dtype)
    _check_hybrid(hy, T, x.dtype)
    d_ff = hy.d_ff
    _check_weights(d_ff, dm, x.dtype, wg_t=wg_t, wu_t=wu_t, wd=wd)
    if out is None:
        f = dict(dtype=torch.float32, device=x.device)
        out = (torch.empty((T, dm), **f), torch.empty((d_ff, dm), **f),
               torch.empty((d_ff, dm), **f), torch.empty((d_ff, dm), **f))
    if len(out) != 4:
        raise TwellError("out: expected (dx, dwg_t, dwu_t, dwd)")
    dx, dwg, dwu, dwd = out
    _req(dx, "dx", (T, dm), torch.float32)
    for name, t in (("dwg_t", dwg), ("dwu_t", dwu), ("dwd", dwd)):
        _req(t, name, (d_ff, dm), torch.float32)
    dev = _on_gpu(("x", x), ("dy", dy), *_hybrid_tensors(hy), ("wg_t", wg_t), ("wu_t", wu_t),
                  ("wd", wd), ("dx", dx), ("dwg_t", dwg), ("dwu_t", dwu), ("dwd", dwd),
                  ("status", status), ("workspace", workspace))
    _status(status, dev)
    need = bwd_workspace_bytes(_dt(x), T, dm, d_ff, hy.K, hy.max_ovf)
    workspace = _ws(workspace, need, dev)
    nbytes = 0 if workspace is None else workspace.numel()
    ch = hy.c()
    _check(load().hybrid_ffn_bwd(_dt(x), _ptr(x), _ptr(dy), ctypes.byref(ch), _ptr(wg_t),
                                 _ptr(wu_t), _ptr(wd), dm, float(l1), _ptr(dx), _ptr(dwg),
                                 _ptr(dwu),
                                 _ptr(dwd), _ptr(workspace), nbytes, _ptr(status),
                                 _timing(timing), _stream(x.device)), "hybrid_ffn_bwd")
    return out
