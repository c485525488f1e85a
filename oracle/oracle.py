"""ctypes binding to the plain-C float64 oracle in ``twell_oracle.c``.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP path and does not import it. Inputs are float64 numpy arrays
(bf16 and fp32 storage values convert to float64 exactly); this file only
marshals them, every step of the arithmetic is in the C source, which cites
the passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "twell_oracle.c")
LIB = os.path.join(HERE, "libtwell_oracle.so")

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-Wall", "-o", tmp, SRC])
    os.replace(tmp, LIB)
    return LIB


def load(path: str) -> ctypes.CDLL:
    """Load an oracle build and make it the one this module calls."""
    global _lib
    L = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int
    L.orc_gate.argtypes = [P, P, I, I, I, P]
    L.orc_twell_pack.argtypes = [P, I, I, I, I, P, P, P]
    L.orc_ffn_dense.argtypes = [P, P, P, P, I, I, I, P]
    L.orc_ffn_twell.argtypes = [P, P, P, P, I, I, I, P, P, I, P]
    L.orc_to_hybrid.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, P]
    D = ctypes.c_double
    L.orc_ffn_hybrid.argtypes = [P, I, I, I, P, P, P, P, I, P, P, P, P]
    L.orc_bwd_hybrid.argtypes = [P, P, I, I, I, P, P, P, P, I, P, P, P, P, D, P, P, P, P]
    L.orc_bwd_dense.argtypes = [P, P, I, I, I, P, P, P, D, P, P, P, P]
    L.orc_num_threads.argtypes = []
    L.orc_set_num_threads.argtypes = [I]
    _lib = L
    return L


def lib() -> ctypes.CDLL:
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        load(LIB)
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (timing only; results do not
    depend on it)."""
    lib().orc_set_num_threads(int(n))


def gate(x, wg_t) -> np.ndarray:
    x, wg_t = _f64(x), _f64(wg_t)
    T, dm = x.shape
    dff = wg_t.shape[0]
    g = np.empty((T, dff))
    lib().orc_gate(_p(x), _p(wg_t), T, dm, dff, _p(g))
    return g


def twell_pack(g, tile_c: int = 128, W: int = 128) -> dict:
    g = _f64(g)
    T, dff = g.shape
    assert dff % tile_c == 0 and 1 <= W <= tile_c
    nt = dff // tile_c
    count = np.zeros((T, nt), np.int32)
    col = np.full((T, nt, W), -1, np.int32)
    val = np.zeros((T, nt, W))
    over = lib().orc_twell_pack(_p(g), T, dff, tile_c, W, _p(count), _p(col), _p(val))
    return {"count": count, "col": col, "val": val, "overflow": bool(over),
            "tile_c": tile_c, "W": W, "d_ff": dff}


def ffn_dense(x, wg_t, wu_t, wd) -> np.ndarray:
    x, wg_t, wu_t, wd = map(_f64, (x, wg_t, wu_t, wd))
    T, dm = x.shape
    y = np.empty((T, dm))
    lib().orc_ffn_dense(_p(x), _p(wg_t), _p(wu_t), _p(wd), T, dm, wg_t.shape[0], _p(y))
    return y


def ffn_twell(x, tw: dict, wu_t, wd) -> np.ndarray:
    x, wu_t, wd = map(_f64, (x, wu_t, wd))
    count, col, val = _i32(tw["count"]), _i32(tw["col"]), _f64(tw["val"])
    T, dm = x.shape
    nt, W = count.shape[1], col.shape[2]
    y = np.empty((T, dm))
    lib().orc_ffn_twell(_p(x), _p(count), _p(col), _p(val), T, nt, W, _p(wu_t), _p(wd), dm, _p(y))
    return y


def to_hybrid(tw: dict, K: int, max_ovf: int) -> dict:
    count, col, val = _i32(tw["count"]), _i32(tw["col"]), _f64(tw["val"])
    T, nt = count.shape
    W = col.shape[2]
    dff = tw["d_ff"]
    row_nnz = np.zeros(T, np.int32)
    row_slot = np.zeros(T, np.int32)
    ell_col = np.full((T, K), -1, np.int32)
    ell_val = np.zeros((T, K))
    ovf_rows = np.full(max(max_ovf, 1), -1, np.int32)
    dense = np.zeros((max(max_ovf, 1), dff))
    n_ovf = np.zeros(1, np.int32)
    cap = lib().orc_to_hybrid(_p(count), _p(col), _p(val), T, nt, W, dff, K, max_ovf,
                              _p(row_nnz), _p(row_slot), _p(ell_col), _p(ell_val),
                              _p(ovf_rows), _p(dense), _p(n_ovf))
    return {"row_nnz": row_nnz, "row_slot": row_slot, "ell_col": ell_col, "ell_val": ell_val,
            "ovf_rows": ovf_rows[:max_ovf], "dense": dense[:max_ovf], "n_ovf": int(n_ovf[0]),
            "capacity_exceeded": bool(cap), "K": K, "max_ovf": max_ovf, "d_ff": dff}


def ffn_hybrid(x, hy: dict, wu_t, wd):
    """Forward over a hybrid's entries (ELL rows and dense backup rows)."""
    x, wu_t, wd = map(_f64, (x, wu_t, wd))
    T, dm = x.shape
    dff = hy["d_ff"]
    row_nnz, row_slot, ell_col = _i32(hy["row_nnz"]), _i32(hy["row_slot"]), _i32(hy["ell_col"])
    ell_val = _f64(hy["ell_val"])
    dense = _f64(hy["dense"]) if hy["dense"].size else np.zeros((1, dff))
    assert not hy.get("capacity_exceeded", False)
    y = np.empty((T, dm))
    rc = lib().orc_ffn_hybrid(_p(x), T, dm, dff, _p(row_nnz), _p(row_slot), _p(ell_col),
                              _p(ell_val), hy["K"], _p(dense), _p(wu_t), _p(wd), _p(y))
    if rc:
        raise MemoryError("oracle forward ran out of memory")
    return y


def bwd_hybrid(x, dy, hy: dict, wg_t, wu_t, wd, l1: float = 0.0):
    """Backward on the hybrid's pattern, with the gradient of an activation
    penalty l1 * sum(h) added; returns (dx, dwg_t, dwu_t, dwd)."""
    x, dy, wg_t, wu_t, wd = map(_f64, (x, dy, wg_t, wu_t, wd))
    T, dm = x.shape
    dff = wg_t.shape[0]
    K = hy["K"]
    row_nnz, row_slot, ell_col = _i32(hy["row_nnz"]), _i32(hy["row_slot"]), _i32(hy["ell_col"])
    ell_val = _f64(hy["ell_val"])
    dense = _f64(hy["dense"]) if hy["dense"].size else np.zeros((1, dff))
    assert not hy.get("capacity_exceeded", False)
    dx = np.empty((T, dm))
    dwg, dwu, dwd = (np.empty((dff, dm)) for _ in range(3))
    rc = lib().orc_bwd_hybrid(_p(x), _p(dy), T, dm, dff, _p(row_nnz), _p(row_slot), _p(ell_col),
                              _p(ell_val), K, _p(dense), _p(wg_t), _p(wu_t), _p(wd),
                              float(l1), _p(dx), _p(dwg), _p(dwu), _p(dwd))
    if rc:
        raise MemoryError("oracle backward ran out of memory")
    return dx, dwg, dwu, dwd


def bwd_dense(x, dy, wg_t, wu_t, wd, l1: float = 0.0):
    """Dense backward of the layer (with the gradient of the activation
    penalty l1 * sum(ReLU(x W_g))); returns (dx, dwg_t, dwu_t, dwd)."""
    x, dy, wg_t, wu_t, wd = map(_f64, (x, dy, wg_t, wu_t, wd))
    T, dm = x.shape
    dff = wg_t.shape[0]
    dx = np.empty((T, dm))
    dwg, dwu, dwd = (np.empty((dff, dm)) for _ in range(3))
    rc = lib().orc_bwd_dense(_p(x), _p(dy), T, dm, dff, _p(wg_t), _p(wu_t), _p(wd), float(l1),
                             _p(dx), _p(dwg), _p(dwu), _p(dwd))
    if rc:
        raise MemoryError("oracle backward ran out of memory")
    return dx, dwg, dwu, dwd
