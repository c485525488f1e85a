"""Seeded synthetic inputs for the activation-sparse ReLU-gated FFN.

This module only draws numbers. It holds none of the layer's arithmetic, so
both the HIP path and the CPU oracle can consume what it produces.

The pages ("Sparser, Faster, Lighter Transformer Language Models", summary on
gist.science, section 4) measure trained 0.5B-2B gated Transformer++ models on
FineWeb. Neither the data nor the weights are available, so these generators
stand in for them with the same layer shapes and a controlled gate density:

* ``x ~ N(0, 1)`` with ``x[:, 0] = 1``; ``W_g, W_u ~ N(0, 1/d_model)``;
  ``W_d ~ N(0, 1/d_ff)`` (fan-in scaling).
* Column 0 of the gate weights (the weight that multiplies ``x[:, 0] = 1``) is
  set to ``Phi^-1(rho)``, an offset that leaves every gate pre-activation with
  probability about ``rho`` of being positive (section 2.A of the summary page
  reports more than 99% exact zeros after ReLU + L1 training).
* A skewed variant moves a seeded 5% of the rows to a higher density by
  scaling ``x[t, 0]``; this imitates the token-dependent activity that
  section 4 of the summary page describes (informative tokens fire more
  neurons) and is what the hybrid ELL + dense-backup layout is for.

Every array is drawn in float64 from ``numpy.random.default_rng([seed,
stream])`` with a fixed stream per tensor, scaled, rounded to float32 and then
(round-to-nearest-even, by torch) to the storage dtype.

Storage layouts (row-major), one contiguous ``d_model`` vector per neuron:
``x, dy: [T][d_model]``; ``wg_t, wu_t, wd: [d_ff][d_model]`` where row ``i``
of ``wg_t`` / ``wu_t`` is column ``i`` of ``W_g`` / ``W_u`` and row ``i`` of
``wd`` is row ``i`` of ``W_d``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch
from scipy.special import ndtri

STREAM_WG, STREAM_WU, STREAM_WD, STREAM_X, STREAM_DY, STREAM_PERM = range(6)

TILE_C = 128  # TwELL column-tile width used by every workload


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic layer configuration."""

    name: str
    T: int
    d_model: int
    d_ff: int
    dtype: str  # "f32" or "bf16"
    density: float
    skew_frac: float = 0.0  # fraction of rows moved to ``skew_density``
    skew_density: float = 0.0
    K: int = 128  # hybrid ELL width cap
    max_ovf: int = 1024  # hybrid dense-backup capacity (rows)
    width: int = TILE_C  # TwELL slots per (row, tile)

    @property
    def n_tiles(self) -> int:
        return self.d_ff // TILE_C

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workload families (model-scale shapes of the summary page, section 4).
TINY_F32 = Workload("tiny-fp32", 64, 256, 1024, "f32", 0.02)
SCALE_0P5B = Workload("0.5b-fwd-1pct", 4096, 1024, 2816, "bf16", 0.01, width=32)
SCALE_1P5B = Workload("1.5b-fwd", 8192, 2048, 5632, "bf16", 0.01, width=32)
SWEEP_1P5B = (0.005, 0.01, 0.02, 0.05, 0.20)
DECODE_2B = Workload("2b-decode", 1, 2304, 6144, "bf16", 0.01, width=32)
DECODE_T = (1, 8, 32, 64)
TRAIN_1P5B = Workload("1.5b-train-skewed", 8192, 2048, 5632, "bf16", 0.01,
                      skew_frac=0.05, skew_density=0.30, K=128, max_ovf=1024,
                      width=TILE_C)


def sweep_workload(density: float) -> Workload:
    """The 1.5B forward at one sweep density. TwELL width 32 up to 5% (at most
    about 6.4 expected nonzeros per 128-column tile) and 64 at 20% (about 26)."""
    return SCALE_1P5B.with_(density=density, width=32 if density <= 0.05 else 64)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _round_scalar(v: float, dtype: str) -> float:
    return float(_store(np.array([v]), dtype)[0].float())


def make_inputs(w: Workload, seed: int = 0, with_dy: bool = False) -> dict:
    """Gaussian inputs of workload ``w``; returns CPU tensors in storage dtype.

    Keys: ``x, wg_t, wu_t, wd`` (and ``dy`` if asked), plus ``skew_rows`` (the
    seeded rows whose density is raised, possibly empty).
    """
    T, dm, dff = w.T, w.d_model, w.d_ff
    off = _round_scalar(float(ndtri(w.density)), w.dtype)
    wg = _rng(seed, STREAM_WG).standard_normal((dff, dm)) / math.sqrt(dm)
    wg[:, 0] = off
    wu = _rng(seed, STREAM_WU).standard_normal((dff, dm)) / math.sqrt(dm)
    wd = _rng(seed, STREAM_WD).standard_normal((dff, dm)) / math.sqrt(dff)
    x = _rng(seed, STREAM_X).standard_normal((T, dm))
    x[:, 0] = 1.0
    skew_rows = np.zeros(0, dtype=np.int64)
    if w.skew_frac > 0.0:
        n_skew = int(round(w.skew_frac * T))
        skew_rows = np.sort(_rng(seed, STREAM_PERM).permutation(T)[:n_skew])
        x[skew_rows, 0] = _round_scalar(float(ndtri(w.skew_density)) / off, w.dtype)
    out = {"x": _store(x, w.dtype), "wg_t": _store(wg, w.dtype),
           "wu_t": _store(wu, w.dtype), "wd": _store(wd, w.dtype),
           "skew_rows": torch.from_numpy(skew_rows)}
    if with_dy:
        out["dy"] = _store(_rng(seed, STREAM_DY).standard_normal((T, dm)), w.dtype)
    return out


def make_integer_inputs(T: int, d_model: int, d_ff: int, dtype: str, density: float,
                        seed: int = 0, with_dy: bool = False,
                        skew_rows: int = 0) -> dict:
    """Inputs whose entries are small integers in {-1, 0, 1}.

    Every product and partial sum of the layer is then an integer small enough
    to be exact in float32 accumulation, so the GPU path and the oracle must
    agree bit for bit, including exact ``g == 0`` ties at the ReLU.
    ``x[:, 0] = 1`` and ``wg_t[:, 0] = -c`` with ``c`` chosen so about
    ``density`` of the gates are positive. ``skew_rows`` seeded rows get
    ``x[t, 0] = 0`` instead, which removes the offset and raises their density
    to about one half (dense-backup rows for the hybrid layout).
    """
    std = math.sqrt((d_model - 1) * 4.0 / 9.0)
    c = int(round(-float(ndtri(density)) * std))
    wg = _rng(seed, STREAM_WG).integers(-1, 2, (d_ff, d_model)).astype(np.float64)
    wg[:, 0] = -c
    wu = _rng(seed, STREAM_WU).integers(-1, 2, (d_ff, d_model)).astype(np.float64)
    wd = _rng(seed, STREAM_WD).integers(-1, 2, (d_ff, d_model)).astype(np.float64)
    x = _rng(seed, STREAM_X).integers(-1, 2, (T, d_model)).astype(np.float64)
    x[:, 0] = 1.0
    rows = np.zeros(0, dtype=np.int64)
    if skew_rows > 0:
        rows = np.sort(_rng(seed, STREAM_PERM).permutation(T)[:skew_rows])
        x[rows, 0] = 0.0
    out = {"x": _store(x, dtype), "wg_t": _store(wg, dtype), "wu_t": _store(wu, dtype),
           "wd": _store(wd, dtype), "skew_rows": torch.from_numpy(rows)}
    if with_dy:
        out["dy"] = _store(_rng(seed, STREAM_DY).integers(-1, 2, (T, d_model)), dtype)
    return out
