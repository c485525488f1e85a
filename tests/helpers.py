"""Shared test helpers: comparison rules and host-side decoding of the layouts.

Comparison rules (tolerances as fixed for this layer):
* TwELL pattern: per (row, tile) the GPU's and the oracle's column sets may
  differ only at columns whose oracle pre-activation has |g| < 1e-3; the
  count equals the size of the stored set; columns ascend inside a tile.
* bf16 inputs, fp32 accumulation: |gpu - ref| <= 2e-2 * (|ref| + 1e-2) for
  every element.
* fp32 inputs, "1e-5 relative", element by element against the size of the
  terms that make up each element:
      |gpu - ref| <= 1e-5 * (|ref| + mag)
  where mag is the sum of the absolute values of every product that enters
  the element (for g[t, i]: sum_k |x[t, k] wg_t[i, k]|; for y and the
  gradients the same sum taken through every level of the computation). A
  rounding error of fp32 accumulation is proportional to that sum, not to
  |ref|, which can cancel towards zero; an element whose terms are all small
  gets a small bound, whatever the rest of the array holds. mag is computed
  in float64 by the oracle itself run on the absolute values of the inputs:
  every output of the layer is a sum of products of inputs, so that run
  returns exactly the sum of the absolute terms.
* integer-valued inputs: bit-exact.

Padding: the layouts leave slots past a (row, tile)'s count, ELL slots past a
row's length and backup rows past n_ovf unspecified. Every upload here fills
them with NaN values and in-range columns or rows, so a kernel that used one
would turn its output into NaN or a wrong sum, not into a silent exact zero.
"""
from __future__ import annotations

import numpy as np
import torch

BAND = 1e-3
TOL = {"bf16": 2e-2, "f32": 1e-5}


def f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, np.float64)


def to_storage(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Round float64 values to the storage dtype (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float64))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def tolerance(ref, dtype: str, mag=None, extra=None) -> np.ndarray:
    """Per-element bound on |gpu - ref| (rules in the module docstring). mag:
    the elements' sums of absolute terms (required for fp32); extra: an
    allowance added for entries a test knows to be ambiguous."""
    ref = f64(ref)
    if dtype == "f32":
        assert mag is not None, "fp32 comparisons need the sums of absolute terms"
        mag = f64(mag)
        assert mag.shape == ref.shape
        tol = TOL[dtype] * (np.abs(ref) + mag)
    else:
        tol = TOL[dtype] * (np.abs(ref) + 1e-2)
    if extra is not None:
        tol = tol + f64(extra)
    return tol


def assert_close(gpu, ref, dtype: str, what: str = "", mag=None, extra=None):
    gpu, ref = f64(gpu), f64(ref)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    tol = tolerance(ref, dtype, mag, extra)
    err = np.abs(gpu - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r}")


def twell_dense(count, col, val, d_ff: int):
    """TwELL arrays (numpy) -> (values [T][d_ff], stored mask [T][d_ff])."""
    count, col, val = np.asarray(count), np.asarray(col).astype(np.int64), f64(val)
    T, nt, W = col.shape
    keep = np.arange(W)[None, None, :] < np.minimum(count, W)[:, :, None]
    rows = np.broadcast_to(np.arange(T)[:, None, None], col.shape)
    H = np.zeros((T, d_ff))
    M = np.zeros((T, d_ff), bool)
    assert np.all((col[keep] >= 0) & (col[keep] < d_ff))
    H[rows[keep], col[keep]] = val[keep]
    M[rows[keep], col[keep]] = True
    return H, M


def assert_twell_matches(tw_gpu, g_ref: np.ndarray, dtype: str, W: int, exact: bool = False,
                         g_mag=None):
    """GPU TwELL (torch tensors) against the oracle's pre-activations; g_mag:
    the gate's sums of absolute terms (gate_mag), needed for fp32 values."""
    count = tw_gpu.count.cpu().numpy()
    col = tw_gpu.col.cpu().numpy()
    val = tw_gpu.val.cpu()
    T, dff = g_ref.shape
    nt = dff // 128
    assert count.shape == (T, nt)
    n_store = np.minimum(count, W)
    H, M = twell_dense(count, col, val, dff)
    # stored columns lie in their tile and ascend
    c = col.astype(np.int64)
    keep = np.arange(W)[None, None, :] < n_store[:, :, None]
    tile_of = np.broadcast_to(np.arange(nt)[None, :, None], c.shape)
    assert np.all(c[keep] // 128 == tile_of[keep])
    asc = (np.diff(c, axis=2) > 0) | ~keep[:, :, 1:]
    assert np.all(asc), "columns not ascending inside a tile"
    Mref = g_ref > 0
    # count is the size of the g > 0 set the GPU saw (== stored set if lossless)
    if np.all(count <= W):
        assert np.array_equal(count, M.reshape(T, nt, 128).sum(2))
    diff = M ^ Mref
    if exact:
        assert not diff.any(), f"{diff.sum()} pattern mismatches"
        ref_vals = f64(to_storage(np.where(Mref, g_ref, 0.0), dtype))
        assert np.array_equal(H, ref_vals), "values differ"
    else:
        if diff.any():
            amb = np.abs(g_ref[diff])
            assert np.all(amb < BAND), f"pattern mismatch outside the ambiguity band: {amb.max()}"
        both = M & Mref
        assert_close(H[both], g_ref[both], dtype, "TwELL values",
                     mag=None if g_mag is None else f64(g_mag)[both])


def poison_cols(shape, d_ff: int, seed: int = 99) -> np.ndarray:
    """In-range column indices for padding slots (seeded)."""
    return np.random.default_rng(seed).integers(0, d_ff, shape)


def oracle_twell_for_gpu(orc, g_ref, W: int, dtype: str, device, poison: bool = True):
    """Oracle TwELL with values rounded to the storage dtype, as numpy and as
    device tensors (int32 counts, int16 columns). Padding slots (at or past
    min(count, W)) carry NaN values and in-range columns unless poison is
    False."""
    tw = orc.twell_pack(g_ref, W=W)
    tw_r = dict(tw)
    tw_r["val"] = f64(to_storage(tw["val"], dtype))
    T, nt = tw["count"].shape
    pad = np.arange(W)[None, None, :] >= np.minimum(tw["count"], W)[:, :, None]
    col = tw["col"].copy()
    val = tw_r["val"].copy()
    if poison:
        col[pad] = poison_cols(col.shape, nt * 128)[pad]
        val[pad] = np.nan
    else:
        col[pad] = 0
        val[pad] = 0.0
    dev = (torch.from_numpy(tw["count"]).to(device),
           torch.from_numpy(col.astype(np.int16)).to(device),
           to_storage(val, dtype).to(device))
    return tw_r, dev


def poisoned_twell(tw_mod, T: int, d_ff: int, W: int, dtype, device):
    """An empty TwELL for a GPU call to fill: counts 0, every slot NaN with an
    in-range column; the call must overwrite what it defines and nothing it
    leaves unspecified may matter downstream."""
    nt = d_ff // 128
    col = torch.from_numpy(poison_cols((T, nt, W), d_ff).astype(np.int16)).to(device)
    val = torch.full((T, nt, W), float("nan"), dtype=dtype, device=device)
    return tw_mod.Twell(torch.zeros((T, nt), dtype=torch.int32, device=device), col, val)


def poisoned_hybrid(tw_mod, T: int, d_ff: int, K: int, max_ovf: int, dtype, device):
    """An empty hybrid for twell_to_hybrid to fill, every unspecified part
    poisoned: ELL values NaN with in-range columns, backup rows NaN, backup
    row ids in range."""
    col = torch.from_numpy(poison_cols((T, K), d_ff, 98).astype(np.int16)).to(device)
    return tw_mod.Hybrid(
        torch.zeros(T, dtype=torch.int32, device=device),
        torch.zeros(T, dtype=torch.int32, device=device), col,
        torch.full((T, K), float("nan"), dtype=dtype, device=device),
        torch.from_numpy(np.random.default_rng(97).integers(0, max(T, 1), max_ovf)
                         .astype(np.int32)).to(device),
        torch.full((max_ovf, d_ff), float("nan"), dtype=dtype, device=device),
        torch.zeros(1, dtype=torch.int32, device=device))


# ---- sums of absolute terms (the fp32 rule's mag), from the oracle itself
def gate_mag(orc, x, wg_t) -> np.ndarray:
    """sum_k |x[t, k] wg_t[i, k]| for every (t, i)."""
    return orc.gate(np.abs(f64(x)), np.abs(f64(wg_t)))


def ffn_twell_mag(orc, x, tw: dict, wu_t, wd) -> np.ndarray:
    """The fused forward's sums of absolute terms over a TwELL's entries."""
    ta = dict(tw)
    ta["val"] = np.abs(f64(tw["val"]))
    return orc.ffn_twell(np.abs(f64(x)), ta, np.abs(f64(wu_t)), np.abs(f64(wd)))


def hybrid_abs(hy: dict) -> dict:
    ha = dict(hy)
    ha["ell_val"] = np.abs(f64(hy["ell_val"]))
    ha["dense"] = np.abs(f64(hy["dense"]))
    return ha


def ffn_hybrid_mag(orc, x, hy: dict, wu_t, wd) -> np.ndarray:
    return orc.ffn_hybrid(np.abs(f64(x)), hybrid_abs(hy), np.abs(f64(wu_t)), np.abs(f64(wd)))


def bwd_hybrid_mag(orc, x, dy, hy: dict, wg_t, wu_t, wd, l1: float = 0.0):
    """(dx, dwg_t, dwu_t, dwd) sums of absolute terms on a hybrid's pattern."""
    A = lambda a: np.abs(f64(a))
    return orc.bwd_hybrid(A(x), A(dy), hybrid_abs(hy), A(wg_t), A(wu_t), A(wd), l1=abs(l1))


def forward_e2e_bounds(orc, x, wg_t, wu_t, wd, W: int):
    """Bounds for y of the GPU's own gate + pack + forward against the oracle's
    forward over the oracle's TwELL (W slots). Returns (mag, extra):
      mag   the forward's sums of absolute terms with each stored h replaced
            by its gate's sum of absolute terms (which bounds h and the
            rounding of h on the GPU);
      extra for entries whose pre-activation lies in the |g| < 1e-3 band (the
            GPU may store them or not): sum over such entries of
            2e-3 * sum_k |x wu_t| * |wd|, what storing one can add."""
    g = orc.gate(f64(x), f64(wg_t))
    gm = gate_mag(orc, x, wg_t)
    tw = orc.twell_pack(g, W=W)
    tm = orc.twell_pack(np.where(g > 0, gm, 0.0), W=W)  # same pattern, val = mag
    mag = ffn_twell_mag(orc, x, tm, wu_t, wd)
    band = orc.twell_pack(np.where(np.abs(g) < BAND, 2 * BAND, 0.0), W=128)
    extra = ffn_twell_mag(orc, x, band, wu_t, wd)
    assert np.array_equal(tm["count"], tw["count"])
    return mag, extra


def hybrid_to_numpy(hy) -> dict:
    return {"row_nnz": hy.row_nnz.cpu().numpy(), "row_slot": hy.row_slot.cpu().numpy(),
            "ell_col": hy.ell_col.cpu().numpy().astype(np.int32), "ell_val": f64(hy.ell_val),
            "ovf_rows": hy.ovf_rows.cpu().numpy(), "dense": f64(hy.dense),
            "n_ovf": int(hy.n_ovf.cpu()[0]), "K": hy.K, "max_ovf": hy.max_ovf, "d_ff": hy.d_ff}


def assert_hybrid_equal(gpu: dict, ref: dict):
    """Exact comparison of the parts of a hybrid the layout defines."""
    assert gpu["n_ovf"] == ref["n_ovf"]
    assert np.array_equal(gpu["row_nnz"], ref["row_nnz"])
    assert np.array_equal(gpu["row_slot"], ref["row_slot"])
    K = ref["K"]
    for t in np.nonzero(ref["row_slot"] < 0)[0]:
        n = ref["row_nnz"][t]
        assert np.array_equal(gpu["ell_col"][t, :n], ref["ell_col"][t, :n]), t
        assert np.array_equal(gpu["ell_val"][t, :n], ref["ell_val"][t, :n]), t
    n = min(ref["n_ovf"], ref["max_ovf"])
    assert np.array_equal(gpu["ovf_rows"][:n], ref["ovf_rows"][:n])
    assert np.array_equal(gpu["dense"][:n], ref["dense"][:n])
    assert K == gpu["K"]
