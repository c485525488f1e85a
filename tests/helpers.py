"""Shared test helpers: comparison rules and host-side decoding of the layouts.

Comparison rules (tolerances as fixed for this layer):
* TwELL pattern: per (row, tile) the GPU's and the oracle's column sets may
  differ only at columns whose oracle pre-activation has |g| < 1e-3; the
  count equals the size of the stored set; columns ascend inside a tile.
* bf16 inputs, fp32 accumulation: |gpu - ref| <= 2e-2 * (|ref| + 1e-2) for
  every element.
* fp32 inputs, "1e-5 relative" read norm-wise over the compared array:
  max |gpu - ref| <= 1e-5 * max |ref|. An element-wise relative bound cannot
  hold in fp32: a d_model-term dot product accumulated in fp32 carries an
  absolute error near sqrt(d_model) * 2^-24 * |partial sums| (about 1e-6
  here), which exceeds 1e-5 * |ref| wherever the sum cancels towards zero.
* integer-valued inputs: bit-exact.
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


def assert_close(gpu, ref, dtype: str, what: str = ""):
    gpu, ref = f64(gpu), f64(ref)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if dtype == "f32":
        tol = np.full(ref.shape, TOL[dtype] * max(np.abs(ref).max(initial=0.0), 1e-30))
    else:
        tol = TOL[dtype] * (np.abs(ref) + 1e-2)
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


def assert_twell_matches(tw_gpu, g_ref: np.ndarray, dtype: str, W: int, exact: bool = False):
    """GPU TwELL (torch tensors) against the oracle's pre-activations."""
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
        assert_close(H[both], g_ref[both], dtype, "TwELL values")


def oracle_twell_for_gpu(orc, g_ref, W: int, dtype: str, device):
    """Oracle TwELL with values rounded to the storage dtype, as numpy and as
    device tensors (int32 counts, int16 columns)."""
    tw = orc.twell_pack(g_ref, W=W)
    val_s = to_storage(tw["val"], dtype)
    tw_r = dict(tw)
    tw_r["val"] = f64(val_s)
    col = np.where(tw["col"] < 0, 0, tw["col"]).astype(np.int16)
    dev = (torch.from_numpy(tw["count"]).to(device), torch.from_numpy(col).to(device),
           val_s.to(device))
    return tw_r, dev


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
