"""Pins of the comparison rules in helpers.py (CPU only).

The fp32 rule bounds each element by 1e-5 * (|ref| + mag), mag being the sum
of the absolute values of the products that make up the element. These tests
show that the rule catches what the earlier array-wide rule (1e-5 times the
largest |ref| of the array) let through, and pin the mag helpers against
brute-force sums of absolute terms.
"""
import numpy as np
import pytest

from activation_sparse_ffn_gemm_amd import synth
from helpers import (BAND, assert_close, bwd_hybrid_mag, f64, ffn_hybrid_mag, ffn_twell_mag,
                     forward_e2e_bounds, gate_mag, oracle_twell_for_gpu, tolerance)


def old_rule_ok(gpu, ref):
    """The array-wide rule the element-wise one replaces."""
    return np.all(np.abs(gpu - ref) <= 1e-5 * np.abs(ref).max())


def test_planted_error_on_small_element_synthetic():
    """A 1e-4 error on an element of size 0.004 whose terms are all small:
    the array-wide rule accepts it (the array also holds 100), the
    element-wise rule rejects it."""
    ref = np.array([100.0, 0.004])
    mag = np.array([100.0, 0.01])
    gpu = ref + np.array([0.0, 1e-4])
    assert old_rule_ok(gpu, ref)
    with pytest.raises(AssertionError):
        assert_close(gpu, ref, "f32", "planted", mag=mag)
    assert_close(ref + np.array([5e-4, 1e-8]), ref, "f32", "rounding-sized", mag=mag)


def test_planted_error_on_oracle_output(orc):
    """On the tiny fp32 layer's y: an error of half the array-wide bound,
    planted on the element with the smallest terms, passes the old rule and
    fails the element-wise one; the unperturbed output passes."""
    w = synth.TINY_F32
    d = synth.make_inputs(w)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    tw_r, _ = oracle_twell_for_gpu(orc, g, 128, "f32", "cpu")
    y = orc.ffn_twell(f64(d["x"]), tw_r, f64(d["wu_t"]), f64(d["wd"]))
    mag = ffn_twell_mag(orc, d["x"], tw_r, d["wu_t"], d["wd"])
    assert np.all(mag >= np.abs(y) * (1 - 1e-12))
    i = np.unravel_index(np.argmin(np.abs(y) + mag), y.shape)
    planted = y.copy()
    planted[i] += 0.5 * 1e-5 * np.abs(y).max()
    assert old_rule_ok(planted, y)
    assert tolerance(y, "f32", mag)[i] < 0.5 * 1e-5 * np.abs(y).max()
    with pytest.raises(AssertionError):
        assert_close(planted, y, "f32", "y", mag=mag)
    assert_close(y, y, "f32", "y", mag=mag)


def test_fp32_rule_needs_mag():
    with pytest.raises(AssertionError):
        assert_close(np.zeros(3), np.zeros(3), "f32")


def _tiny(seed=3, T=5, dm=7, dff=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, dm))
    wg = rng.standard_normal((dff, dm))
    wg[:, 0] -= 1.0
    return x, wg, rng.standard_normal((dff, dm)), rng.standard_normal((dff, dm)), \
        rng.standard_normal((T, dm))


def test_gate_mag_brute_force(orc):
    x, wg, _, _, _ = _tiny()
    want = np.array([[sum(abs(x[t, k] * wg[i, k]) for k in range(x.shape[1]))
                      for i in range(wg.shape[0])] for t in range(x.shape[0])])
    assert np.allclose(gate_mag(orc, x, wg), want, rtol=1e-14, atol=0)


def test_forward_mags_brute_force(orc):
    """ffn_twell_mag and ffn_hybrid_mag equal sum_i |h_i| (sum_k |x_k wu_ik|)
    |wd_ij| written out with numpy."""
    x, wg, wu, wd, _ = _tiny()
    g = orc.gate(x, wg)
    h = np.where(g > 0, g, 0.0)
    want = np.einsum("ti,ti,ij->tj", np.abs(h), np.abs(x) @ np.abs(wu).T, np.abs(wd))
    tw = orc.twell_pack(g)
    assert np.allclose(ffn_twell_mag(orc, x, tw, wu, wd), want, rtol=1e-12, atol=0)
    nnz = (g > 0).sum(1)
    hy = orc.to_hybrid(tw, int(np.sort(nnz)[-2]), 4)  # some rows go to the backup
    assert hy["n_ovf"] >= 1
    assert np.allclose(ffn_hybrid_mag(orc, x, hy, wu, wd), want, rtol=1e-12, atol=0)


def test_backward_mags_brute_force(orc):
    """bwd_hybrid_mag equals the backward's sums of absolute terms written out
    with numpy: da = dy wd^T, du = da h, dg = da u + l1 on the pattern,
    dx = du wu + dg wg, dW_d = a^T dy, dW_u = du^T x, dW_g = dg^T x, every
    factor replaced by its absolute value (and every inner sum by its sum of
    absolute terms)."""
    x, wg, wu, wd, dy = _tiny()
    g = orc.gate(x, wg)
    P = g > 0
    A = np.abs
    hm = np.where(P, A(g), 0.0)
    um = A(x) @ A(wu).T
    dam = A(dy) @ A(wd).T
    l1 = 0.25
    a = hm * um
    du = np.where(P, dam * hm, 0.0)
    dg = np.where(P, dam * um + l1, 0.0)
    want = (du @ A(wu) + dg @ A(wg), dg.T @ A(x), du.T @ A(x), a.T @ A(dy))
    tw = orc.twell_pack(g)
    hy = orc.to_hybrid(tw, 128, 8)
    got = bwd_hybrid_mag(orc, x, dy, hy, wg, wu, wd, l1=l1)
    for a_, b_ in zip(got, want):
        assert np.allclose(a_, b_, rtol=1e-12, atol=1e-300)


def test_forward_e2e_bounds(orc):
    """The end-to-end bound covers h by its gate's sum of absolute terms, and
    its band allowance is zero on rows with no pre-activation in the band."""
    w = synth.TINY_F32
    d = synth.make_inputs(w)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    tw_r, _ = oracle_twell_for_gpu(orc, g, 128, "f32", "cpu")
    mag, extra = forward_e2e_bounds(orc, d["x"], d["wg_t"], d["wu_t"], d["wd"], 128)
    base = ffn_twell_mag(orc, d["x"], tw_r, d["wu_t"], d["wd"])
    assert np.all(mag >= base)
    in_band = (np.abs(g) < BAND).any(1)
    assert in_band.any() and not in_band.all()
    assert np.all(extra[~in_band] == 0.0) and np.all(extra[in_band].max(1) > 0)
