"""Pins for the CPU oracle: each check comes from outside the oracle itself.

* a hand-derived worked example (tests/golden/worked_example.json);
* library routines computing the same quantity by another route (torch
  float64 matmul for the forward, torch autograd for the backward);
* invariants the method fixes (dense and TwELL-sparse forward agree bit for
  bit, TwELL and the hybrid decode back to ReLU(x W_g), counts add up);
* central finite differences of the loss <y, dy>;
* brute force over every input row of a tiny layer, ties at g == 0 included;
* a closed form for the expected number of nonzeros of the Gaussian inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import ndtr

from activation_sparse_ffn_gemm_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def f64(t):
    return t.double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def storage(ex):
    """Math-layout weights of the worked example -> storage layouts."""
    Wg, Wu, Wd = (np.array(ex[k], np.float64) for k in ("W_g", "W_u", "W_d"))
    return np.array(ex["x"], np.float64), Wg.T.copy(), Wu.T.copy(), Wd.copy()


def torch_layer(x, wg_t, wu_t, wd, dy=None, l1=0.0):
    """Dense layer by torch (float64); returns y and, given dy, the gradients
    of sum(y * dy) + l1 * sum(ReLU(x W_g))."""
    X = torch.tensor(x, requires_grad=dy is not None)
    G = torch.tensor(wg_t, requires_grad=dy is not None)
    U = torch.tensor(wu_t, requires_grad=dy is not None)
    D = torch.tensor(wd, requires_grad=dy is not None)
    h = torch.relu(X @ G.T)
    y = (h * (X @ U.T)) @ D
    if dy is None:
        return y.detach().numpy()
    ((y * torch.tensor(dy)).sum() + l1 * h.sum()).backward()
    return y.detach().numpy(), X.grad.numpy(), G.grad.numpy(), U.grad.numpy(), D.grad.numpy()


def twell_to_dense(tw):
    T, nt = tw["count"].shape
    out = np.zeros((T, tw["d_ff"]))
    for t in range(T):
        for j in range(nt):
            for s in range(min(tw["count"][t, j], tw["W"])):
                out[t, tw["col"][t, j, s]] = tw["val"][t, j, s]
    return out


def hybrid_to_dense(hy, T):
    out = np.zeros((T, hy["d_ff"]))
    for t in range(T):
        if hy["row_slot"][t] < 0:
            n = hy["row_nnz"][t]
            out[t, hy["ell_col"][t, :n]] = hy["ell_val"][t, :n]
        else:
            out[t] = hy["dense"][hy["row_slot"][t]]
    return out


# ---------------------------------------------------------------- worked example
def test_worked_example_forward(orc):
    ex = json.load(open(GOLDEN))
    x, wg_t, wu_t, wd = storage(ex)
    g = orc.gate(x, wg_t)
    assert np.array_equal(g, np.array(ex["g"], np.float64))
    tw = orc.twell_pack(g, tile_c=2, W=2)
    ref = ex["twell_tile2"]
    assert np.array_equal(tw["count"], ref["count"])
    for t in range(2):
        for j in range(2):
            n = tw["count"][t, j]
            assert list(tw["col"][t, j, :n]) == ref["col"][t][j]
            assert list(tw["val"][t, j, :n]) == ref["val"][t][j]
    assert np.array_equal(twell_to_dense(tw), np.array(ex["h"], np.float64))
    y_ref = np.array(ex["y"], np.float64)
    assert np.array_equal(orc.ffn_dense(x, wg_t, wu_t, wd), y_ref)
    assert np.array_equal(orc.ffn_twell(x, tw, wu_t, wd), y_ref)
    # the same layer at the production tile width (one 128-column tile, zero padded)
    xp = np.zeros((2, 64)); xp[:, :2] = x
    pad = lambda w: np.pad(w, ((0, 124), (0, 62)))
    tw128 = orc.twell_pack(orc.gate(xp, pad(wg_t)), tile_c=128, W=128)
    assert tw128["count"].tolist() == [[2], [2]]
    assert tw128["col"][0, 0, :2].tolist() == [0, 2] and tw128["col"][1, 0, :2].tolist() == [1, 2]
    assert np.array_equal(orc.ffn_twell(xp, tw128, pad(wu_t), pad(wd))[:, :2], y_ref)


def test_worked_example_hybrid_and_backward(orc):
    ex = json.load(open(GOLDEN))
    x, wg_t, wu_t, wd = storage(ex)
    dy = np.array(ex["dy"], np.float64)
    tw = orc.twell_pack(orc.gate(x, wg_t), tile_c=2, W=2)
    h2 = orc.to_hybrid(tw, K=2, max_ovf=4)
    r = ex["hybrid_K2"]
    assert h2["row_nnz"].tolist() == r["row_nnz"] and h2["row_slot"].tolist() == r["row_slot"]
    assert h2["ell_col"].tolist() == r["ell_col"] and h2["ell_val"].tolist() == r["ell_val"]
    assert h2["n_ovf"] == r["n_ovf"]
    h1 = orc.to_hybrid(tw, K=1, max_ovf=4)
    r = ex["hybrid_K1"]
    assert h1["row_slot"].tolist() == r["row_slot"] and h1["n_ovf"] == r["n_ovf"]
    assert h1["ovf_rows"][:2].tolist() == r["ovf_rows"]
    assert h1["dense"][:2].tolist() == r["dense"]
    want = [np.array(ex[k], np.float64) for k in ("dx", "dW_g", "dW_u", "dW_d")]
    want[1], want[2] = want[1].T, want[2].T  # storage layouts of dW_g, dW_u
    for hy in (h2, h1):  # all-ELL and all-backup give the same gradients and y
        got = orc.bwd_hybrid(x, dy, hy, wg_t, wu_t, wd)
        for a, b in zip(got, want):
            assert np.array_equal(a, b)
        assert np.array_equal(orc.ffn_hybrid(x, hy, wu_t, wd), np.array(ex["y"], np.float64))
    for a, b in zip(orc.bwd_dense(x, dy, wg_t, wu_t, wd), want):
        assert np.array_equal(a, b)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("kind", ["gauss", "int"])
def test_dense_equals_twell_sparse_bitwise(orc, kind):
    """Skipped zeros contribute exactly 0, so the sums agree bit for bit."""
    if kind == "gauss":
        d = synth.make_inputs(synth.TINY_F32)
    else:
        d = synth.make_integer_inputs(64, 256, 1024, "f32", 0.02)
    x, wg_t, wu_t, wd = (f64(d[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    tw = orc.twell_pack(orc.gate(x, wg_t))
    assert not tw["overflow"]
    yd = orc.ffn_dense(x, wg_t, wu_t, wd)
    ys = orc.ffn_twell(x, tw, wu_t, wd)
    assert np.array_equal(yd, ys)


def test_twell_roundtrip_and_counts(orc):
    d = synth.make_inputs(synth.TINY_F32)
    x, wg_t = f64(d["x"]), f64(d["wg_t"])
    g = orc.gate(x, wg_t)
    g_lib = (torch.tensor(x) @ torch.tensor(wg_t).T).numpy()
    np.testing.assert_allclose(g, g_lib, rtol=0, atol=1e-12)
    tw = orc.twell_pack(g)
    assert np.array_equal(twell_to_dense(tw), np.maximum(g, 0.0))
    assert np.array_equal(tw["count"].sum(1), (g > 0).sum(1))
    # columns ascending inside every tile and inside the tile's range
    for t in range(g.shape[0]):
        for j in range(tw["count"].shape[1]):
            c = tw["col"][t, j, :tw["count"][t, j]]
            assert np.all(np.diff(c) > 0) and np.all(c // 128 == j)


def test_twell_width_cap(orc):
    """W below the count keeps the true count and the first W columns."""
    g = np.zeros((3, 256))
    g[0, [5, 9, 100, 127]] = [1.0, 2.0, 3.0, 4.0]
    g[1, 130] = 0.5
    g[2, 7] = -1.0
    g[2, 8] = 0.0
    g[2, 9] = -0.0
    g[2, 10] = np.nan
    tw = orc.twell_pack(g, W=2)
    assert tw["overflow"]
    assert tw["count"].tolist() == [[4, 0], [0, 1], [0, 0]]
    assert tw["col"][0, 0].tolist() == [5, 9] and tw["val"][0, 0].tolist() == [1.0, 2.0]
    assert tw["col"][1, 1, 0] == 130
    assert not orc.twell_pack(g, W=4)["overflow"]


def test_hybrid_invariants(orc):
    d = synth.make_integer_inputs(96, 128, 512, "f32", 0.03, skew_rows=9)
    x, wg_t = f64(d["x"]), f64(d["wg_t"])
    g = orc.gate(x, wg_t)
    tw = orc.twell_pack(g)
    nnz = (g > 0).sum(1)
    K = int(np.sort(nnz)[-12])  # some rows sit exactly at the cap
    hy = orc.to_hybrid(tw, K=K, max_ovf=32)
    assert np.array_equal(hy["row_nnz"], nnz)
    ovf = np.nonzero(nnz > K)[0]
    assert hy["n_ovf"] == len(ovf) and not hy["capacity_exceeded"]
    assert hy["ovf_rows"][:len(ovf)].tolist() == ovf.tolist()  # ascending rows
    assert np.all(hy["row_slot"][ovf] == np.arange(len(ovf)))
    assert np.all(hy["row_slot"][nnz <= K] == -1)
    assert np.any(nnz == K) and np.all(hy["row_slot"][nnz == K] == -1)  # tie stays ELL
    for t in np.nonzero(nnz <= K)[0]:
        assert np.all(np.diff(hy["ell_col"][t, :nnz[t]]) > 0)
    assert np.array_equal(hybrid_to_dense(hy, g.shape[0]), np.maximum(g, 0.0))
    small = orc.to_hybrid(tw, K=K, max_ovf=len(ovf) - 1)
    assert small["capacity_exceeded"] and small["n_ovf"] == len(ovf)


@pytest.mark.parametrize("kind", ["gauss", "int"])
def test_hybrid_forward_equals_twell_forward(orc, kind):
    """The hybrid-routed forward (ELL rows + dense backup rows) sums the same
    terms in the same order as the TwELL forward: bitwise equal."""
    if kind == "int":
        d = synth.make_integer_inputs(96, 128, 512, "f32", 0.03, skew_rows=9)
    else:
        d = synth.make_inputs(synth.Workload("t", 80, 96, 384, "f32", 0.05, skew_frac=0.1,
                                             skew_density=0.4))
    x, wg_t, wu_t, wd = (f64(d[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    tw = orc.twell_pack(orc.gate(x, wg_t))
    K = int(np.median(tw["count"].sum(1)))
    hy = orc.to_hybrid(tw, K=K, max_ovf=64)
    assert 0 < hy["n_ovf"] < 64
    assert np.array_equal(orc.ffn_hybrid(x, hy, wu_t, wd), orc.ffn_twell(x, tw, wu_t, wd))


# ---------------------------------------------------------------- library routines
def test_forward_matches_torch(orc):
    d = synth.make_inputs(synth.TINY_F32)
    x, wg_t, wu_t, wd = (f64(d[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    y = orc.ffn_twell(x, orc.twell_pack(orc.gate(x, wg_t)), wu_t, wd)
    np.testing.assert_allclose(y, torch_layer(x, wg_t, wu_t, wd), rtol=1e-10, atol=1e-12)


def test_forward_matches_torch_row_subset_0p5b(orc):
    """Rows are independent: 48 rows of the 0.5B-scale inputs check exactly."""
    d = synth.make_inputs(synth.SCALE_0P5B)
    x = f64(d["x"][:48])
    wg_t, wu_t, wd = (f64(d[k]) for k in ("wg_t", "wu_t", "wd"))
    y = orc.ffn_twell(x, orc.twell_pack(orc.gate(x, wg_t), W=128), wu_t, wd)
    np.testing.assert_allclose(y, torch_layer(x, wg_t, wu_t, wd), rtol=1e-9, atol=1e-11)


def test_hybrid_forward_matches_torch(orc):
    d = synth.make_inputs(synth.Workload("t", 40, 64, 256, "f32", 0.08, skew_frac=0.125,
                                         skew_density=0.5))
    x, wg_t, wu_t, wd = (f64(d[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    tw = orc.twell_pack(orc.gate(x, wg_t))
    hy = orc.to_hybrid(tw, K=int(np.median(tw["count"].sum(1))), max_ovf=40)
    assert hy["n_ovf"] > 0
    np.testing.assert_allclose(orc.ffn_hybrid(x, hy, wu_t, wd), torch_layer(x, wg_t, wu_t, wd),
                               rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("skew,l1", [(0, 0.0), (5, 0.0), (5, 0.375)])
def test_backward_matches_autograd(orc, skew, l1):
    d = synth.make_inputs(synth.Workload("t", 40, 64, 256, "f32", 0.08), with_dy=True)
    if skew:
        d = synth.make_inputs(synth.Workload("t", 40, 64, 256, "f32", 0.08, skew_frac=0.125,
                                             skew_density=0.5), with_dy=True)
    x, wg_t, wu_t, wd, dy = (f64(d[k]) for k in ("x", "wg_t", "wu_t", "wd", "dy"))
    tw = orc.twell_pack(orc.gate(x, wg_t))
    nnz = tw["count"].sum(1)
    K = int(np.median(nnz))
    hy = orc.to_hybrid(tw, K=K, max_ovf=40)
    assert 0 < hy["n_ovf"] < 40
    _, gx, gg, gu, gd = torch_layer(x, wg_t, wu_t, wd, dy, l1=l1)
    got = orc.bwd_hybrid(x, dy, hy, wg_t, wu_t, wd, l1=l1)
    for a, b in zip(got, (gx, gg, gu, gd)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    # the dense formulas agree with the sparse ones bit for bit (zeros are exact)
    for a, b in zip(orc.bwd_dense(x, dy, wg_t, wu_t, wd, l1=l1), got):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("l1", [0.0, 0.25])
def test_backward_finite_differences(orc, l1):
    """Central differences of sum(y * dy) + l1 * sum(ReLU(x W_g))."""
    rng = np.random.default_rng(7)
    T, dm, dff = 3, 4, 128
    x = rng.standard_normal((T, dm))
    wg_t, wu_t, wd = (rng.standard_normal((dff, dm)) for _ in range(3))
    dy = rng.standard_normal((T, dm))
    g = orc.gate(x, wg_t)
    assert np.abs(g).min() > 1e-3  # no gate within reach of the kink

    def loss(x_, wg_, wu_, wd_):
        penalty = float(np.maximum(x_ @ wg_.T, 0.0).sum())
        return float((orc.ffn_dense(x_, wg_, wu_, wd_) * dy).sum()) + l1 * penalty

    hy = orc.to_hybrid(orc.twell_pack(g), K=128, max_ovf=1)
    grads = orc.bwd_hybrid(x, dy, hy, wg_t, wu_t, wd, l1=l1)
    params = [x, wg_t, wu_t, wd]
    eps = 1e-6
    for p_idx, grad in enumerate(grads):
        for idx in [(0, 0), (1, 2), (2, 3)]:
            up = [p.copy() for p in params]
            dn = [p.copy() for p in params]
            up[p_idx][idx] += eps
            dn[p_idx][idx] -= eps
            fd = (loss(*up) - loss(*dn)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * (1 + abs(fd)), (p_idx, idx, fd, grad[idx])


def test_brute_force_tiny_layer(orc):
    """Every row of {-1,0,1}^3 through a 3 -> 128 layer: ties at g == 0 included.

    All values are small integers, so torch's float64 results are exact and
    must match bit for bit, forward and backward (ReLU'(0) = 0 in both).
    """
    rows = np.array(np.meshgrid([-1, 0, 1], [-1, 0, 1], [-1, 0, 1], indexing="ij"),
                    np.float64).reshape(3, -1).T
    rng = np.random.default_rng(3)
    wg_t, wu_t, wd = (rng.integers(-2, 3, (128, 3)).astype(np.float64) for _ in range(3))
    dy = rng.integers(-2, 3, rows.shape).astype(np.float64)
    g = orc.gate(rows, wg_t)
    assert np.sum(g == 0) > 100  # plenty of exact ties
    tw = orc.twell_pack(g)
    y_t, gx, gg, gu, gd = torch_layer(rows, wg_t, wu_t, wd, dy)
    assert np.array_equal(orc.ffn_twell(rows, tw, wu_t, wd), y_t)
    for K in (2, 128):
        hy = orc.to_hybrid(tw, K=K, max_ovf=27)
        for a, b in zip(orc.bwd_hybrid(rows, dy, hy, wg_t, wu_t, wd), (gx, gg, gu, gd)):
            assert np.array_equal(a, b)


# ---------------------------------------------------------------- closed form
@pytest.mark.parametrize("w", [synth.TINY_F32, synth.SCALE_0P5B.with_(T=512)])
def test_expected_nnz_closed_form(orc, w):
    """Given W_g, g[t,i] ~ N(x[t,0] W_g[0,i], sum_{k>0} W_g[k,i]^2), so
    E[nnz] = sum_{t,i} Phi(x[t,0] W_g[0,i] / sigma_i)."""
    d = synth.make_inputs(w)
    x, wg_t = f64(d["x"]), f64(d["wg_t"])
    tw = orc.twell_pack(orc.gate(x, wg_t), W=128)
    nnz = int(tw["count"].sum())
    sigma = np.sqrt((wg_t[:, 1:] ** 2).sum(1))
    e = float(ndtr(np.outer(x[:, 0], wg_t[:, 0]) / sigma[None, :]).sum())
    assert abs(nnz - e) <= 6 * math.sqrt(e), (nnz, e)
    assert abs(nnz / (w.T * w.d_ff) - w.density) < 0.25 * w.density


def test_skewed_rows_density(orc):
    w = synth.TRAIN_1P5B.with_(T=400, d_model=256, d_ff=1024)
    d = synth.make_inputs(w)
    x, wg_t = f64(d["x"]), f64(d["wg_t"])
    nnz = orc.twell_pack(orc.gate(x, wg_t))["count"].sum(1)
    rows = d["skew_rows"].numpy()
    assert len(rows) == 20
    hot = nnz[rows].mean() / 1024
    cold = np.delete(nnz, rows).mean() / 1024
    assert abs(hot - 0.30) < 0.03 and abs(cold - 0.01) < 0.004
