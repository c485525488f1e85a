"""GPU parity of twell_gate_pack, twell_ffn_fwd and twell_to_hybrid against the
oracle, through the C-ABI. Inputs flow one way only: oracle -> GPU."""
import numpy as np
import pytest
import torch

from activation_sparse_ffn_gemm_amd import _lib as tw
from activation_sparse_ffn_gemm_amd import synth
from helpers import (assert_close, assert_hybrid_equal, assert_twell_matches, f64,
                     ffn_twell_mag, forward_e2e_bounds, gate_mag, hybrid_to_numpy,
                     oracle_twell_for_gpu, poisoned_hybrid, poisoned_twell, to_storage)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(*a):
    print("[case]", *a, flush=True)


def upload(d, keys=("x", "wg_t", "wu_t", "wd")):
    return [d[k].to(DEV) for k in keys]


def status_word():
    return torch.zeros(1, dtype=torch.int32, device=DEV)


# ------------------------------------------------------------ gate + TwELL
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,dm,dff", [(1, 64, 128), (33, 192, 640), (64, 4096, 256),
                                      (65, 128, 384), (200, 256, 384), (333, 512, 1024),
                                      (2000, 256, 16384)])
def test_gate_pack_integer_exact(orc, dtype, T, dm, dff):
    """Integer inputs: every sum is exact, so count, col and val match bit for
    bit, including exact g == 0 ties (not stored). T <= 64 runs the few-token
    kernel (T = 33: a second, one-token chunk), T > 64 the tiled one with
    192-token tiles, and 2000 x 16384 (512 tiles of 256 x 256) the 256-token
    tiles with a ragged last token tile."""
    if dtype == "f32" and dm > 2048:
        pytest.skip("fp32 limit is d_model <= 2048")
    announce("gate_pack int", dtype, T, dm, dff)
    d = synth.make_integer_inputs(T, dm, dff, dtype, 0.03)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    assert np.sum(g == 0) > 0 or T < 10
    x, wg = upload(d, ("x", "wg_t"))
    st = status_word()
    out = tw.gate_pack(x, wg, width=128, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_twell_matches(out, g, dtype, 128, exact=True)


@pytest.mark.parametrize("w", [synth.TINY_F32, synth.SCALE_0P5B],
                         ids=lambda w: w.name)
def test_gate_pack_gaussian(orc, w):
    announce("gate_pack gauss", w.name)
    d = synth.make_inputs(w)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    x, wg = upload(d, ("x", "wg_t"))
    st = status_word()
    out = tw.gate_pack(x, wg, width=w.width, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_twell_matches(out, g, w.dtype, w.width, g_mag=gate_mag(orc, d["x"], d["wg_t"]))


def test_gate_pack_1p5b_sampled_rows(orc):
    """Full 8192 x 2048 x 5632 launch; 256 seeded rows checked by the oracle."""
    w = synth.SCALE_1P5B
    announce("gate_pack 1.5b sampled", w.T)
    d = synth.make_inputs(w)
    x, wg = upload(d, ("x", "wg_t"))
    st = status_word()
    out = tw.gate_pack(x, wg, width=w.width, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rows = np.sort(np.random.default_rng(11).choice(w.T, 256, replace=False))
    g = orc.gate(f64(d["x"][rows]), f64(d["wg_t"]))
    sub = tw.Twell(out.count[rows], out.col[rows], out.val[rows])
    assert_twell_matches(sub, g, w.dtype, w.width)


@pytest.mark.parametrize("T", [40, 70])
def test_gate_pack_width_overflow(orc, T):
    """A dense tile (x[:,0] = 0 removes the offset, ~50% positive) with W = 8:
    true count kept, first 8 columns stored, device flag raised (few-token and
    tiled kernels)."""
    announce("gate_pack width overflow", T)
    d = synth.make_integer_inputs(T, 128, 256, "bf16", 0.02, skew_rows=T)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    ref = orc.twell_pack(g, W=8)
    assert ref["overflow"]
    x, wg = upload(d, ("x", "wg_t"))
    st = status_word()
    out = tw.gate_pack(x, wg, width=8, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & tw.DEV_TILE_OVERFLOW
    assert np.array_equal(out.count.cpu().numpy(), ref["count"])
    n = np.minimum(ref["count"], 8)
    col = out.col.cpu().numpy()
    val = f64(out.val)
    rv = f64(to_storage(ref["val"], "bf16"))
    for t in range(T):
        for j in range(2):
            k = n[t, j]
            assert np.array_equal(col[t, j, :k], ref["col"][t, j, :k])
            assert np.array_equal(val[t, j, :k], rv[t, j, :k])


def test_gate_pack_all_zero_and_empty(orc):
    announce("gate_pack zero/empty")
    x = torch.zeros((5, 64), dtype=torch.bfloat16, device=DEV)
    wg = torch.ones((256, 64), dtype=torch.bfloat16, device=DEV)
    out = tw.gate_pack(x, wg)
    torch.cuda.synchronize()
    assert int(out.count.sum()) == 0
    empty = tw.gate_pack(x[:0], wg)  # T == 0: valid no-op
    torch.cuda.synchronize()
    assert empty.count.shape == (0, 2)


@pytest.mark.parametrize("T", [64, 1000])
def test_gate_pack_deterministic(T):
    announce("gate_pack determinism", T)
    d = synth.make_inputs(synth.SCALE_0P5B.with_(T=T))
    x, wg = upload(d, ("x", "wg_t"))
    a = tw.gate_pack(x, wg, width=32)
    b = tw.gate_pack(x, wg, width=32)
    torch.cuda.synchronize()
    assert torch.equal(a.count, b.count)
    n = torch.minimum(a.count, torch.tensor(32, device=DEV))
    keep = torch.arange(32, device=DEV)[None, None, :] < n[:, :, None]
    assert torch.equal(a.col[keep], b.col[keep])
    assert torch.equal(a.val[keep].view(torch.int16), b.val[keep].view(torch.int16))


# ------------------------------------------------------------ fused up/down
def _fwd_on_oracle_twell(orc, d, dtype, W):
    x64 = f64(d["x"])
    g = orc.gate(x64, f64(d["wg_t"]))
    tw_r, (cnt, col, val) = oracle_twell_for_gpu(orc, g, W, dtype, DEV)
    y_ref = orc.ffn_twell(x64, tw_r, f64(d["wu_t"]), f64(d["wd"]))
    x, wu, wd = upload(d, ("x", "wu_t", "wd"))
    y = tw.ffn_fwd(x, tw.Twell(cnt, col, val), wu, wd)
    torch.cuda.synchronize()
    return y, y_ref, g, tw_r


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,dm,dff", [(1, 64, 128), (77, 320, 384), (130, 1024, 512),
                                      (40, 2304, 768), (33, 2048, 384), (64, 4096, 256),
                                      (65, 896, 640), (1029, 2048, 4096), (1029, 2304, 4096)])
def test_ffn_fwd_integer_exact(orc, dtype, T, dm, dff):
    """Integer inputs: y matches the oracle bit for bit. 1029 tokens with 16 MB
    or more of weights take the two-pass XCD-local path, with a ragged last
    group of tokens: d_model 2048 reads each XCD's slice of wd in place,
    d_model 2304 (slices of 576 bytes) from a slice-major copy."""
    if dtype == "f32" and dm > 2048:
        pytest.skip("fp32 limit is d_model <= 2048")
    announce("ffn_fwd int", dtype, T, dm, dff)
    d = synth.make_integer_inputs(T, dm, dff, dtype, 0.05)
    y, y_ref, _, _ = _fwd_on_oracle_twell(orc, d, dtype, 128)
    assert np.array_equal(f64(y), y_ref)


@pytest.mark.parametrize("dtype,T,dm,dff,W", [("f32", 77, 320, 384, 1), ("bf16", 77, 320, 384, 5),
                                              ("bf16", 300, 1024, 2816, 7),
                                              ("bf16", 1029, 2048, 4096, 7)])
def test_ffn_fwd_narrow_width_exact(orc, dtype, T, dm, dff, W):
    """TwELL widths below the 8 slots a lane stages at once, with tiles holding
    more nonzeros than W (the first W are stored, as the oracle's pack keeps
    them): the staging reads slots of the next tile and past the row's last
    tile, which must never be used. 1029 tokens take the two-pass path."""
    announce("ffn_fwd narrow W", dtype, T, dm, dff, W)
    d = synth.make_integer_inputs(T, dm, dff, dtype, 0.05)
    y, y_ref, g, _ = _fwd_on_oracle_twell(orc, d, dtype, W)
    assert orc.twell_pack(g, W=W)["overflow"]
    assert np.array_equal(f64(y), y_ref)


@pytest.mark.parametrize("w", [synth.TINY_F32, synth.SCALE_0P5B, synth.DECODE_2B.with_(T=64),
                               synth.DECODE_2B.with_(T=1)], ids=lambda w: f"{w.name}-{w.T}")
def test_ffn_fwd_on_oracle_twell(orc, w):
    announce("ffn_fwd on oracle TwELL", w.name, w.T)
    d = synth.make_inputs(w)
    y, y_ref, _, tw_r = _fwd_on_oracle_twell(orc, d, w.dtype, w.width)
    assert_close(y, y_ref, w.dtype, "y", mag=ffn_twell_mag(orc, d["x"], tw_r, d["wu_t"], d["wd"]))


@pytest.mark.parametrize("T", [8, 300])
def test_ffn_fwd_deterministic(T):
    """Fixed summation order: two calls give the same bits."""
    announce("ffn_fwd determinism", T)
    w = synth.DECODE_2B.with_(T=T)
    x, wg, wu, wd = upload(synth.make_inputs(w))
    t = tw.gate_pack(x, wg, width=w.width)
    a = tw.ffn_fwd(x, t, wu, wd)
    b = tw.ffn_fwd(x, t, wu, wd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("w", [synth.TINY_F32, synth.SCALE_0P5B] +
                         [synth.DECODE_2B.with_(T=t) for t in synth.DECODE_T],
                         ids=lambda w: f"{w.name}-{w.T}")
def test_forward_end_to_end(orc, w):
    """GPU gate_pack -> GPU ffn_fwd against the oracle's dense-layer output
    (entries in the |g| < 1e-3 band contribute below the tolerance)."""
    announce("forward e2e", w.name, w.T)
    d = synth.make_inputs(w)
    x64 = f64(d["x"])
    g = orc.gate(x64, f64(d["wg_t"]))
    tw_r, _ = oracle_twell_for_gpu(orc, g, 128, w.dtype, "cpu")
    y_ref = orc.ffn_twell(x64, tw_r, f64(d["wu_t"]), f64(d["wd"]))
    x, wg, wu, wd = upload(d)
    st = status_word()
    t = tw.gate_pack(x, wg, width=w.width, status=st,
                     out=poisoned_twell(tw, w.T, w.d_ff, w.width, x.dtype, DEV))
    y = tw.ffn_fwd(x, t, wu, wd, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    mag, extra = (forward_e2e_bounds(orc, d["x"], d["wg_t"], d["wu_t"], d["wd"], w.width)
                  if w.dtype == "f32" else (None, None))
    assert_close(y, y_ref, w.dtype, "y", mag=mag, extra=extra)


def test_forward_1p5b_sweep_sampled(orc):
    """1.5B-scale layer at every density of the sweep: full launch, 128 rows
    checked (rows are independent)."""
    rows = np.sort(np.random.default_rng(5).choice(8192, 128, replace=False))
    for rho in synth.SWEEP_1P5B:
        w = synth.sweep_workload(rho)  # the widths bench.py's sweep runs
        announce("forward 1.5b sweep", rho)
        d = synth.make_inputs(w)
        x, wg, wu, wd = upload(d)
        st = status_word()
        t = tw.gate_pack(x, wg, width=w.width, status=st,
                         out=poisoned_twell(tw, w.T, w.d_ff, w.width, x.dtype, DEV))
        y = tw.ffn_fwd(x, t, wu, wd)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        x64 = f64(d["x"][rows])
        g = orc.gate(x64, f64(d["wg_t"]))
        tw_r, _ = oracle_twell_for_gpu(orc, g, w.width, "bf16", "cpu")
        y_ref = orc.ffn_twell(x64, tw_r, f64(d["wu_t"]), f64(d["wd"]))
        assert_close(y[rows], y_ref, "bf16", f"y rho={rho}")
        del x, wg, wu, wd, t, y
        torch.cuda.empty_cache()


# ------------------------------------------------------------ TwELL -> hybrid
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_to_hybrid_on_oracle_twell_exact(orc, dtype):
    announce("to_hybrid exact", dtype)
    d = synth.make_integer_inputs(300, 128, 640, dtype, 0.03, skew_rows=17)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    nnz = (g > 0).sum(1)
    K = int(np.sort(nnz)[-25])
    for max_ovf in (64, 10):
        tw_r, (cnt, col, val) = oracle_twell_for_gpu(orc, g, 128, dtype, DEV)
        ref = orc.to_hybrid(tw_r, K, max_ovf)
        st = status_word()
        hy = tw.to_hybrid(tw.Twell(cnt, col, val), K, max_ovf, status=st,
                          out=poisoned_hybrid(tw, 300, 640, K, max_ovf, val.dtype, DEV))
        torch.cuda.synchronize()
        assert bool(int(st.item()) & tw.DEV_OVF_CAPACITY) == ref["capacity_exceeded"]
        assert_hybrid_equal(hybrid_to_numpy(hy), ref)


@pytest.mark.parametrize("dtype,dff", [("bf16", 640), ("bf16", 16512), ("f32", 8320)])
def test_to_hybrid_wide_rows_exact(orc, dtype, dff):
    """Backup rows built in the workgroup's 32 KB LDS row buffer (640) and, when
    a row is wider than it (16512 bf16, 8320 f32), straight in memory; 203
    tokens leave a ragged last block of rows."""
    announce("to_hybrid wide rows", dtype, dff)
    d = synth.make_integer_inputs(203, 128, dff, dtype, 0.03, skew_rows=11)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    K = int(np.sort((g > 0).sum(1))[-12])
    tw_r, (cnt, col, val) = oracle_twell_for_gpu(orc, g, 128, dtype, DEV)
    ref = orc.to_hybrid(tw_r, K, 64)
    assert ref["n_ovf"] >= 11
    st = status_word()
    hy = tw.to_hybrid(tw.Twell(cnt, col, val), K, 64, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_hybrid_equal(hybrid_to_numpy(hy), ref)


def test_to_hybrid_end_to_end_integer(orc):
    """GPU gate_pack -> GPU to_hybrid on integer inputs equals the oracle."""
    announce("to_hybrid e2e int")
    d = synth.make_integer_inputs(257, 256, 512, "bf16", 0.02, skew_rows=13)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    tw_r, _ = oracle_twell_for_gpu(orc, g, 128, "bf16", "cpu")
    ref = orc.to_hybrid(tw_r, 40, 32)
    x, wg = upload(d, ("x", "wg_t"))
    t = tw.gate_pack(x, wg, out=poisoned_twell(tw, 257, 512, 128, x.dtype, DEV))
    hy = tw.to_hybrid(t, 40, 32, out=poisoned_hybrid(tw, 257, 512, 40, 32, x.dtype, DEV))
    torch.cuda.synchronize()
    assert_hybrid_equal(hybrid_to_numpy(hy), ref)
    assert ref["n_ovf"] == 13


def test_to_hybrid_training_layer(orc):
    """Skewed 1.5B training layer (K = 128): the GPU's own TwELL -> hybrid;
    rows and backup checked against the oracle's, exactly where no entry of the
    row lies in the ambiguity band."""
    w = synth.TRAIN_1P5B
    announce("to_hybrid training layer")
    d = synth.make_inputs(w)
    x, wg = upload(d, ("x", "wg_t"))
    st = status_word()
    t = tw.gate_pack(x, wg, width=w.width, status=st)
    hy = tw.to_hybrid(t, w.K, w.max_ovf, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    gpu = hybrid_to_numpy(hy)
    skew = d["skew_rows"].numpy()
    assert gpu["n_ovf"] == len(skew) == 410
    assert np.array_equal(gpu["ovf_rows"][:410], skew)
    rows = np.sort(np.random.default_rng(2).choice(w.T, 96, replace=False))
    rows = np.union1d(rows, skew[:16])
    g = orc.gate(f64(d["x"][rows]), f64(d["wg_t"]))
    for r, t_ in enumerate(rows):
        pos = g[r] > 0
        amb = np.abs(g[r]) < 1e-3
        assert gpu["row_nnz"][t_] == pos.sum() or amb.any()
        if amb.any():
            continue
        if gpu["row_slot"][t_] < 0:
            n = gpu["row_nnz"][t_]
            assert np.array_equal(gpu["ell_col"][t_, :n], np.nonzero(pos)[0])
            assert_close(gpu["ell_val"][t_, :n], g[r][pos], "bf16", "ell")
        else:
            dense = gpu["dense"][gpu["row_slot"][t_]]
            assert np.array_equal(dense != 0, pos)
            assert_close(dense[pos], g[r][pos], "bf16", "backup")
