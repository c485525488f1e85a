"""GPU parity of hybrid_ffn_bwd against the oracle's backward, through the C-ABI.

The hybrid fed to the GPU is the oracle's (values rounded to the storage
dtype), and the oracle's backward runs on exactly those values: inputs flow
oracle -> GPU only. The ReLU derivative is discontinuous, so the pattern must
be the same on both sides; the GPU's own pattern is checked in test_gpu_fwd.
"""
import numpy as np
import pytest
import torch

from activation_sparse_ffn_gemm_amd import _lib as tw
from activation_sparse_ffn_gemm_amd import synth
from helpers import (assert_close, bwd_hybrid_mag, f64, oracle_twell_for_gpu, poison_cols,
                     poisoned_hybrid, poisoned_twell, to_storage)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dx", "dwg_t", "dwu_t", "dwd")


def announce(*a):
    print("[case]", *a, flush=True)


def oracle_hybrid(orc, d, dtype, K, max_ovf, rows=None):
    """Oracle TwELL -> hybrid of inputs d, values rounded to storage dtype."""
    x = f64(d["x"] if rows is None else d["x"][rows])
    g = orc.gate(x, f64(d["wg_t"]))
    tw_r, _ = oracle_twell_for_gpu(orc, g, 128, dtype, "cpu")
    return orc.to_hybrid(tw_r, K, max_ovf)


def upload_hybrid(ref: dict, dtype: str) -> tw.Hybrid:
    """The oracle's hybrid on the GPU, its unspecified parts poisoned: ELL
    slots past a row's length (all slots of backup rows) get NaN values and
    in-range columns, backup rows past n_ovf NaN, their row ids in range."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    mo, T, K, dff = ref["max_ovf"], ref["row_nnz"].shape[0], ref["K"], ref["d_ff"]
    ell_len = np.where(ref["row_slot"] < 0, ref["row_nnz"], 0)
    pad = np.arange(K)[None, :] >= ell_len[:, None]
    col = np.where(pad, poison_cols((T, K), dff, 96), ref["ell_col"]).astype(np.int16)
    val = np.where(pad, np.nan, ref["ell_val"])
    n = min(ref["n_ovf"], mo)
    rows = ref["ovf_rows"][:mo].copy()
    rows[n:] = np.random.default_rng(95).integers(0, max(T, 1), mo - n)
    dense = ref["dense"][:mo].copy()
    dense[n:] = np.nan
    return tw.Hybrid(
        torch.from_numpy(ref["row_nnz"].copy()).to(DEV),
        torch.from_numpy(ref["row_slot"].copy()).to(DEV),
        torch.from_numpy(col).to(DEV),
        torch.from_numpy(val).to(tdt).to(DEV),
        torch.from_numpy(rows.astype(np.int32)).to(DEV) if mo else
        torch.zeros(0, dtype=torch.int32, device=DEV),
        torch.from_numpy(dense).to(tdt).to(DEV).reshape(mo, dff),
        torch.tensor([ref["n_ovf"]], dtype=torch.int32, device=DEV))


def run_bwd(d, hy, dtype, l1=0.0):
    x, dy, wg, wu, wd = (d[k].to(DEV) for k in ("x", "dy", "wg_t", "wu_t", "wd"))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = tw.ffn_bwd(x, dy, hy, wg, wu, wd, status=st, l1=l1)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return out


def oracle_bwd(orc, d, ref, l1=0.0):
    return orc.bwd_hybrid(f64(d["x"]), f64(d["dy"]), ref, f64(d["wg_t"]), f64(d["wu_t"]),
                          f64(d["wd"]), l1=l1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,dm,dff,K,skew,l1", [(1, 64, 128, 8, 0, 0.0),
                                                (150, 192, 384, 12, 9, 0.0),
                                                (300, 512, 1024, 40, 21, 0.0),
                                                (77, 320, 256, 128, 0, 0.0),
                                                (150, 192, 384, 12, 9, 0.5),
                                                (130, 128, 16384, 512, 5, 0.0),
                                                (1024, 2048, 4096, 256, 51, 0.0),
                                                (1024, 2304, 4096, 256, 51, 0.0),
                                                (1024, 2048, 2048, 256, 51, 0.0)])
def test_bwd_integer_exact(orc, dtype, T, dm, dff, K, skew, l1):
    """Integer inputs (and an L1 weight of 0.5): ELL gathers and the backup
    rows' hi/lo MFMA products are exact, so every gradient matches the oracle
    bit for bit. d_ff 16384 gives 256 groups of 64 neurons (the column offsets
    sum many group totals) and 16 mask chunks. The last two shapes (1024
    tokens, 16 MB or more of weights in bf16) take the XCD-local dx pass
    (slices of 512 and 576 bytes); the 1024-token f32 shape (d_model 2048 by
    d_ff 2048, 16 MB in f32) takes it with float32 MFMA backup products."""
    if T == 1024 and (dtype == "f32") != (dff == 2048):
        pytest.skip("one dtype per two-pass shape")
    announce("bwd int", dtype, T, dm, dff, K, skew, l1)
    d = synth.make_integer_inputs(T, dm, dff, dtype, 0.03, with_dy=True, skew_rows=skew)
    ref = oracle_hybrid(orc, d, dtype, K, 64)
    assert (ref["n_ovf"] > 0) == (skew > 0)
    got = run_bwd(d, upload_hybrid(ref, dtype), dtype, l1=l1)
    want = oracle_bwd(orc, d, ref, l1=l1)
    for n, a, b in zip(NAMES, got, want):
        assert np.array_equal(f64(a), b), n


@pytest.mark.parametrize("w", [
    synth.Workload("small-f32", 96, 256, 512, "f32", 0.03, skew_frac=0.1, skew_density=0.4,
                   K=40, max_ovf=16),
    synth.Workload("small-bf16", 200, 384, 640, "bf16", 0.02, skew_frac=0.05, skew_density=0.3,
                   K=48, max_ovf=16),
    synth.Workload("all-ell-bf16", 256, 1024, 2816, "bf16", 0.01, K=128, max_ovf=8),
], ids=lambda w: w.name)
def test_bwd_gaussian(orc, w):
    announce("bwd gauss", w.name)
    d = synth.make_inputs(w, with_dy=True)
    ref = oracle_hybrid(orc, d, w.dtype, w.K, w.max_ovf)
    got = run_bwd(d, upload_hybrid(ref, w.dtype), w.dtype)
    want = oracle_bwd(orc, d, ref)
    mags = bwd_hybrid_mag(orc, d["x"], d["dy"], ref, d["wg_t"], d["wu_t"], d["wd"])
    for n, a, b, m in zip(NAMES, got, want, mags):
        assert_close(a, b, w.dtype, n, mag=m)


def test_capacity_exceeded_large_layer(orc):
    """A large layer (1029 tokens, 16 MB of weights: the two-pass forward with
    its second stream, the XCD-split dx pass) whose backup rows outnumber the
    capacity: the GPU conversion raises OVF_CAPACITY (and nothing else), the
    forward and the backward still run to the end, and the rows they keep
    defined (the ELL rows and the first max_ovf backup rows: y and dx) equal
    the oracle's over a hybrid with room for every backup row."""
    announce("capacity exceeded, large layer")
    T, dm, dff, K, mo = 1029, 2048, 4096, 256, 16
    d = synth.make_integer_inputs(T, dm, dff, "bf16", 0.03, with_dy=True, skew_rows=51)
    x64 = f64(d["x"])
    g = orc.gate(x64, f64(d["wg_t"]))
    tw_r, (cnt, col, val) = oracle_twell_for_gpu(orc, g, 128, "bf16", DEV)
    short = orc.to_hybrid(tw_r, K, mo)
    full = orc.to_hybrid(tw_r, K, T)
    assert short["capacity_exceeded"] and full["n_ovf"] > mo and not full["capacity_exceeded"]
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    hy = tw.to_hybrid(tw.Twell(cnt, col, val), K, mo, status=st)
    x, dy, wg, wu, wd = (d[k].to(DEV) for k in ("x", "dy", "wg_t", "wu_t", "wd"))
    y = tw.hybrid_fwd(x, hy, wu, wd, status=st)
    dx = tw.ffn_bwd(x, dy, hy, wg, wu, wd, status=st)[0]
    torch.cuda.synchronize()
    assert int(st.item()) == tw.DEV_OVF_CAPACITY
    slot = full["row_slot"]
    kept = (slot < 0) | (slot < mo)
    assert kept.sum() == T - (full["n_ovf"] - mo)
    want_y = orc.ffn_hybrid(x64, full, f64(d["wu_t"]), f64(d["wd"]))
    want_dx = oracle_bwd(orc, d, full)[0]
    assert np.array_equal(f64(y)[kept], want_y[kept])
    assert np.array_equal(f64(dx)[kept], want_dx[kept])


def test_bwd_training_layer_full(orc):
    """The skewed 1.5B training layer at full size (T = 8192, 410 backup rows),
    with the recipe's L1 weight 2e-5: every gradient element against the
    oracle on the same hybrid."""
    w = synth.TRAIN_1P5B
    announce("bwd training layer full")
    d = synth.make_inputs(w, with_dy=True)
    ref = oracle_hybrid(orc, d, w.dtype, w.K, w.max_ovf)
    assert ref["n_ovf"] == 410
    got = run_bwd(d, upload_hybrid(ref, w.dtype), w.dtype, l1=2e-5)
    want = oracle_bwd(orc, d, ref, l1=2e-5)
    for n, a, b in zip(NAMES, got, want):
        assert_close(a, b, w.dtype, n)


def test_bwd_deterministic(orc):
    w = synth.Workload("det", 512, 256, 768, "bf16", 0.02, skew_frac=0.05, skew_density=0.3,
                       K=40, max_ovf=64)
    announce("bwd determinism")
    d = synth.make_inputs(w, with_dy=True)
    hy = upload_hybrid(oracle_hybrid(orc, d, w.dtype, w.K, w.max_ovf), w.dtype)
    a = run_bwd(d, hy, w.dtype)
    b = run_bwd(d, hy, w.dtype)
    for n, p, q in zip(NAMES, a, b):
        assert torch.equal(p, q), n


def test_bwd_empty_and_no_backup(orc):
    """T == 0 writes zero weight gradients; max_ovf == 0 runs ELL rows only."""
    announce("bwd empty")
    d = synth.make_integer_inputs(40, 128, 256, "bf16", 0.03, with_dy=True)
    wg, wu, wd = (d[k].to(DEV) for k in ("wg_t", "wu_t", "wd"))
    hy0 = tw.empty_hybrid(0, 256, 16, 0, torch.bfloat16, DEV)
    f = dict(dtype=torch.float32, device=DEV)
    out = (torch.empty((0, 128), **f),) + tuple(torch.full((256, 128), 7.0, **f) for _ in range(3))
    x0 = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    tw.ffn_bwd(x0, x0, hy0, wg, wu, wd, out=out)
    torch.cuda.synchronize()
    for o in out[1:]:
        assert int(torch.count_nonzero(o)) == 0
    ref = oracle_hybrid(orc, d, "bf16", 128, 0)
    assert ref["n_ovf"] == 0
    got = run_bwd(d, upload_hybrid(ref, "bf16"), "bf16")
    for n, a, b in zip(NAMES, got, oracle_bwd(orc, d, ref)):
        assert np.array_equal(f64(a), b), n


def test_backward_end_to_end_integer(orc):
    """GPU gate_pack -> to_hybrid -> bwd on integer inputs equals the oracle's
    backward on its own hybrid (patterns are exact, so they agree)."""
    announce("bwd e2e int")
    d = synth.make_integer_inputs(384, 256, 768, "bf16", 0.02, with_dy=True, skew_rows=19)
    ref = oracle_hybrid(orc, d, "bf16", 48, 32)
    x, wg = d["x"].to(DEV), d["wg_t"].to(DEV)
    t = tw.gate_pack(x, wg, out=poisoned_twell(tw, 384, 768, 128, torch.bfloat16, DEV))
    hy = tw.to_hybrid(t, 48, 32, out=poisoned_hybrid(tw, 384, 768, 48, 32, torch.bfloat16, DEV))
    got = run_bwd(d, hy, "bf16")
    for n, a, b in zip(NAMES, got, oracle_bwd(orc, d, ref)):
        assert np.array_equal(f64(a), b), n
