"""GPU parity of hybrid_ffn_fwd (the training forward over the hybrid layout)
against the oracle's forward over the same hybrid, through the C-ABI.

As for the backward, the hybrid fed to the GPU is the oracle's (values rounded
to the storage dtype): inputs flow oracle -> GPU only.
"""
import numpy as np
import pytest
import torch

from activation_sparse_ffn_gemm_amd import _lib as tw
from activation_sparse_ffn_gemm_amd import synth
from helpers import assert_close, f64, ffn_hybrid_mag, poisoned_hybrid, poisoned_twell
from test_gpu_bwd import oracle_hybrid, upload_hybrid

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(*a):
    print("[case]", *a, flush=True)


def run_fwd(d, hy):
    x, wu, wd = (d[k].to(DEV) for k in ("x", "wu_t", "wd"))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = tw.hybrid_fwd(x, hy, wu, wd, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,dm,dff,K,skew", [(1, 64, 128, 8, 0), (150, 192, 384, 12, 9),
                                             (300, 512, 1024, 40, 21), (77, 320, 256, 128, 0),
                                             (1029, 2048, 4096, 256, 51),
                                             (1029, 2304, 4096, 256, 51),
                                             (1029, 2048, 2048, 256, 51)])
def test_hybrid_fwd_integer_exact(orc, dtype, T, dm, dff, K, skew):
    """Integer inputs: the ELL gathers and the backup rows' hi/lo MFMA products
    are exact, so y matches the oracle bit for bit. The 1029-token shapes with
    16 MB or more of weights take the two-pass XCD-local ELL path, with a
    ragged last group of tokens and the backup products on the second stream:
    in bf16 wd's slices read in place (d_model 2048) and from a slice-major
    copy (d_model 2304); in f32 (float32 MFMA products, one array per
    intermediate) d_model 2048 by d_ff 2048."""
    if T == 1029 and (dtype == "f32") != (dff == 2048):
        pytest.skip("one dtype per two-pass shape")
    announce("hyb fwd int", dtype, T, dm, dff, K, skew)
    d = synth.make_integer_inputs(T, dm, dff, dtype, 0.03, skew_rows=skew)
    ref = oracle_hybrid(orc, d, dtype, K, 64)
    assert (ref["n_ovf"] > 0) == (skew > 0)
    y = run_fwd(d, upload_hybrid(ref, dtype))
    want = orc.ffn_hybrid(f64(d["x"]), ref, f64(d["wu_t"]), f64(d["wd"]))
    assert np.array_equal(f64(y), want)


@pytest.mark.parametrize("w", [
    synth.Workload("small-f32", 96, 256, 512, "f32", 0.03, skew_frac=0.1, skew_density=0.4,
                   K=40, max_ovf=16),
    synth.Workload("small-bf16", 200, 384, 640, "bf16", 0.02, skew_frac=0.05, skew_density=0.3,
                   K=48, max_ovf=16),
    synth.Workload("all-ell-bf16", 256, 1024, 2816, "bf16", 0.01, K=128, max_ovf=8),
], ids=lambda w: w.name)
def test_hybrid_fwd_gaussian(orc, w):
    announce("hyb fwd gauss", w.name)
    d = synth.make_inputs(w)
    ref = oracle_hybrid(orc, d, w.dtype, w.K, w.max_ovf)
    y = run_fwd(d, upload_hybrid(ref, w.dtype))
    mag = ffn_hybrid_mag(orc, d["x"], ref, d["wu_t"], d["wd"])
    assert_close(y, orc.ffn_hybrid(f64(d["x"]), ref, f64(d["wu_t"]), f64(d["wd"])), w.dtype, "y",
                 mag=mag)


def test_hybrid_fwd_training_layer_full(orc):
    """The skewed 1.5B training layer at full size (T = 8192, 410 backup rows
    holding most of the nonzeros): every y element against the oracle."""
    w = synth.TRAIN_1P5B
    announce("hyb fwd training layer full")
    d = synth.make_inputs(w)
    ref = oracle_hybrid(orc, d, w.dtype, w.K, w.max_ovf)
    assert ref["n_ovf"] == 410
    y = run_fwd(d, upload_hybrid(ref, w.dtype))
    assert_close(y, orc.ffn_hybrid(f64(d["x"]), ref, f64(d["wu_t"]), f64(d["wd"])), w.dtype, "y")


def test_hybrid_fwd_concurrent_threads(orc):
    """Two host threads, each on a stream of its own, run the large-layer
    forward (1029 tokens, 16 MB weights: the backup rows' products go to the
    library's second stream) at the same time, four calls each: every result
    equals the one-thread result bit for bit, and no status bit is raised."""
    import threading
    announce("hyb fwd two threads")
    d = synth.make_integer_inputs(1029, 2048, 4096, "bf16", 0.03, skew_rows=51)
    ref = oracle_hybrid(orc, d, "bf16", 256, 64)
    assert ref["n_ovf"] > 0
    hy = upload_hybrid(ref, "bf16")
    want = run_fwd(d, hy)
    x, wu, wd = (d[k].to(DEV) for k in ("x", "wu_t", "wd"))
    torch.cuda.synchronize()
    got, errors = [[], []], []

    def work(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(4):
                    st = torch.zeros(1, dtype=torch.int32, device=DEV)
                    got[k].append((tw.hybrid_fwd(x, hy, wu, wd, status=st), st))
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(2):
        assert len(got[k]) == 4
        for y, st in got[k]:
            assert int(st.item()) == 0
            assert torch.equal(y, want)


def test_hybrid_fwd_agrees_with_twell_fwd():
    """On one TwELL, the forward over its hybrid and the TwELL forward are the
    same sums (GPU against GPU; each is checked against the oracle above)."""
    w = synth.Workload("e2e", 512, 256, 768, "bf16", 0.02, skew_frac=0.05, skew_density=0.3,
                       K=40, max_ovf=64, width=128)
    announce("hyb fwd vs twell fwd")
    d = synth.make_inputs(w)
    x, wg, wu, wd = (d[k].to(DEV) for k in ("x", "wg_t", "wu_t", "wd"))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    t = tw.gate_pack(x, wg, width=w.width, status=st,
                     out=poisoned_twell(tw, w.T, w.d_ff, w.width, torch.bfloat16, DEV))
    y_tw = tw.ffn_fwd(x, t, wu, wd, status=st)
    hy = tw.to_hybrid(t, w.K, w.max_ovf, status=st,
                      out=poisoned_hybrid(tw, w.T, w.d_ff, w.K, w.max_ovf, torch.bfloat16, DEV))
    y_hy = tw.hybrid_fwd(x, hy, wu, wd, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(hy.n_ovf.item()) > 0
    np.testing.assert_allclose(f64(y_hy), f64(y_tw), rtol=2e-5, atol=2e-5 * float(y_tw.abs().max()))


def test_hybrid_fwd_empty_and_no_backup(orc):
    announce("hyb fwd empty")
    hy0 = tw.empty_hybrid(0, 256, 16, 4, torch.bfloat16, DEV)
    hy0.n_ovf.zero_()
    x0 = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    wu = torch.zeros((256, 64), dtype=torch.bfloat16, device=DEV)
    assert tw.hybrid_fwd(x0, hy0, wu, wu).shape == (0, 64)
    d = synth.make_integer_inputs(40, 128, 256, "bf16", 0.03)
    ref = oracle_hybrid(orc, d, "bf16", 128, 0)
    assert ref["n_ovf"] == 0
    y = run_fwd(d, upload_hybrid(ref, "bf16"))
    assert np.array_equal(f64(y), orc.ffn_hybrid(f64(d["x"]), ref, f64(d["wu_t"]), f64(d["wd"])))
