"""GPU parity of twell_decode_fwd (the whole layer for few tokens in one call,
three launches) against the oracle, through the C-ABI: its TwELL output
against the oracle's pre-activations, its y against the oracle's forward."""
import numpy as np
import pytest
import torch

from activation_sparse_ffn_gemm_amd import _lib as tw
from activation_sparse_ffn_gemm_amd import synth
from helpers import (assert_close, assert_twell_matches, f64, forward_e2e_bounds, gate_mag,
                     oracle_twell_for_gpu, poisoned_twell)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(*a):
    print("[case]", *a, flush=True)


def run_decode(d, width, status_ok=True):
    x, wg, wu, wd = (d[k].to(DEV) for k in ("x", "wg_t", "wu_t", "wd"))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, y = tw.decode_fwd(x, wg, wu, wd, width=width, status=st,
                           out=poisoned_twell(tw, x.shape[0], wg.shape[0], width, x.dtype, DEV))
    torch.cuda.synchronize()
    if status_ok:
        assert int(st.item()) == 0
    return out, y, int(st.item())


def oracle_forward(orc, d, dtype, W):
    x64 = f64(d["x"])
    g = orc.gate(x64, f64(d["wg_t"]))
    tw_r, _ = oracle_twell_for_gpu(orc, g, W, dtype, "cpu")
    return g, orc.ffn_twell(x64, tw_r, f64(d["wu_t"]), f64(d["wd"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,dm,dff", [(1, 64, 128), (2, 256, 384), (3, 1024, 1024),
                                      (4, 2304, 6144), (5, 512, 256), (8, 2304, 768),
                                      (33, 512, 1024), (64, 1024, 384), (64, 4096, 256)])
def test_decode_integer_exact(orc, dtype, T, dm, dff):
    """Integer inputs: the TwELL and y match the oracle bit for bit. T <= 4:
    the matrix-vector gate (1, 2 and 4 tokens per lane); T = 33: a second,
    one-token chunk in the MFMA gate."""
    if dtype == "f32" and dm > 2048:
        pytest.skip("fp32 limit is d_model <= 2048")
    announce("decode int", dtype, T, dm, dff)
    d = synth.make_integer_inputs(T, dm, dff, dtype, 0.04)
    g, y_ref = oracle_forward(orc, d, dtype, 128)
    out, y, _ = run_decode(d, 128)
    assert_twell_matches(out, g, dtype, 128, exact=True)
    assert np.array_equal(f64(y), y_ref)


@pytest.mark.parametrize("w", [synth.DECODE_2B.with_(T=t) for t in synth.DECODE_T] +
                         [synth.TINY_F32.with_(T=64), synth.SCALE_0P5B.with_(T=16)],
                         ids=lambda w: f"{w.name}-{w.T}")
def test_decode_gaussian(orc, w):
    """The pages' workload shapes (2B decode at T = 1, 8, 32, 64; tiny fp32;
    0.5B with 16 tokens): TwELL against the oracle's g, y against the oracle's
    forward over its own TwELL."""
    announce("decode gauss", w.name, w.T)
    d = synth.make_inputs(w)
    g, y_ref = oracle_forward(orc, d, w.dtype, w.width)
    out, y, _ = run_decode(d, w.width)
    f32 = w.dtype == "f32"
    assert_twell_matches(out, g, w.dtype, w.width,
                         g_mag=gate_mag(orc, d["x"], d["wg_t"]) if f32 else None)
    mag, extra = (forward_e2e_bounds(orc, d["x"], d["wg_t"], d["wu_t"], d["wd"], w.width)
                  if f32 else (None, None))
    assert_close(y, y_ref, w.dtype, "y", mag=mag, extra=extra)


def test_decode_agrees_with_two_calls():
    """twell_decode_fwd against twell_gate_pack + twell_ffn_fwd on the same
    inputs (GPU against GPU; each is checked against the oracle)."""
    w = synth.DECODE_2B.with_(T=32)
    announce("decode vs gate_pack + ffn_fwd")
    d = synth.make_inputs(w)
    x, wg, wu, wd = (d[k].to(DEV) for k in ("x", "wg_t", "wu_t", "wd"))
    t2 = tw.gate_pack(x, wg, width=w.width)
    y2 = tw.ffn_fwd(x, t2, wu, wd)
    t1, y1 = tw.decode_fwd(x, wg, wu, wd, width=w.width)
    torch.cuda.synchronize()
    # the two gate kernels sum d_model in different orders: a g within rounding
    # of 0 may fall either way
    assert int((t1.count != t2.count).sum()) <= 2
    np.testing.assert_allclose(f64(y1), f64(y2), rtol=1e-3, atol=1e-3 * float(y2.abs().max()))


@pytest.mark.parametrize("T", [1, 4, 12])
def test_decode_width_overflow(orc, T):
    """Dense rows with W = 8: true counts kept, first 8 entries stored and
    used, device flag raised (matrix-vector and MFMA gates)."""
    announce("decode width overflow", T)
    d = synth.make_integer_inputs(T, 128, 256, "bf16", 0.02, skew_rows=T)
    g = orc.gate(f64(d["x"]), f64(d["wg_t"]))
    ref = orc.twell_pack(g, W=8)
    assert ref["overflow"]
    out, y, st = run_decode(d, 8, status_ok=False)
    assert st & tw.DEV_TILE_OVERFLOW
    assert np.array_equal(out.count.cpu().numpy(), ref["count"])
    tw_r, _ = oracle_twell_for_gpu(orc, g, 8, "bf16", "cpu")
    y_ref = orc.ffn_twell(f64(d["x"]), tw_r, f64(d["wu_t"]), f64(d["wd"]))
    assert np.array_equal(f64(y), y_ref)


def test_decode_deterministic_and_empty():
    announce("decode determinism / empty")
    w = synth.DECODE_2B.with_(T=8)
    d = synth.make_inputs(w)
    x, wg, wu, wd = (d[k].to(DEV) for k in ("x", "wg_t", "wu_t", "wd"))
    ta, ya = tw.decode_fwd(x, wg, wu, wd, width=w.width)
    tb, yb = tw.decode_fwd(x, wg, wu, wd, width=w.width)
    torch.cuda.synchronize()
    assert torch.equal(ta.count, tb.count) and torch.equal(ya, yb)
    t0, y0 = tw.decode_fwd(x[:0], wg, wu, wd, width=w.width)
    torch.cuda.synchronize()
    assert t0.count.shape == (0, w.d_ff // 128) and y0.shape == (0, w.d_model)
    # all-zero gate: every count 0, y = 0
    tz, yz = tw.decode_fwd(torch.zeros_like(x), wg, wu, wd, width=w.width)
    torch.cuda.synchronize()
    assert int(tz.count.abs().sum()) == 0 and not bool(yz.any())
