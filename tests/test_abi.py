"""C-ABI checks that need no GPU: the library loads, exports every function
include/twell.h declares, and rejects bad arguments on the host before any
launch (the error paths return before touching the device)."""
import ctypes
import os
import re

import pytest

from activation_sparse_ffn_gemm_amd import _lib as tw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twell.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    return tw.load()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(tw.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.twell_status_str(code)
    assert L.twell_status_str(99) == b"unknown status"


FAKE = 0x100000  # 16-byte aligned, never dereferenced (the calls fail validation first)


def twell_c(T=4, d_ff=256, width=128, dtype=tw.TWELL_BF16, ptr=FAKE):
    return tw.TwellC(T, d_ff, width, dtype, ptr, ptr, ptr)


def hybrid_c(T=4, d_ff=256, K=16, max_ovf=4, dtype=tw.TWELL_BF16, ptr=FAKE):
    return tw.HybridC(T, d_ff, K, max_ovf, dtype, *([ptr] * 7))


def gate(L, dt=tw.TWELL_BF16, x=FAKE, w=FAKE, T=4, dm=64, out=None, ws=FAKE, nb=1 << 30):
    out = out or twell_c(T=T)
    return L.twell_gate_pack(dt, x, w, T, dm, ctypes.byref(out), ws, nb, None, None, None)


def test_gate_pack_validation(L):
    assert gate(L, dt=7) == -3
    assert gate(L, x=0) == -1
    assert gate(L, out=twell_c(dtype=tw.TWELL_F32)) == -3       # dtype mismatch
    assert gate(L, dm=96) == -2                                   # d_model % 64
    assert gate(L, dm=8192) == -2                                 # d_model too large
    assert gate(L, dt=tw.TWELL_F32, dm=4096,
                out=twell_c(dtype=tw.TWELL_F32)) == -2            # fp32 limit 2048
    assert gate(L, out=twell_c(d_ff=200)) == -2                   # d_ff % 128
    assert gate(L, out=twell_c(d_ff=65536)) == -2                 # int16 columns
    assert gate(L, out=twell_c(width=0)) == -2
    assert gate(L, out=twell_c(width=129)) == -2
    assert gate(L, T=5, out=twell_c(T=4)) == -2                   # T mismatch
    assert gate(L, x=FAKE + 2) == -4                              # misaligned
    assert gate(L, out=twell_c(ptr=0)) == -1                      # NULL arrays
    assert gate(L, T=0, out=twell_c(T=0, ptr=0)) == 0             # T == 0: no-op
    need = L.twell_gate_workspace_bytes(tw.TWELL_BF16, 4, 64, 256)
    assert need >= 4 * 256 * 4                                    # few tokens: partials of g
    assert gate(L, nb=need - 1) == -5
    assert gate(L, ws=0, nb=0) == -5
    assert gate(L, ws=FAKE + 4) == -4
    assert L.twell_gate_workspace_bytes(tw.TWELL_BF16, 65, 64, 256) == 0  # tiled kernel: none
    big = twell_c(T=100)
    assert gate(L, T=100, out=big, ws=0, nb=0, x=FAKE + 2) == -4  # no workspace needed


def test_ffn_fwd_validation(L):
    t = twell_c()
    f = lambda **k: L.twell_ffn_fwd(k.get("dt", tw.TWELL_BF16), k.get("x", FAKE),
                                    ctypes.byref(k.get("t", t)), FAKE, FAKE, k.get("dm", 64),
                                    k.get("y", FAKE), k.get("ws", FAKE), k.get("nb", 1 << 30),
                                    None, None, None)
    assert f(dt=9) == -3
    assert f(y=0) == -1
    assert f(dm=100) == -2
    assert f(y=FAKE + 4) == -4
    assert f(t=twell_c(dtype=tw.TWELL_F32)) == -3
    assert f(t=twell_c(T=0, ptr=0)) == 0
    need = L.twell_fwd_workspace_bytes(tw.TWELL_BF16, 4, 64, 256, 128)
    if need:
        assert f(nb=need - 1) == -5                       # workspace too small
        assert f(ws=FAKE + 4) == -4


def test_to_hybrid_validation(L):
    f = lambda t, h: L.twell_to_hybrid(ctypes.byref(t), ctypes.byref(h), None, None, None)
    assert f(twell_c(), hybrid_c(T=5)) == -2            # T mismatch
    assert f(twell_c(), hybrid_c(K=0)) == -2
    assert f(twell_c(), hybrid_c(K=300)) == -2          # K > d_ff
    assert f(twell_c(), hybrid_c(max_ovf=-1)) == -2
    assert f(twell_c(), hybrid_c(dtype=tw.TWELL_F32)) == -3
    assert f(twell_c(), hybrid_c(ptr=0)) == -1
    assert f(twell_c(d_ff=384), hybrid_c()) == -2       # d_ff mismatch


def test_bwd_validation(L):
    h = hybrid_c()
    need = L.hybrid_bwd_workspace_bytes(tw.TWELL_BF16, 4, 64, 256, 16, 4)
    assert need > 0

    def f(ws=FAKE, nbytes=None, dm=64, dx=FAKE, hh=h, dt=tw.TWELL_BF16, l1=0.0):
        return L.hybrid_ffn_bwd(dt, FAKE, FAKE, ctypes.byref(hh), FAKE, FAKE, FAKE, dm, l1, dx,
                                FAKE, FAKE, FAKE, ws, need if nbytes is None else nbytes,
                                None, None, None)
    assert f(l1=float("nan")) == -2
    assert f(l1=float("inf")) == -2
    assert f(nbytes=need - 1) == -5
    assert f(ws=0) == -5
    assert f(dx=0) == -1
    assert f(dm=32) == -2
    assert f(dx=FAKE + 8) == -4
    assert f(dt=tw.TWELL_F32) == -3
    assert f(hh=hybrid_c(max_ovf=-2)) == -2


def test_hybrid_fwd_validation(L):
    h = hybrid_c()
    need = L.hybrid_fwd_workspace_bytes(tw.TWELL_BF16, 4, 64, 256, 16, 4)
    assert need > 0
    assert L.hybrid_fwd_workspace_bytes(tw.TWELL_BF16, 4, 64, 256, 16, 0) == 0  # no backup rows

    def f(ws=FAKE, nbytes=None, dm=64, y=FAKE, hh=h, dt=tw.TWELL_BF16, x=FAKE):
        return L.hybrid_ffn_fwd(dt, x, ctypes.byref(hh), FAKE, FAKE, dm, y, ws,
                                need if nbytes is None else nbytes, None, None, None)
    assert f(nbytes=need - 1) == -5
    assert f(ws=0) == -5
    assert f(y=0) == -1
    assert f(x=0) == -1
    assert f(dm=32) == -2
    assert f(dt=tw.TWELL_F32) == -3
    assert f(hh=hybrid_c(K=0)) == -2
    assert f(y=FAKE + 8) == -4


def test_decode_fwd_validation(L):
    t = twell_c()
    need = L.twell_decode_workspace_bytes(tw.TWELL_BF16, 4, 64, 256, 128)
    # at least the gate partials (one slice or more) and one float per TwELL slot
    assert need >= 4 * 256 * 4 + 4 * 2 * 128 * 4
    assert L.twell_decode_workspace_bytes(tw.TWELL_BF16, 65, 64, 256, 128) == 0   # T limit
    assert L.twell_decode_workspace_bytes(tw.TWELL_BF16, 4, 96, 256, 128) == 0    # d_model % 64
    assert L.twell_decode_workspace_bytes(tw.TWELL_BF16, 4, 64, 200, 128) == 0    # d_ff % 128
    assert L.twell_decode_workspace_bytes(tw.TWELL_F32, 4, 4096, 256, 128) == 0   # fp32 limit

    def f(dt=tw.TWELL_BF16, x=FAKE, w=FAKE, dm=64, tt=t, y=FAKE, ws=FAKE, nb=None):
        return L.twell_decode_fwd(dt, x, w, w, w, dm, ctypes.byref(tt), y, ws,
                                  need if nb is None else nb, None, None, None)
    assert f(dt=9) == -3
    assert f(w=0) == -1
    assert f(y=0) == -1
    assert f(x=0) == -1
    assert f(dm=100) == -2
    assert f(tt=twell_c(T=65)) == -2
    assert f(tt=twell_c(dtype=tw.TWELL_F32)) == -3
    assert f(y=FAKE + 4) == -4
    assert f(nb=need - 1) == -5
    assert f(ws=0) == -5
    assert f(ws=FAKE + 4) == -4
    assert f(tt=twell_c(T=0, ptr=0), x=0, y=0, nb=0, ws=0) == 0   # T == 0: no-op


def test_few_token_ffn_workspace(L):
    """twell_ffn_fwd on few tokens keeps one float per TwELL slot."""
    for T, dff, W in ((1, 6144, 32), (64, 256, 128), (7, 1024, 8)):
        assert L.twell_fwd_workspace_bytes(tw.TWELL_BF16, T, 2304, dff, W) == T * (dff // 128) * W * 4


def test_bwd_rejects_32bit_slot_overflow(L):
    """T * K past 2^31 - 1 (ELL slot numbers are 32-bit) is refused on the host."""
    big = hybrid_c(T=1 << 20, d_ff=4096, K=4096)   # 2^32 slots
    assert L.hybrid_bwd_workspace_bytes(tw.TWELL_BF16, 1 << 20, 64, 4096, 4096, 4) == 0
    assert L.hybrid_ffn_bwd(tw.TWELL_BF16, FAKE, FAKE, ctypes.byref(big), FAKE, FAKE, FAKE, 64,
                            0.0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None, None, None) == -2
    assert L.twell_to_hybrid(ctypes.byref(twell_c(T=1 << 20, d_ff=4096)), ctypes.byref(big),
                             None, None, None) == -2


# ---- the Python wrappers check every tensor before the C-ABI sees a pointer.
# Host tensors are enough here: shape, dtype and layout are checked first, and
# a well-formed call on host tensors is refused for its device, so no call
# ever reaches the library.
import torch  # noqa: E402

BF = torch.bfloat16


def _t(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def _raises(match, fn, *a, **k):
    with pytest.raises(tw.TwellError, match=match):
        fn(*a, **k)


def test_wrapper_gate_pack_checks():
    x, wg = _t(8, 64), _t(256, 64)
    _raises("wg_t: shape", tw.gate_pack, x, _t(256, 128))
    _raises("wg_t: dtype", tw.gate_pack, x, _t(256, 64, dtype=torch.float32))
    _raises("contiguous", tw.gate_pack, x, _t(64, 256).t())          # a transposed view
    _raises("x: expected", tw.gate_pack, _t(8), wg)
    out = tw.empty_twell(9, 256, 32, BF, "cpu")
    _raises("twell.count: shape", tw.gate_pack, x, wg, out=out)      # T mismatch
    out = tw.empty_twell(8, 384, 32, BF, "cpu")
    _raises("d_ff", tw.gate_pack, x, wg, out=out)
    _raises("GPU only", tw.gate_pack, x, wg)                         # right shapes, host memory


def test_wrapper_ffn_fwd_checks():
    x = _t(8, 64)
    t = tw.empty_twell(8, 256, 32, BF, "cpu")
    w = _t(256, 64)
    _raises("wu_t: shape", tw.ffn_fwd, x, t, _t(128, 64), w)
    _raises("wd: shape", tw.ffn_fwd, x, t, w, _t(256, 32))
    _raises("y: shape", tw.ffn_fwd, x, t, w, w, y=torch.zeros(7, 64))
    _raises("y: dtype", tw.ffn_fwd, x, t, w, w, y=_t(8, 64))
    _raises("twell.val: dtype", tw.ffn_fwd, x,
            tw.Twell(t.count, t.col, t.val.float()), w, w)
    _raises("GPU only", tw.ffn_fwd, x, t, w, w)


def test_wrapper_decode_checks():
    x, w = _t(65, 64), _t(256, 64)
    _raises("at most 64", tw.decode_fwd, x, w, w, w)
    _raises("wu_t: shape", tw.decode_fwd, x[:4], w, _t(256, 128), w)
    _raises("GPU only", tw.decode_fwd, x[:4].contiguous(), w, w, w)


def test_wrapper_hybrid_checks():
    T, dff, K, mo = 8, 256, 16, 4
    t = tw.empty_twell(T, dff, 32, BF, "cpu")
    hy = tw.empty_hybrid(T, dff, K, mo, BF, "cpu")
    _raises("K, max_ovf", tw.to_hybrid, t, K + 1, mo, out=hy)
    _raises("hybrid.ell_val: dtype", tw.to_hybrid, t, K, mo,
            out=tw.Hybrid(hy.row_nnz, hy.row_slot, hy.ell_col, hy.ell_val.float(), hy.ovf_rows,
                          hy.dense, hy.n_ovf))
    _raises("GPU only", tw.to_hybrid, t, K, mo, out=hy)
    x, w = _t(T, 64), _t(dff, 64)
    _raises("wu_t: shape", tw.hybrid_fwd, x, hy, _t(dff, 128), w)
    _raises("hybrid.row_nnz: shape", tw.hybrid_fwd, _t(T + 1, 64), hy, w, w)
    _raises("GPU only", tw.hybrid_fwd, x, hy, w, w)
    f = dict(dtype=torch.float32)
    good = (torch.zeros(T, 64, **f),) + tuple(torch.zeros(dff, 64, **f) for _ in range(3))
    _raises("dy: shape", tw.ffn_bwd, x, _t(T, 128), hy, w, w, w)
    _raises("wg_t: shape", tw.ffn_bwd, x, x, hy, _t(dff + 128, 64), w, w)
    _raises("dwd: shape", tw.ffn_bwd, x, x, hy, w, w, w,
            out=good[:3] + (torch.zeros(dff, 32, **f),))
    _raises("dx: dtype", tw.ffn_bwd, x, x, hy, w, w, w, out=(_t(T, 64),) + good[1:])
    _raises("workspace", tw.ffn_bwd, x, x, hy, w, w, w, out=good,
            workspace=torch.zeros(4, dtype=torch.float32))
    _raises("GPU only", tw.ffn_bwd, x, x, hy, w, w, w, out=good)


def test_decode_noalloc_validation(L):
    """The allocation-free decode call checks its arguments as twell_decode_fwd
    does and refuses, on the host, a call needing more than the static
    scratch."""
    f = lambda tt, dm=64, y=FAKE, x=FAKE: L.twell_decode_fwd_noalloc(
        tw.TWELL_BF16, x, FAKE, FAKE, FAKE, dm, ctypes.byref(tt), y, None, None, None)
    assert f(twell_c(), y=0) == -1
    assert f(twell_c(), dm=100) == -2
    assert f(twell_c(T=65)) == -2
    assert f(twell_c(), y=FAKE + 4) == -4
    big = twell_c(T=64, d_ff=32768, width=128)
    assert L.twell_decode_workspace_bytes(tw.TWELL_BF16, 64, 4096, 32768, 128) > tw.STATIC_SCRATCH_BYTES
    for T in (1, 8, 32, 64):   # the 2B decode layer fits
        assert L.twell_decode_workspace_bytes(tw.TWELL_BF16, T, 2304, 6144, 128) <= tw.STATIC_SCRATCH_BYTES
    assert f(big, dm=4096) == -7
    assert b"scratch" in L.twell_status_str(-7)
    assert f(twell_c(T=0, ptr=0), x=0, y=0) == 0   # T == 0: nothing to do
