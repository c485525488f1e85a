"""twell_decode_fwd_noalloc (the decode layer with the library's static
scratch instead of a caller workspace) against twell_decode_fwd, through the
C-ABI: identical TwELL and y, bit for bit, on two calls in a row, the second
with fewer tokens and a narrower layer, and a refusal, launching nothing, of a
call that needs more scratch than the static array holds."""
import ctypes

import pytest
import torch

from activation_sparse_ffn_gemm_amd import _lib as tw
from activation_sparse_ffn_gemm_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(w):
    d = synth.make_inputs(w)
    return [d[k].to(DEV) for k in ("x", "wg_t", "wu_t", "wd")]


def _keep(t, W):
    return torch.arange(W, device=DEV)[None, None, :] < t.count.clamp(max=W)[:, :, None]


def test_noalloc_equals_workspace_call():
    cases = [synth.DECODE_2B.with_(T=64), synth.DECODE_2B.with_(T=3, d_model=1024, d_ff=2048)]
    for w in cases:
        print("[case] noalloc", w.T, w.d_model, w.d_ff, flush=True)
        x, wg, wu, wd = _inputs(w)
        need = tw.decode_workspace_bytes(tw.TWELL_BF16, w.T, w.d_model, w.d_ff, w.width)
        assert 0 < need <= tw.STATIC_SCRATCH_BYTES
        st_a = torch.zeros(1, dtype=torch.int32, device=DEV)
        ta, ya = tw.decode_fwd(x, wg, wu, wd, width=w.width, status=st_a)
        tb = tw.empty_twell(w.T, w.d_ff, w.width, torch.bfloat16, DEV)
        yb = torch.full((w.T, w.d_model), float("nan"), device=DEV)
        st_b = torch.zeros(1, dtype=torch.int32, device=DEV)
        tw.decode_fwd_noalloc(x, wg, wu, wd, tb, yb, status=st_b)
        torch.cuda.synchronize()
        assert int(st_a.item()) == 0 and int(st_b.item()) == 0
        assert torch.equal(ta.count, tb.count)
        k = _keep(ta, w.width)
        assert torch.equal(ta.col[k], tb.col[k])
        assert torch.equal(ta.val[k].view(torch.int16), tb.val[k].view(torch.int16))
        assert torch.equal(ya, yb)
        assert int(ta.count.sum()) > 0


def test_noalloc_refuses_oversized_call():
    """T = 64 over d_model 4096 and d_ff 32768 with 128 slots per tile needs
    16 MiB of scratch, more than the 12 MiB array: refused on the host (nothing launched), through the C-ABI."""
    L = tw.load()
    T, dm, dff, W = 64, 4096, 32768, 128
    assert tw.decode_workspace_bytes(tw.TWELL_BF16, T, dm, dff, W) > tw.STATIC_SCRATCH_BYTES
    x = torch.zeros((T, dm), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((256, dm), dtype=torch.bfloat16, device=DEV)  # never read
    out = tw.empty_twell(T, dff, W, torch.bfloat16, DEV)
    y = torch.zeros((T, dm), device=DEV)
    c = out.c()
    rc = L.twell_decode_fwd_noalloc(tw.TWELL_BF16, x.data_ptr(), w.data_ptr(), w.data_ptr(),
                                    w.data_ptr(), dm, ctypes.byref(c), y.data_ptr(), None, None,
                                    None)
    assert rc == -7
    assert b"scratch" in L.twell_status_str(rc)
