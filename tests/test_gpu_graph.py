"""The library neither allocates nor synchronises, so a whole training step
(gate + pack, TwELL -> hybrid, forward over the hybrid, backward) can be
captured in a HIP graph. Each replay, with the program's own eager work and
synchronisations between replays, must reproduce the eager step bit for bit."""
import pytest
import torch

from activation_sparse_ffn_gemm_amd import _lib as tw
from activation_sparse_ffn_gemm_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("w", [
    synth.Workload("graph-skewed", 512, 256, 768, "bf16", 0.02, skew_frac=0.05, skew_density=0.3,
                   K=40, max_ovf=64, width=128),
    # 1029 tokens and 16 MB weights: the XCD-split forward, whose backup
    # products run on a second stream when called eagerly and in order on the
    # captured stream, so replays check the two orders agree bit for bit
    synth.Workload("graph-split", 1029, 2048, 4096, "bf16", 0.01, skew_frac=0.05,
                   skew_density=0.3, K=128, max_ovf=128, width=128),
    synth.DECODE_2B.with_(T=8),
], ids=lambda w: w.name)
def test_step_graph_replays_equal_eager(w):
    print("[case] graph", w.name, flush=True)
    d = synth.make_inputs(w, with_dy=True)
    x, wg, wu, wd, dy = (d[k].to(DEV) for k in ("x", "wg_t", "wu_t", "wd", "dy"))
    T, dm, dff = w.T, w.d_model, w.d_ff
    K, mo = (w.K or 128), (w.max_ovf or 16)
    bf = torch.bfloat16
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    twl = tw.empty_twell(T, dff, w.width, bf, DEV)
    hy = tw.empty_hybrid(T, dff, K, mo, bf, DEV)
    y = torch.empty((T, dm), dtype=torch.float32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    grads = tuple(torch.empty(s, **f32) for s in ((T, dm), (dff, dm), (dff, dm), (dff, dm)))
    u8 = dict(dtype=torch.uint8, device=DEV)
    gws = torch.empty(max(1, tw.gate_workspace_bytes(tw.TWELL_BF16, T, dm, dff)), **u8)
    hws = torch.empty(max(1, tw.hybrid_fwd_workspace_bytes(tw.TWELL_BF16, T, dm, dff, K, mo)), **u8)
    bws = torch.empty(tw.bwd_workspace_bytes(tw.TWELL_BF16, T, dm, dff, K, mo), **u8)

    def step():
        tw.gate_pack(x, wg, width=w.width, out=twl, status=st, workspace=gws)
        tw.to_hybrid(twl, K, mo, out=hy, status=st)
        tw.hybrid_fwd(x, hy, wu, wd, y=y, workspace=hws, status=st)
        tw.ffn_bwd(x, dy, hy, wg, wu, wd, out=grads, workspace=bws, status=st, l1=2e-5)

    step()
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref = [y.clone()] + [g.clone() for g in grads]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(4):
        for t in [y, *grads]:
            t.fill_(-1.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip([y, *grads], ref):
            assert torch.equal(a, b)
    assert int(st.item()) == 0
