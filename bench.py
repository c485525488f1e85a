"""Benchmark of the activation-sparse ReLU-gated FFN hot path on one MI355X.

One step = one training pass of the whole path over one batch of synthetic
input: twell_gate_pack (gate GEMM + TwELL epilogue) -> twell_to_hybrid ->
hybrid_ffn_fwd (the forward over the hybrid: ELL rows by gathers, backup rows
by dense products) -> hybrid_ffn_bwd (dx, dW_g, dW_u, dW_d for a synthetic
dy). The default workload is the 0.5B-scale layer at 1% gate density
(T = 4096 tokens, d_model = 1024, d_ff = 2816, bf16). Inputs are resident in
HBM before the timed region. Prints one JSON line.

Beside the step it reports: per-stage times (HIP events on the stream the
kernels run on), the roofline of the dominant kernel, the inference forward
(twell_gate_pack -> twell_ffn_fwd) timed on its own, the same layer run dense
in bf16 by torch (forward, and forward + backward), and the CPU oracle timed
on this host (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "0.5b-1pct": dict(T=4096, d_model=1024, d_ff=2816, density=0.01, width=32, K=128,
                      max_ovf=256, skew_frac=0.0, skew_density=0.0),
    "1.5b-1pct": dict(T=8192, d_model=2048, d_ff=5632, density=0.01, width=32, K=128,
                      max_ovf=512, skew_frac=0.0, skew_density=0.0),
    "1.5b-train-skewed": dict(T=8192, d_model=2048, d_ff=5632, density=0.01, width=128, K=128,
                              max_ovf=1024, skew_frac=0.05, skew_density=0.30),
}


# Source files whose text decides each kernel's memory traffic: counters taken
# on other sources describe another kernel and are not reported.
CSRC = os.path.join(ROOT, "activation_sparse_ffn_gemm_amd", "csrc")
KERNEL_SOURCES = {
    "gate_pack_kernel": "gate_pack.hip", "ffn_fwd_kernel": "ffn_fwd.hip",
    "fwd_up_kernel": "ffn_fwd.hip", "fwd_down_kernel": "ffn_fwd.hip",
    "hyb_rows_kernel": "to_hybrid.hip", "hyb_slots_kernel": "to_hybrid.hip",
    "hyb_dense_kernel": "to_hybrid.hip", "hfwd_ell_kernel": "hyb_fwd.hip",
    "hfwd_up_kernel": "ffn_fwd.hip", "hfwd_down_kernel": "ffn_fwd.hip",
    "bk_a_kernel": "backup.hip", "bk_y_kernel": "backup.hip", "bk_ud_kernel": "backup.hip",
    "bk_dxdw_kernel": "backup.hip", "dec_gate_part_kernel": "decode.hip",
    "dec_pack_kernel": "decode.hip", "dec_up_kernel": "decode.hip",
    "dec_down_kernel": "decode.hip",
}


def source_closure(name):
    """The source file and every local header it includes, transitively
    (quoted includes, looked up in csrc/ then include/), sorted."""
    import re
    dirs = (CSRC, os.path.join(ROOT, "include"))
    seen, todo = set(), [name]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        path = next(os.path.join(d, f) for d in dirs if os.path.exists(os.path.join(d, f)))
        with open(path) as fh:
            todo += re.findall(r'^\s*#\s*include\s+"([^"]+)"', fh.read(), re.M)
    return sorted(seen)


def kernel_sources_sha256(kernel):
    """sha256 over the kernel's .hip file and the headers it includes."""
    import hashlib
    h = hashlib.sha256()
    dirs = (CSRC, os.path.join(ROOT, "include"))
    for f in source_closure(KERNEL_SOURCES.get(kernel, "bwd.hip")):
        path = next(os.path.join(d, f) for d in dirs if os.path.exists(os.path.join(d, f)))
        with open(path, "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter
    reads for a plain copy of known size), or None with the reason."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as fh:
        rec = json.load(fh)
    k = rec.get("kernels", {}).get(kernel)
    if rec.get("workload") != workload or k is None:
        return None, "no counters for this kernel and workload"
    if k["sources_sha256"] != kernel_sources_sha256(kernel):
        return None, "kernel sources changed since the counters were taken"
    cal = rec["copy_calibration"]
    sf = cal["bytes"] / (cal["fetch_kib"] * 1024.0)
    sw = cal["bytes"] / (cal["write_kib"] * 1024.0)
    b = k["fetch_kib"] * 1024.0 * sf + k["write_kib"] * 1024.0 * sw
    return round(b), (f"rocprofv3 FETCH_SIZE {k['fetch_kib']:.0f} KiB x {sf:.3f} + WRITE_SIZE "
                      f"{k['write_kib']:.0f} KiB x {sw:.3f} per launch (copy-calibrated)")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="0.5b-1pct", choices=sorted(WORKLOADS))
    p.add_argument("--l1", type=float, default=2e-5,
                   help="weight of the L1 activation penalty in the backward (training recipe)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--no-dense", action="store_true", help="skip the dense torch leg")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the few-token (2B decode) leg")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the 1.5B forward density sweep leg")
    p.add_argument("--copy-calib", action="store_true",
                   help="only run a plain device copy of known size (counter calibration)")
    return p.parse_args()


def graph_us(torch, fn, calls=10, replays=20):
    """Mean microseconds of fn() captured in a HIP graph (calls per graph) and
    replayed: launch gaps on the GPU are included, host overhead is not."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * calls)


def decode_leg(torch, tw, synth, dev):
    """The 2B-scale decode configuration (d_model 2304, d_ff 6144, 1%, W = 32)
    at T = 1, 8, 32, 64 tokens: twell_decode_fwd (the whole layer) against the
    dense bf16 layer, both graph-timed, and the weight bytes actually touched
    (W_g whole, plus one wu_t and one wd row per distinct active neuron)."""
    rows = []
    for T in (1, 8, 32, 64):
        w = synth.DECODE_2B.with_(T=T)
        d = synth.make_inputs(w)
        x, wg, wu, wd = (d[k].to(dev) for k in ("x", "wg_t", "wu_t", "wd"))
        out = tw.empty_twell(T, w.d_ff, w.width, torch.bfloat16, dev)
        y = torch.empty((T, w.d_model), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, tw.decode_workspace_bytes(tw.TWELL_BF16, T, w.d_model, w.d_ff,
                                                            w.width)),
                         dtype=torch.uint8, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        sparse = lambda: tw.decode_fwd(x, wg, wu, wd, width=w.width, out=out, y=y, workspace=ws,
                                       status=st)
        sp_us = graph_us(torch, sparse)
        if int(st.item()) != 0:
            raise SystemExit(f"decode T={T}: device status {int(st.item())}")
        gu_t = torch.cat([wg, wu], 0).t().contiguous()
        wd_c = wd.contiguous()
        dff = w.d_ff

        def dense():
            gu = x @ gu_t
            return (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ wd_c
        de_us = graph_us(torch, dense)
        keep = torch.arange(w.width, device=dev)[None, None, :] < out.count.clamp(max=w.width)[:, :, None]
        distinct = int(torch.unique(out.col[keep].long()).numel())
        touched = dff * w.d_model * 2 + distinct * 2 * w.d_model * 2
        rows.append({"T": T, "sparse_us": round(sp_us, 2), "dense_us": round(de_us, 2),
                     "speedup": round(de_us / sp_us, 3), "weight_bytes_touched": touched,
                     "touched_GBps": round(touched / (sp_us * 1e-6) / 1e9, 1),
                     "nnz": int(out.count.clamp(max=w.width).sum())})
    return {"workload": "2b-decode", "d_model": 2304, "d_ff": 6144, "density": 0.01,
            "width": 32, "call": "twell_decode_fwd (gate partials, pack + up, down: 3 launches)",
            "timing": "HIP graph of 10 calls, replayed 20 times", "by_T": rows}


def sweep_leg(torch, tw, synth, dev):
    """The 1.5B-scale forward (T 8192, d_model 2048, d_ff 5632) at gate
    densities 0.5, 1, 2, 5 and 20%: gate GEMM + TwELL pack, then the fused
    up/down, against the dense bf16 forward of the same shape, both
    graph-timed. The TwELL width is 32 slots per tile up to 5% and 64 at 20%
    (about 26 nonzeros per 128-column tile there)."""
    rows = []
    for dens in synth.SWEEP_1P5B:
        w = synth.sweep_workload(dens)
        width = w.width
        d = synth.make_inputs(w)
        x, wg, wu, wd = (d[k].to(dev) for k in ("x", "wg_t", "wu_t", "wd"))
        del d
        T, dm, dff = w.T, w.d_model, w.d_ff
        out = tw.empty_twell(T, dff, width, torch.bfloat16, dev)
        y = torch.empty((T, dm), dtype=torch.float32, device=dev)
        gws = torch.empty(max(1, tw.gate_workspace_bytes(tw.TWELL_BF16, T, dm, dff)),
                          dtype=torch.uint8, device=dev)
        fws = torch.empty(max(1, tw.fwd_workspace_bytes(tw.TWELL_BF16, T, dm, dff, width)),
                          dtype=torch.uint8, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)

        def sparse():
            tw.gate_pack(x, wg, width=width, out=out, status=st, workspace=gws)
            tw.ffn_fwd(x, out, wu, wd, y=y, workspace=fws, status=st)
        sp_us = graph_us(torch, sparse, calls=4, replays=10)
        if int(st.item()) != 0:
            raise SystemExit(f"sweep density {dens}: device status {int(st.item())}")
        nnz = int(out.count.clamp(max=width).sum())
        # per-kernel times: the same calls with events between the kernels
        tms = (tw.KernelTimer(), tw.KernelTimer())
        kern = {}
        for _ in range(5):
            tw.gate_pack(x, wg, width=width, out=out, status=st, workspace=gws, timing=tms[0])
            tw.ffn_fwd(x, out, wu, wd, y=y, workspace=fws, status=st, timing=tms[1])
            torch.cuda.synchronize()
            for tm in tms:
                for name, ms in tm.collect():
                    kern[name] = kern.get(name, 0.0) + ms * 1e3 / 5
        gu_t = torch.cat([wg, wu], 0).t().contiguous()
        wd_c = wd.contiguous()

        def dense():
            gu = x @ gu_t
            return (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ wd_c
        de_us = graph_us(torch, dense, calls=4, replays=10)
        rows.append({"density": dens, "measured_density": round(nnz / (T * dff), 5),
                     "width": width, "sparse_us": round(sp_us, 1), "dense_us": round(de_us, 1),
                     "sparse_tokens_per_s": round(T / (sp_us * 1e-6), 1),
                     "dense_tokens_per_s": round(T / (de_us * 1e-6), 1),
                     "speedup": round(de_us / sp_us, 3),
                     "kernel_us": {k: round(v, 1) for k, v in kern.items()}})
        del x, wg, wu, wd, out, y, gws, fws, gu_t, wd_c
        torch.cuda.empty_cache()
    return {"workload": "1.5b-fwd", "T": 8192, "d_model": 2048, "d_ff": 5632,
            "call": "twell_gate_pack + twell_ffn_fwd (inference forward)",
            "timing": "HIP graph of 4 calls, replayed 10 times", "by_density": rows}


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "libtwell runs on one GPU only; the layer is not sharded "
                                   "across GPUs (bench.py --gpus 1)"}), flush=True)
        sys.exit(2)
    import torch

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if a.copy_calib:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    from activation_sparse_ffn_gemm_amd import _lib as tw
    from activation_sparse_ffn_gemm_amd import synth

    cfg = WORKLOADS[a.workload]
    w = synth.Workload(a.workload, cfg["T"], cfg["d_model"], cfg["d_ff"], "bf16", cfg["density"],
                       skew_frac=cfg["skew_frac"], skew_density=cfg["skew_density"],
                       K=cfg["K"], max_ovf=cfg["max_ovf"], width=cfg["width"])
    d = synth.make_inputs(w, with_dy=True)
    x, wg, wu, wd, dy = (d[k].to(dev) for k in ("x", "wg_t", "wu_t", "wd", "dy"))
    T, dm, dff = w.T, w.d_model, w.d_ff

    # preallocated outputs and workspaces: the timed region allocates nothing
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    twl = tw.empty_twell(T, dff, w.width, torch.bfloat16, dev)
    y = torch.empty((T, dm), dtype=torch.float32, device=dev)
    fws_n = tw.fwd_workspace_bytes(tw.TWELL_BF16, T, dm, dff, w.width)
    fws = torch.empty(max(fws_n, 1), dtype=torch.uint8, device=dev)
    hfws_n = tw.hybrid_fwd_workspace_bytes(tw.TWELL_BF16, T, dm, dff, w.K, w.max_ovf)
    hfws = torch.empty(max(hfws_n, 1), dtype=torch.uint8, device=dev)
    hy = tw.empty_hybrid(T, dff, w.K, w.max_ovf, torch.bfloat16, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    grads = (torch.empty((T, dm), **f32), torch.empty((dff, dm), **f32),
             torch.empty((dff, dm), **f32), torch.empty((dff, dm), **f32))
    bws = torch.empty(tw.bwd_workspace_bytes(tw.TWELL_BF16, T, dm, dff, w.K, w.max_ovf),
                      dtype=torch.uint8, device=dev)

    stages = ("gate_pack", "to_hybrid", "hybrid_fwd", "bwd")
    timers = {k: tw.KernelTimer() for k in stages}

    def step(timed=False):
        tm = timers if timed else {k: None for k in stages}
        tw.gate_pack(x, wg, width=w.width, out=twl, status=st, timing=tm["gate_pack"])
        tw.to_hybrid(twl, w.K, w.max_ovf, out=hy, status=st, timing=tm["to_hybrid"])
        tw.hybrid_fwd(x, hy, wu, wd, y=y, workspace=hfws, status=st, timing=tm["hybrid_fwd"])
        tw.ffn_bwd(x, dy, hy, wg, wu, wd, out=grads, workspace=bws, status=st,
                   timing=tm["bwd"], l1=a.l1)

    ftimers = {k: tw.KernelTimer() for k in ("gate_pack", "ffn_fwd")}

    def fwd_step(timed=False):
        tm = ftimers if timed else {k: None for k in ftimers}
        tw.gate_pack(x, wg, width=w.width, out=twl, status=st, timing=tm["gate_pack"])
        tw.ffn_fwd(x, twl, wu, wd, y=y, workspace=fws, status=st, timing=tm["ffn_fwd"])

    for _ in range(a.warmup):
        step()
        fwd_step()
    torch.cuda.synchronize()
    if int(st.item()) != 0:
        raise SystemExit(f"device status {int(st.item())}: a TwELL tile or the backup overflowed")
    nnz = int(torch.minimum(twl.count, torch.tensor(w.width, device=dev)).sum())
    n_ovf = int(hy.n_ovf.item())
    ell_rows = hy.row_slot < 0
    nnz_ell = int(hy.row_nnz[ell_rows].sum())

    # timed region: K steps back to back, bracketed by synchronisation; the
    # first and last of each call's events bracket the whole step
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record()
    for _ in range(a.steps):
        step()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e_start.elapsed_time(e_end) / a.steps

    # per-kernel durations: the same steps again, each call with its events
    kern_ms, stage_ms = {}, {k: 0.0 for k in stages}
    for _ in range(a.steps):
        step(timed=True)
        torch.cuda.synchronize()
        for k in stages:
            for name, ms in timers[k].collect():
                kern_ms[name] = kern_ms.get(name, 0.0) + ms / a.steps
                stage_ms[k] += ms / a.steps

    # inference forward on its own: gate + TwELL pack, fused up/down
    torch.cuda.synchronize()
    e_start.record()
    for _ in range(a.steps):
        fwd_step()
    e_end.record()
    torch.cuda.synchronize()
    inf_ms = e_start.elapsed_time(e_end) / a.steps
    fwd_kern = {}
    for _ in range(a.steps):
        fwd_step(timed=True)
        torch.cuda.synchronize()
        for k in ftimers:
            for name, ms in ftimers[k].collect():
                fwd_kern[name] = fwd_kern.get(name, 0.0) + ms / a.steps

    # ---- roofline of each kernel: algorithmic work of one launch. Bytes count
    # every row a kernel's algorithm reads (a gathered row once per use, as
    # the gather performs it), the index/value arrays it reads and what it
    # writes; flops count the dense contractions' 2 m n k.
    n_t = dff // 128
    nblk = (T + 63) // 64                        # 64-row blocks of the CSC masks
    dx_split = T >= 1024 and dff * dm * 2 >= (16 << 20)  # the backward's XCD-local dx pass
    row_b = dm * 2                               # one bf16 row of d_model
    T_ell = T - n_ovf
    twell_b = T * n_t * 4 + nnz * 4              # count + (int16 col, bf16 val) per entry
    work = {
        "gate_pack_kernel": ("mfma", 2.0 * T * dm * dff,
                             "2 d_model d_ff flop per token (TwELL written in the epilogue)"),
        "ffn_fwd_kernel": ("hbm", nnz * 2 * row_b + T * row_b + T * dm * 4 + twell_b,
                           "per nonzero one wu_t row + one wd row; x, y, TwELL once"),
        "fwd_up_kernel": ("hbm", nnz * row_b + T * row_b + twell_b + 2 * dff * row_b + nnz * 6,
                          "per nonzero one wu_t row; x, TwELL once; wd slice-major copy "
                          "(read + write); a and column per nonzero written"),
        "fwd_down_kernel": ("hbm", nnz * row_b + nnz * 6 + T * dm * 4,
                            "per nonzero one wd row (as 8 slices); a and column per nonzero; y"),
        "hyb_rows_kernel": ("hbm", T * n_t * 4 + nnz_ell * 8 + 4 * T,
                            "TwELL counts + ELL rows' entries read; ELL entries, row_nnz written"),
        "hyb_dense_kernel": ("hbm", n_ovf * n_t * (4 + 128 * 4) + n_ovf * dff * 2 + 8 * T,
                             "backup rows' TwELL tiles read, dense backup, row_slot written"),
        "bwd_neuron_kernel": ("hbm", nnz_ell * (2 * row_b + 4 + 2 + 8) + dff * (2 * row_b + 3 * dm * 4),
                              "per ELL nonzero one x row + one dy row + CSC slot, h, du/dg; "
                              "per neuron wu_t + wd rows and three fp32 dW rows"),
        "bwd_dx_kernel": ("hbm", nnz_ell * (2 * row_b + 10) + 8 * T + T_ell * dm * 4,
                          "per ELL nonzero one wu_t row + one wg_t row + col, du, dg; dx rows"),
        "bwd_dxs_kernel": ("hbm", nnz_ell * (2 * row_b + 10) + 8 * T + T_ell * dm * 4,
                           "per ELL nonzero one wu_t row + one wg_t row (as 8 slices each) + col, "
                           "du, dg; dx rows"),
        "hfwd_ell_kernel": ("hbm", nnz_ell * (2 * row_b + 4) + T_ell * (row_b + dm * 4),
                            "per ELL nonzero one wu_t row + one wd row + (col, h); x, y rows"),
        "hfwd_up_kernel": ("hbm", nnz_ell * (row_b + 8) + T_ell * row_b + 2 * dff * row_b,
                           "per ELL nonzero one wu_t row + (col, h) + a written; x rows; wd "
                           "slice-major copy (read + write)"),
        "hfwd_down_kernel": ("hbm", nnz_ell * (row_b + 6) + T_ell * dm * 4,
                             "per ELL nonzero one wd row (as 8 slices) + (col, a); y rows"),
        "bk_a_kernel": ("mfma", 2.0 * n_ovf * dm * dff, "A = h_O (.) x_O W_u (1 GEMM)"),
        "bk_y_kernel": ("mfma", 2.0 * n_ovf * dm * dff, "y_O = A W_d (1 GEMM)"),
        "bk_ud_kernel": ("mfma", 2 * 2.0 * n_ovf * dm * dff, "u_O and da_O (2 GEMMs)"),
        "bk_dxdw_kernel": ("mfma", 5 * 2.0 * n_ovf * dm * dff,
                           "dx_O = du W_u^T + dg W_g^T (2 GEMMs) and dW_d, dW_u, dW_g += "
                           "(3 GEMMs)"),
        "mask_kernel": ("hbm", 8 * T + nnz_ell * 2 + nblk * dff * 12
                        + (4 * dff * row_b if dx_split else 0)
                        + (4 * dff * row_b + 4 * n_ovf * row_b if n_ovf > 0 else 0),
                        "row_nnz, row_slot per row, column per ELL entry read; 64-row block "
                        "mask and count per neuron written; on the same launch the slice-major "
                        "wu_t, wg_t copy (XCD-local dx) and the backup's transposed W_u, W_g, "
                        "x_O, dy_O (read + write)"),
        "blk_prefix_kernel": ("hbm", nblk * dff * 12 + dff * 4,
                              "block counts read twice and rewritten as prefixes; totals"),
        "colptr_kernel": ("hbm", dff * 8 + 4, "neuron totals read, column pointers written"),
        "csc_fill_kernel": ("hbm", 8 * T + nnz_ell * 22,
                            "per ELL entry: column, mask, block prefix, column pointer read, "
                            "slot written"),
    }
    peak = {"mfma": BF16_PEAK_TFLOPS, "hbm": HBM_PEAK_GBS}
    unit = {"mfma": "TFLOP/s", "hbm": "GB/s"}
    scale = {"mfma": 1e12, "hbm": 1e9}
    def entries(kms):
        res = {}
        for name, ms in kms.items():
            ent = {"ms": round(ms, 4)}
            if name in work and work[name][1] > 0:
                b, wk, desc = work[name]
                ach = wk / (ms * 1e-3) / scale[b]
                ent.update(bound=b, achieved=round(ach, 1), unit=unit[b],
                           frac=round(ach / peak[b], 4), work=wk, work_unit=desc)
            res[name] = ent
        return res

    per_kernel = entries(kern_ms)
    dom = max((k for k in kern_ms if k in work and work[k][1] > 0), key=lambda k: kern_ms[k])
    b, wk, desc = work[dom]
    ach = wk / (kern_ms[dom] * 1e-3) / scale[b]
    traffic, traffic_note = measured_traffic(dom, a.workload)
    roofline = {"kernel": dom, "bound": b, "achieved": round(ach, 1), "peak": peak[b],
                "unit": unit[b], "frac": round(ach / peak[b], 4), "traffic": traffic,
                "traffic_note": traffic_note,
                "note": ("algorithmic bytes count every gathered row once per use; rows served "
                         "again from L2 or the MALL let them run above the HBM peak, and "
                         "traffic (HBM-side bytes from the counters) is then below them"
                         if b == "hbm" else "algorithmic flops of the dense contraction"),
                "launch_ms": round(kern_ms[dom], 4),
                "work_per_launch": wk, "work_unit": desc}

    # ---- layer memory: what the sparse path keeps between forward and backward
    # (the hybrid; the TwELL is dropped once converted) and what it needs at
    # its peak (TwELL + hybrid + workspaces), against the dense layer's below
    nbytes = lambda *ts: sum(t.numel() * t.element_size() for t in ts)
    hy_b = nbytes(hy.row_nnz, hy.row_slot, hy.ell_col, hy.ell_val, hy.ovf_rows, hy.dense,
                  hy.n_ovf)
    tw_b = nbytes(twl.count, twl.col, twl.val)
    memory = {"hybrid_bytes": hy_b, "twell_bytes": tw_b, "fwd_workspace_bytes": hfws_n,
              "bwd_workspace_bytes": bws.numel(),
              "sparse_saved_activation_bytes": hy_b,
              "sparse_step_peak_bytes": tw_b + hy_b + max(hfws_n, bws.numel()),
              "note": "activation memory only; x, dy, weights, y and gradients are the same "
                      "for both layers"}

    # ---- dense bf16 layer, same shapes, torch (hipBLASLt) as a timed black box
    dense = None
    if not a.no_dense:
        wgu_t = torch.cat([wg, wu], 0).t().contiguous()  # [d_model][2 d_ff]
        wd_c = wd.contiguous()

        def dense_fwd(xx):
            gu = xx @ wgu_t
            return (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ wd_c

        p_gu = wgu_t.clone().requires_grad_(True)
        p_d = wd_c.clone().requires_grad_(True)
        xr = x.clone().requires_grad_(True)

        def dense_train():
            gu = xr @ p_gu
            yy = (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ p_d
            yy.backward(dy)

        def timeit(fn, n):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / n

        with torch.no_grad():
            fwd_ms = timeit(lambda: dense_fwd(x), a.steps)
        train_ms = timeit(dense_train, a.steps)
        # activation memory of the dense layer: what autograd keeps between
        # forward and backward, and the step's peak above the resident inputs
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        gu = xr @ p_gu
        yy = (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ p_d
        torch.cuda.synchronize()
        dense_saved = torch.cuda.memory_allocated() - base - yy.numel() * yy.element_size()
        yy.backward(dy)
        torch.cuda.synchronize()
        dense_peak = torch.cuda.max_memory_allocated() - base
        del gu, yy
        dense = {"fwd_tokens_per_s": round(T / (fwd_ms * 1e-3), 1), "fwd_ms": round(fwd_ms, 4),
                 "train_tokens_per_s": round(T / (train_ms * 1e-3), 1),
                 "train_ms": round(train_ms, 4),
                 "train_tflops": round(9 * 2.0 * T * dm * dff / (train_ms * 1e-3) / 1e12, 1),
                 "saved_activation_bytes": int(dense_saved), "step_peak_bytes": int(dense_peak)}
        del p_gu, p_d, xr

    decode = None if a.no_decode else decode_leg(torch, tw, synth, dev)
    sweep = None if a.no_sweep else sweep_leg(torch, tw, synth, dev)

    # ---- CPU oracle on this host (bounded sample of the same workload)
    cpu = None
    if not a.no_cpu:
        import numpy as np
        from oracle import oracle as orc
        f64 = lambda t: t.double().numpy()
        X, WG, WU, WD, DY = (f64(d[k]) for k in ("x", "wg_t", "wu_t", "wd", "dy"))
        Ts = T
        reps, toks, el = 0, 0, 0.0
        while el < 10.0 and reps < 50:
            t1 = time.perf_counter()
            g = orc.gate(X[:Ts], WG)
            tws = orc.twell_pack(g, W=w.width)
            tws["val"] = f64(torch.from_numpy(tws["val"]).to(torch.bfloat16))
            orc.ffn_twell(X[:Ts], tws, WU, WD)
            hys = orc.to_hybrid(tws, w.K, w.max_ovf)
            orc.bwd_hybrid(X[:Ts], DY[:Ts], hys, WG, WU, WD, l1=a.l1)
            el += time.perf_counter() - t1
            toks += Ts
            reps += 1
        cpu = {"value": round(toks / el, 1), "unit": "tokens/s", "cores": orc.num_threads(),
               "kind": "oracle",
               "sample": f"{reps} x the full step (gate, TwELL pack, sparse up/down, hybrid, "
                         f"backward) over all {Ts} tokens of the batch, float64, {el:.1f} s"}

    out = {
        "metric": "FFN-layer tokens/s at 1% gate density vs dense bf16; % MFMA/HBM peak",
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian inputs and weights, gate offset "
                                 "for the target density)",
        "config": {"workload": a.workload, "step": "gate GEMM + TwELL pack, TwELL->hybrid, "
                   "forward over the hybrid, hybrid backward (dx, dW_g, dW_u, dW_d)", "T": T,
                   "d_model": dm, "d_ff": dff,
                   "density": w.density, "measured_density": round(nnz / (T * dff), 5),
                   "nnz": nnz, "nnz_ell": nnz_ell, "n_ovf": n_ovf, "twell_width": w.width,
                   "K": w.K, "max_ovf": w.max_ovf, "l1": a.l1},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "forward": {"step": "gate GEMM + TwELL pack, fused up/down over the TwELL",
                    "ms": round(inf_ms, 4), "tokens_per_s": round(T / (inf_ms * 1e-3), 1),
                    "kernels": entries(fwd_kern)},
        "roofline": roofline,
        "kernels": per_kernel,
        "dense_bf16": dense,
        "memory": memory,
        "decode": decode,
        "density_sweep": sweep,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
