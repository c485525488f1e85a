"""Benchmark of the activation-sparse ReLU-gated FFN hot path on one MI355X.

The headline step is the 1.5B-scale inference forward at 1% gate density
(T = 8192 tokens, d_model = 2048, d_ff = 5632, bf16): twell_gate_pack (gate
GEMM with the TwELL packing in its epilogue) then twell_ffn_fwd (the fused
up/down projections over the TwELL nonzeros). Inputs are resident in HBM
before the timed region. Prints one JSON line.

Beside the headline it reports, each under its own key:
  kernels / roofline  per-kernel HIP-event times on the stream the kernels run
                      on, with each kernel's algorithmic work and its fraction
                      of the MI355X roofline that bounds it;
  dense_bf16          the same layer run dense in bf16 by torch (hipBLASLt),
                      and the gate GEMM alone (x W_g written out as g);
  training_skewed     the 1.5B training layer with skewed rows (95% at 1%,
                      5% at 30%, 410 backup rows): gate + pack -> TwELL to
                      hybrid -> forward over the hybrid -> hybrid backward,
                      against torch autograd of the dense layer; per-kernel
                      rooflines and the layer's memory, both sides measured
                      with torch's allocator;
  fwd_0p5b, train_0p5b  the 0.5B-scale layer (T 4096, 1024 -> 2816, 1%);
  cold                the forward's gather kernels and the decode layer with
                      a 512 MB scratch write before every call (MALL and L2
                      flushed);
  decode              the 2B-scale few-token layer (T = 1, 8, 32, 64);
  density_sweep       the 1.5B forward at gate densities 0.5 .. 20%;
  cpu_baseline        the float64 CPU oracle timed on this host.
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
FLUSH_BYTES = 512 << 20
SETTLE_S = 0.3  # seconds of untimed steps before the warmup (clock ramp)

METRIC = "FFN-layer tokens/s at 1% gate density vs dense bf16; % MFMA/HBM peak"


def workloads(synth):
    """Named workloads: the forward ones time gate_pack + ffn_fwd, the
    training ones the whole training step."""
    return {
        "1.5b-fwd-1pct": (synth.SCALE_1P5B, "fwd"),
        "0.5b-fwd-1pct": (synth.SCALE_0P5B, "fwd"),
        "1.5b-train-skewed": (synth.TRAIN_1P5B, "train"),
        "0.5b-train-1pct": (synth.SCALE_0P5B.with_(name="0.5b-train-1pct", K=128,
                                                    max_ovf=256), "train"),
    }


# Source files whose text decides each kernel's memory traffic: counters taken
# on other sources describe another kernel and are not reported.
CSRC = os.path.join(ROOT, "activation_sparse_ffn_gemm_amd", "csrc")
KERNEL_SOURCES = {
    "gate_pack_kernel": "gate_pack.hip", "ffn_fwd_kernel": "ffn_fwd.hip",
    "fwd_up_kernel": "ffn_fwd.hip", "fwd_down_kernel": "ffn_fwd.hip",
    "hyb_rows_kernel": "to_hybrid.hip", "hyb_backup_kernel": "to_hybrid.hip",
    "hfwd_ell_kernel": "hyb_fwd.hip",
    "hfwd_up_kernel": "ffn_fwd.hip", "hfwd_down_kernel": "ffn_fwd.hip",
    "bk_a_kernel": "backup.hip", "bk_y_kernel": "backup.hip", "bk_out_kernel": "backup.hip",
    "prefix_ud_kernel": "bwd.hip",
    "fill_dxdw_kernel": "bwd.hip", "dec_gate_mm_kernel": "decode.hip",
    "dec_pack_kernel": "decode.hip", "dec_up_kernel": "decode.hip",
    "dec_down_kernel": "decode.hip", "dec_gate_gemv_kernel": "decode.hip",
    "dec_pack_up_kernel": "decode.hip",
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
    """Bytes below L2 (MALL or HBM) per launch of `kernel` on `workload` from
    the committed counter summary (rocprofv3 read requests counted by size,
    plus WRITE_SIZE; both exact on a plain copy of known size), or None with
    the reason."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as fh:
        rec = json.load(fh)
    k = rec.get("workloads", {}).get(workload, {}).get(kernel)
    if k is None:
        return None, "no counters for this kernel and workload"
    if k["sources_sha256"] != kernel_sources_sha256(kernel):
        return None, "kernel sources changed since the counters were taken"
    b = k["read_bytes"] + k["write_kib"] * 1024.0
    return round(b), (f"rocprofv3 per launch: read requests by size (32/64/128 B) = "
                      f"{k['read_bytes'] / 1e6:.1f} MB, WRITE_SIZE {k['write_kib']:.0f} KiB")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="1.5b-fwd-1pct",
                   choices=("1.5b-fwd-1pct", "0.5b-fwd-1pct", "1.5b-train-skewed",
                            "0.5b-train-1pct"))
    p.add_argument("--l1", type=float, default=2e-5,
                   help="weight of the L1 activation penalty in the training backward")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    p.add_argument("--no-dense", action="store_true", help="skip the dense torch legs")
    p.add_argument("--no-train", action="store_true", help="skip the skewed training leg")
    p.add_argument("--no-small", action="store_true", help="skip the 0.5B legs")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-cache leg")
    p.add_argument("--no-decode", action="store_true", help="skip the 2B decode leg")
    p.add_argument("--no-sweep", action="store_true", help="skip the density sweep leg")
    p.add_argument("--no-tiny", action="store_true", help="skip the tiny float32 leg")
    p.add_argument("--only", action="store_true",
                   help="the headline step alone (every other leg skipped)")
    p.add_argument("--copy-calib", action="store_true",
                   help="only run a plain device copy of known size (counter calibration)")
    a = p.parse_args()
    if a.only:
        a.no_cpu = a.no_dense = a.no_train = a.no_small = a.no_cold = True
        a.no_decode = a.no_sweep = a.no_tiny = True
    return a


# ----------------------------------------------------------------- timing
def event_ms(torch, fn, n):
    """Mean ms of n back-to-back calls of fn, HIP events on the current stream."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


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


def kernel_ms(torch, tw, calls, n):
    """Mean per-kernel ms of n runs of `calls`, a list of functions that each
    take a KernelTimer and make one library call (events between kernels).
    The n runs go back to back with one synchronisation at the end (a
    synchronisation after every run would idle the GPU between runs and let
    its clocks drop)."""
    timers = [[tw.KernelTimer() for _ in calls] for _ in range(n)]
    t0 = time.perf_counter()  # making the timers idled the GPU: let the clocks ramp again
    while time.perf_counter() - t0 < 0.1:
        for _ in range(5):
            for c in calls:
                c(None)
        torch.cuda.synchronize()
    for run in timers:
        for c, tm in zip(calls, run):
            c(tm)
    torch.cuda.synchronize()
    out = {}
    for run in timers:
        for tm in run:
            for name, ms in tm.collect():
                out[name] = out.get(name, 0.0) + ms / n
    return out


# ----------------------------------------------------------------- roofline
def kernel_work(ctx):
    """Algorithmic work of one launch of each kernel on a workload: bytes count
    every row a kernel's algorithm reads (a gathered row once per use, as the
    gather performs it), the index/value arrays it reads and what it writes;
    flops count the dense contractions' 2 m n k."""
    T, dm, dff, esz = ctx["T"], ctx["d_model"], ctx["d_ff"], ctx["esz"]
    nnz, nnz_ell, n_ovf = ctx["nnz"], ctx.get("nnz_ell", 0), ctx.get("n_ovf", 0)
    n_t = dff // 128
    nblk = (T + 63) // 64
    dx_split = T >= 1024 and dff * dm * esz >= (16 << 20)
    # the forward's down pass reads wd's XCD slices in place when they are runs
    # of whole 128-byte lines (a row of 256 k words); otherwise the up pass
    # copies wd into a slice-major array first
    ndw = dm * esz // 4
    wd_copy = 0 if ndw % 256 == 0 else 2 * dff * dm * esz
    copy_note = "" if wd_copy == 0 else "; wd slice-major copy (read + write)"
    row_b = dm * esz
    T_ell = T - n_ovf
    twell_b = T * n_t * 4 + nnz * (2 + esz)
    return {
        "gate_pack_kernel": ("mfma", 2.0 * T * dm * dff,
                             "2 d_model d_ff flop per token (TwELL written in the epilogue)"),
        "ffn_fwd_kernel": ("hbm", nnz * 2 * row_b + T * row_b + T * dm * 4 + twell_b,
                           "per nonzero one wu_t row + one wd row; x, y, TwELL once"),
        "fwd_up_kernel": ("hbm", nnz * row_b + T * row_b + twell_b + wd_copy + nnz * 6,
                          "per nonzero one wu_t row; x, TwELL once; a and column per nonzero "
                          "written" + copy_note),
        "fwd_down_kernel": ("hbm", nnz * row_b + nnz * 6 + T * dm * 4,
                            "per nonzero one wd row (as 8 slices); a and column per nonzero; y"),
        "hyb_rows_kernel": ("hbm", T * n_t * 4 + nnz_ell * 8 + 4 * T,
                            "TwELL counts + ELL rows' entries read; ELL entries, row_nnz written"),
        "hyb_backup_kernel": ("hbm", 8 * T + 4 * n_ovf
                              + n_ovf * n_t * (4 + ctx.get("W", 128) * (2 + esz))
                              + n_ovf * dff * esz,
                              "row_nnz read, row_slot and the backup rows' ids written; the "
                              "backup rows' TwELL tiles (counts and every slot) read, dense "
                              "backup rows written"),
        "bwd_neuron_kernel": ("hbm", nnz_ell * (2 * row_b + 4 + 2 + 8)
                              + dff * (2 * row_b + 3 * dm * 4),
                              "per ELL nonzero one x row + one dy row + CSC slot, h, du/dg; "
                              "per neuron wu_t + wd rows and three fp32 dW rows"),
        "bwd_dx_kernel": ("hbm", nnz_ell * (2 * row_b + 10) + 8 * T + T_ell * dm * 4,
                          "per ELL nonzero one wu_t row + one wg_t row + col, du, dg; dx rows"),
        "bwd_dxs_kernel": ("hbm", nnz_ell * (2 * row_b + 10) + 8 * T + T_ell * dm * 4,
                           "per ELL nonzero one wu_t row + one wg_t row (as 8 slices each) + "
                           "col, du, dg; dx rows"),
        "hfwd_ell_kernel": ("hbm", nnz_ell * (2 * row_b + 4) + T_ell * (row_b + dm * 4),
                            "per ELL nonzero one wu_t row + one wd row + (col, h); x, y rows"),
        "hfwd_up_kernel": ("hbm", nnz_ell * (row_b + 8) + T_ell * row_b + wd_copy,
                           "per ELL nonzero one wu_t row + (col, h) + a written; x rows"
                           + copy_note),
        "hfwd_down_kernel": ("hbm", nnz_ell * (row_b + 6) + T_ell * dm * 4,
                             "per ELL nonzero one wd row (as 8 slices) + (col, a); y rows"),
        "bk_a_kernel": ("mfma", 2.0 * n_ovf * dm * dff, "A = h_O (.) x_O W_u (1 GEMM)"),
        "bk_y_kernel": ("mfma", 2.0 * n_ovf * dm * dff, "y_O = A W_d (1 GEMM)"),
        "bk_out_kernel": ("hbm", n_ovf * dm * 4 * (ctx.get("S_y", 1) + 1) + 8 * n_ovf,
                          "per backup row its S_y float32 partials of y_O read, its y row "
                          "written"),
        # the backward's backup products ride on the ELL scans' and fill's
        # launches: with backup rows the products dominate those launches
        "prefix_ud_kernel": (("mfma", 2 * 2.0 * n_ovf * dm * dff,
                              "u_O and da_O (2 GEMMs); the ELL block scans share the launch")
                             if n_ovf > 0 else
                             ("hbm", nblk * dff * 12 + dff * 4 + dff // 16,
                              "block counts read twice and rewritten as prefixes; neuron "
                              "prefixes within groups of 64 and group totals written")),
        "fill_dxdw_kernel": (("mfma", 5 * 2.0 * n_ovf * dm * dff,
                              "dx_O = du W_u^T + dg W_g^T (2 GEMMs) and dW_d, dW_u, dW_g "
                              "(3 GEMMs); the CSC fill shares the launch")
                             if n_ovf > 0 else
                             ("hbm", 8 * T + nnz_ell * 22,
                              "per ELL entry: column, mask, block prefix, neuron prefix read, "
                              "slot written")),
        "mask_kernel": ("hbm", 8 * T + nnz_ell * 2 + nblk * dff * 12
                        + (4 * dff * row_b if dx_split else 0)
                        + (2 * n_ovf * row_b + 2 * ctx.get("R", 0) * row_b if n_ovf > 0 else 0),
                        "row_nnz, row_slot per row, column per ELL entry read; 64-row block "
                        "mask and count per neuron written; on the same launch the slice-major "
                        "wu_t, wg_t copy (XCD-local dx) and the backup rows' x, dy gathered "
                        "(read + write, padded to whole 128-row tiles)"),
    }


PEAK = {"mfma": BF16_PEAK_TFLOPS, "hbm": HBM_PEAK_GBS}
UNIT = {"mfma": "TFLOP/s", "hbm": "GB/s"}
SCALE = {"mfma": 1e12, "hbm": 1e9}


def kernel_entries(kms, work):
    res = {}
    for name, ms in kms.items():
        ent = {"us": round(ms * 1e3, 2)}
        if name in work and work[name][1] > 0:
            b, wk, desc = work[name]
            ach = wk / (ms * 1e-3) / SCALE[b]
            ent.update(bound=b, achieved=round(ach, 1), unit=UNIT[b],
                       frac=round(ach / PEAK[b], 4), work=wk, work_unit=desc)
        res[name] = ent
    return res


def roofline_of(kms, work, workload, alone=None):
    """Roofline entry of the dominant kernel (the longest with a roofline).
    alone: {kernel: ms} for kernels that one library call launches by
    themselves, timed as back-to-back calls with no events between launches;
    that time is used when the dominant kernel has one (events recorded
    around each kernel inside a step add several microseconds to it)."""
    dom = max((k for k in kms if k in work and work[k][1] > 0), key=lambda k: kms[k])
    b, wk, desc = work[dom]
    t_ms = (alone or {}).get(dom, kms[dom])
    ach = wk / (t_ms * 1e-3) / SCALE[b]
    traffic, note = measured_traffic(dom, workload)
    extra = {}
    if alone and dom in alone:
        extra = {"launch_timing": "back-to-back calls that launch only this kernel, HIP events "
                                  "around the run on the launch stream",
                 "in_step_event_us": round(kms[dom] * 1e3, 2)}
    return {"kernel": dom, "bound": b, "achieved": round(ach, 1), "peak": PEAK[b],
            "unit": UNIT[b], "frac": round(ach / PEAK[b], 4), "traffic": traffic,
            "traffic_note": note,
            "note": ("algorithmic bytes count every gathered row once per use; rows served "
                     "again from L2 or the MALL let them run above the HBM peak, and "
                     "traffic (HBM-side bytes from the counters) is then below them"
                     if b == "hbm" else
                     "algorithmic flops of the dense contraction over the kernel's mean "
                     "launch time (HIP events on the launch stream); traffic is the HBM-side "
                     "bytes of one launch"),
            "launch_us": round(t_ms * 1e3, 2), "work_per_launch": wk, "work_unit": desc,
            **extra}


# ----------------------------------------------------------------- helpers
class Layer:
    """Inputs of one workload resident on the GPU, with preallocated outputs
    and workspaces (the timed calls allocate nothing)."""

    def __init__(self, torch, tw, synth, w, dev, with_dy=False):
        d = synth.make_inputs(w, with_dy=with_dy)
        self.w, self.dev, self.tw = w, dev, tw
        self.x, self.wg, self.wu, self.wd = (d[k].to(dev) for k in ("x", "wg_t", "wu_t", "wd"))
        self.dy = d["dy"].to(dev) if with_dy else None
        self.host = d
        T, dm, dff, W = w.T, w.d_model, w.d_ff, w.width
        f32 = w.dtype == "f32"
        bf = tw.TWELL_F32 if f32 else tw.TWELL_BF16  # the element type of the layer
        tdt = torch.float32 if f32 else torch.bfloat16
        self.esz = 4 if f32 else 2
        self.st = torch.zeros(1, dtype=torch.int32, device=dev)
        self.twl = tw.empty_twell(T, dff, W, tdt, dev)
        self.y = torch.empty((T, dm), dtype=torch.float32, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.gws = torch.empty(max(1, tw.gate_workspace_bytes(bf, T, dm, dff)), **u8)
        self.fws = torch.empty(max(1, tw.fwd_workspace_bytes(bf, T, dm, dff, W)), **u8)
        self.train = with_dy
        if with_dy:
            self.hy = tw.empty_hybrid(T, dff, w.K, w.max_ovf, tdt, dev)
            self.hfws = torch.empty(max(1, tw.hybrid_fwd_workspace_bytes(bf, T, dm, dff, w.K,
                                                                         w.max_ovf)), **u8)
            f32 = dict(dtype=torch.float32, device=dev)
            self.grads = (torch.empty((T, dm), **f32), torch.empty((dff, dm), **f32),
                          torch.empty((dff, dm), **f32), torch.empty((dff, dm), **f32))
            self.bws = torch.empty(max(1, tw.bwd_workspace_bytes(bf, T, dm, dff, w.K,
                                                                 w.max_ovf)), **u8)

    # library calls, each optionally with a KernelTimer
    def gate(self, tm=None):
        self.tw.gate_pack(self.x, self.wg, width=self.w.width, out=self.twl, status=self.st,
                          workspace=self.gws, timing=tm)

    def ffn(self, tm=None):
        self.tw.ffn_fwd(self.x, self.twl, self.wu, self.wd, y=self.y, workspace=self.fws,
                        status=self.st, timing=tm)

    def to_hybrid(self, tm=None):
        self.tw.to_hybrid(self.twl, self.w.K, self.w.max_ovf, out=self.hy, status=self.st,
                          timing=tm)

    def hfwd(self, tm=None):
        self.tw.hybrid_fwd(self.x, self.hy, self.wu, self.wd, y=self.y, workspace=self.hfws,
                           status=self.st, timing=tm)

    def bwd(self, tm=None, l1=2e-5):
        self.tw.ffn_bwd(self.x, self.dy, self.hy, self.wg, self.wu, self.wd, out=self.grads,
                        workspace=self.bws, status=self.st, timing=tm, l1=l1)

    def fwd_step(self):
        self.gate()
        self.ffn()

    def train_step(self, l1=2e-5):
        self.gate()
        self.to_hybrid()
        self.hfwd()
        self.bwd(l1=l1)

    def check_status(self, what):
        s = int(self.st.item())
        if s != 0:
            raise SystemExit(f"{what}: device status {s} (a TwELL tile or the backup overflowed)")

    def counts(self, torch):
        W = self.w.width
        nnz = int(torch.clamp(self.twl.count, max=W).sum())
        out = {"T": self.w.T, "d_model": self.w.d_model, "d_ff": self.w.d_ff, "esz": self.esz,
               "nnz": nnz, "W": W}
        if self.train:
            ell = self.hy.row_slot < 0
            out.update(n_ovf=int(self.hy.n_ovf.item()),
                       nnz_ell=int(self.hy.row_nnz[ell].sum()),
                       R=(self.w.max_ovf + 127) // 128 * 128, S_y=self.y_splits())
        return out

    def y_splits(self):
        """K splits of the forward's y_O product, by the library's rule: about
        1024 workgroups over the 128 x 128 tiles of the capacity (rows padded
        to 256), at most 16, at least 16 K steps of 128 bytes each."""
        R = (self.w.max_ovf + 255) // 256 * 256
        tiles = (R // 128) * ((self.w.d_model + 127) // 128)
        nk = (2 if self.esz == 2 else 1) * (self.w.d_ff * self.esz // 128)
        return max(1, min(16, max(1, 1024 // max(tiles, 1)), max(1, nk // 16)))


def dense_fns(torch, L):
    """The dense bf16 layer of the same shapes (torch / hipBLASLt), with the gate
    and up weights fused into one GEMM: forward, and forward + backward."""
    dff = L.w.d_ff
    wgu_t = torch.cat([L.wg, L.wu], 0).t().contiguous()  # [d_model][2 d_ff]
    wd_c = L.wd.contiguous()
    wg_t = L.wg.t().contiguous()

    def fwd():
        gu = L.x @ wgu_t
        return (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ wd_c

    def gate_only():
        return L.x @ wg_t

    state = {}

    def train():
        if not state:
            state["p_gu"] = wgu_t.clone().requires_grad_(True)
            state["p_d"] = wd_c.clone().requires_grad_(True)
            state["xr"] = L.x.clone().requires_grad_(True)
        gu = state["xr"] @ state["p_gu"]
        yy = (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ state["p_d"]
        yy.backward(L.dy)
    return fwd, gate_only, train, state


def nbytes(*ts):
    return sum(t.numel() * t.element_size() for t in ts)


def memory_leg(torch, tw, L, l1):
    """Activation memory of one training step, sparse and dense, both taken from
    torch's caching allocator the same way: every buffer the step creates
    (activations, workspaces, y and the gradients) is allocated inside the
    measured region, the resident inputs and weights outside it. `saved` is
    what stays allocated between forward and backward apart from y; `peak` is
    the step's high-water mark; `peak_excl_grads` subtracts the gradient
    buffers (float32 for the sparse layer, bf16 for torch's) from it."""
    w, dev = L.w, L.dev
    T, dm, dff = w.T, w.d_model, w.d_ff
    bf = tw.TWELL_BF16
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    twl = tw.gate_pack(L.x, L.wg, width=w.width, workspace=torch.empty(
        max(1, tw.gate_workspace_bytes(bf, T, dm, dff)), **u8))
    hy = tw.to_hybrid(twl, w.K, w.max_ovf)
    del twl  # the TwELL is not needed once converted
    hfws = torch.empty(max(1, tw.hybrid_fwd_workspace_bytes(bf, T, dm, dff, w.K, w.max_ovf)),
                       **u8)
    y = tw.hybrid_fwd(L.x, hy, L.wu, L.wd, workspace=hfws)
    del hfws
    torch.cuda.synchronize()
    sp_saved = torch.cuda.memory_allocated() - base - nbytes(y)
    grads = (torch.empty((T, dm), **f32),) + tuple(torch.empty((dff, dm), **f32)
                                                   for _ in range(3))
    bws = torch.empty(max(1, tw.bwd_workspace_bytes(bf, T, dm, dff, w.K, w.max_ovf)), **u8)
    tw.ffn_bwd(L.x, L.dy, hy, L.wg, L.wu, L.wd, out=grads, workspace=bws, l1=l1)
    torch.cuda.synchronize()
    sp_peak = torch.cuda.max_memory_allocated() - base
    sp_grads = nbytes(*grads)
    del hy, y, grads, bws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    dff_ = dff
    p_gu = torch.cat([L.wg, L.wu], 0).t().contiguous().requires_grad_(True)
    p_d = L.wd.contiguous().requires_grad_(True)
    xr = L.x.clone().requires_grad_(True)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    gu = xr @ p_gu
    yy = (torch.relu(gu[:, :dff_]) * gu[:, dff_:]) @ p_d
    torch.cuda.synchronize()
    de_saved = torch.cuda.memory_allocated() - base - nbytes(yy)
    yy.backward(L.dy)
    torch.cuda.synchronize()
    de_peak = torch.cuda.max_memory_allocated() - base
    de_grads = nbytes(xr.grad, p_gu.grad, p_d.grad)
    del gu, yy, p_gu, p_d, xr
    torch.cuda.empty_cache()
    return {
        "method": "torch.cuda.memory_allocated / max_memory_allocated around one training "
                  "step; inputs and weights resident before, everything the step creates "
                  "inside",
        "sparse": {"saved_bytes": int(sp_saved), "peak_bytes": int(sp_peak),
                   "grad_bytes": int(sp_grads), "peak_excl_grads": int(sp_peak - sp_grads)},
        "dense_bf16": {"saved_bytes": int(de_saved), "peak_bytes": int(de_peak),
                       "grad_bytes": int(de_grads), "peak_excl_grads": int(de_peak - de_grads)},
        "saved_ratio": round(sp_saved / max(de_saved, 1), 4),
        "peak_ratio": round(sp_peak / max(de_peak, 1), 4),
        "peak_excl_grads_ratio": round((sp_peak - sp_grads) / max(de_peak - de_grads, 1), 4),
    }


def forward_leg(torch, tw, L, steps, workload, dense=True):
    """Sparse forward (gate_pack + ffn_fwd) against the dense bf16 layer."""
    ms = event_ms(torch, L.fwd_step, steps)
    L.check_status(workload)
    ctx = L.counts(torch)
    work = kernel_work(ctx)
    kms = kernel_ms(torch, tw, [L.gate, L.ffn], steps)
    T = L.w.T
    alone = {}
    if T > tw.DECODE_T:  # the gate call is then one kernel
        alone["gate_pack_kernel"] = event_ms(torch, lambda: L.gate(None), 4 * steps)
    out = {"workload": workload, "T": T, "d_model": L.w.d_model, "d_ff": L.w.d_ff,
           "density": L.w.density, "measured_density": round(ctx["nnz"] / (T * L.w.d_ff), 5),
           "nnz": ctx["nnz"], "twell_width": L.w.width,
           "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
           "kernels": kernel_entries(kms, work),
           "roofline": roofline_of(kms, work, workload, alone)}
    if dense:
        fwd, gate_only, _, _ = dense_fns(torch, L)
        with torch.no_grad():
            dms = event_ms(torch, fwd, steps)
            gms = event_ms(torch, gate_only, steps)
        out["dense_bf16"] = {
            "ms": round(dms, 4), "tokens_per_s": round(T / (dms * 1e-3), 1),
            "tflops": round(3 * 2.0 * T * L.w.d_model * L.w.d_ff / (dms * 1e-3) / 1e12, 1),
            "gate_gemm_alone_us": round(gms * 1e3, 2),
            "gate_gemm_alone_tflops": round(2.0 * T * L.w.d_model * L.w.d_ff / (gms * 1e-3)
                                            / 1e12, 1),
            "note": "torch/hipBLASLt: x [W_g W_u] in one GEMM, ReLU, product, W_d; the gate "
                    "GEMM alone writes g = x W_g as bf16"}
        out["speedup_vs_dense"] = round(dms / ms, 4)
    return out, kms, work


def train_leg(torch, tw, L, steps, workload, l1, dense=True):
    """Training step (gate_pack -> to_hybrid -> hybrid_fwd -> hybrid_bwd)
    against torch autograd of the dense bf16 layer."""
    ms = event_ms(torch, lambda: L.train_step(l1), steps)
    L.check_status(workload)
    ctx = L.counts(torch)
    work = kernel_work(ctx)
    kms = kernel_ms(torch, tw, [L.gate, L.to_hybrid, L.hfwd, lambda tm: L.bwd(tm, l1)], steps)
    T = L.w.T
    out = {"workload": workload, "T": T, "d_model": L.w.d_model, "d_ff": L.w.d_ff,
           "density": L.w.density, "skew_frac": L.w.skew_frac,
           "skew_density": L.w.skew_density, "K": L.w.K, "max_ovf": L.w.max_ovf,
           "twell_width": L.w.width, "l1": l1,
           "measured_density": round(ctx["nnz"] / (T * L.w.d_ff), 5), "nnz": ctx["nnz"],
           "nnz_ell": ctx["nnz_ell"], "n_ovf": ctx["n_ovf"],
           "step": "gate GEMM + TwELL pack, TwELL->hybrid, forward over the hybrid, hybrid "
                   "backward (dx, dW_g, dW_u, dW_d)",
           "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
           "kernels": kernel_entries(kms, work), "roofline": roofline_of(kms, work, workload),
           "kernels_note": "per-kernel times from a separate pass with events between the kernels, "
                           "every kernel in order on one stream; in the timed step a large "
                           "layer's backup-row forward products (bk_*) run on a second stream "
                           "beside its ELL passes"}
    bk = [k for k in kms if (k.startswith("bk_") and k != "bk_out_kernel")
          or (ctx["n_ovf"] > 0 and k in ("prefix_ud_kernel", "fill_dxdw_kernel"))]
    if bk:
        fl = sum(work[k][1] for k in bk)
        t = sum(kms[k] for k in bk)
        out["backup_products"] = {"kernels": bk, "us": round(t * 1e3, 2), "flop": fl,
                                  "tflops": round(fl / (t * 1e-3) / 1e12, 1),
                                  "frac": round(fl / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                                  "note": "the launches of the backward's products also run "
                                          "the ELL block scans and the CSC fill"}
    if dense:
        _, _, train, state = dense_fns(torch, L)
        dms = event_ms(torch, train, steps)
        out["dense_bf16"] = {
            "ms": round(dms, 4), "tokens_per_s": round(T / (dms * 1e-3), 1),
            "tflops": round(9 * 2.0 * T * L.w.d_model * L.w.d_ff / (dms * 1e-3) / 1e12, 1),
            "note": "torch autograd of the dense layer (x [W_g W_u] fused), bf16"}
        out["speedup_vs_dense"] = round(dms / ms, 4)
        state.clear()
        out["memory"] = memory_leg(torch, tw, L, l1)
    return out


def cold_leg(torch, tw, synth, L, n=10):
    """Cold-cache figures: a 512 MB scratch write (more than the 256 MB MALL and
    every L2) before each call, then the call timed with events. The forward
    of the headline layer (per kernel) and the decode layer at T = 1..64,
    each beside its dense bf16 counterpart measured the same way."""
    dev = L.dev
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def flush():
        scratch.fill_(1)

    def timed(fn, reps):
        for _ in range(3):  # first launches load code objects and pick GEMM kernels
            fn()
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(reps)]
        for a, b in e:
            flush()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in e) / reps

    fwd_ms = timed(L.fwd_step, n)
    timers = [tw.KernelTimer(), tw.KernelTimer()]
    kms = {}
    for _ in range(n):
        flush()
        L.gate(timers[0])
        L.ffn(timers[1])
        torch.cuda.synchronize()
        for tm in timers:
            for name, ms in tm.collect():
                kms[name] = kms.get(name, 0.0) + ms / n
    dfwd, _, _, _ = dense_fns(torch, L)
    with torch.no_grad():
        dense_ms = timed(dfwd, n)
    out = {"method": f"{FLUSH_BYTES >> 20} MB scratch write before every call; events "
                     "around the call", "calls": n,
           "forward": {"workload": L.w.name, "ms": round(fwd_ms, 4),
                       "kernel_us": {k: round(v * 1e3, 2) for k, v in kms.items()},
                       "dense_bf16_ms": round(dense_ms, 4),
                       "speedup_vs_dense": round(dense_ms / fwd_ms, 4)}}
    rows = []
    for T in synth.DECODE_T:
        w = synth.DECODE_2B.with_(T=T)
        d = synth.make_inputs(w)
        x, wg, wu, wd = (d[k].to(dev) for k in ("x", "wg_t", "wu_t", "wd"))
        o = tw.empty_twell(T, w.d_ff, w.width, torch.bfloat16, dev)
        y = torch.empty((T, w.d_model), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, tw.decode_workspace_bytes(tw.TWELL_BF16, T, w.d_model, w.d_ff,
                                                           w.width)),
                         dtype=torch.uint8, device=dev)
        sp = timed(lambda: tw.decode_fwd(x, wg, wu, wd, width=w.width, out=o, y=y,
                                         workspace=ws), n)
        gu_t = torch.cat([wg, wu], 0).t().contiguous()
        wd_c = wd.contiguous()
        dff = w.d_ff
        with torch.no_grad():
            de = timed(lambda: _dense_small(torch, x, gu_t, wd_c, dff), n)
        rows.append({"T": T, "sparse_us": round(sp * 1e3, 2), "dense_us": round(de * 1e3, 2),
                     "speedup": round(de / sp, 3)})
    out["decode"] = rows
    del scratch
    torch.cuda.empty_cache()
    return out


def _dense_small(torch, x, gu_t, wd_c, dff):
    gu = x @ gu_t
    return (torch.relu(gu[:, :dff]) * gu[:, dff:]) @ wd_c


def decode_leg(torch, tw, synth, dev):
    """The 2B-scale decode configuration (d_model 2304, d_ff 6144, 1%, W = 32)
    at T = 1, 8, 32, 64 tokens: twell_decode_fwd (the whole layer) against the
    dense bf16 layer, both graph-timed, with per-kernel event times and the
    weight bytes actually touched (W_g whole, plus one wu_t and one wd row per
    distinct active neuron)."""
    rows = []
    for T in synth.DECODE_T:
        w = synth.DECODE_2B.with_(T=T)
        d = synth.make_inputs(w)
        x, wg, wu, wd = (d[k].to(dev) for k in ("x", "wg_t", "wu_t", "wd"))
        out = tw.empty_twell(T, w.d_ff, w.width, torch.bfloat16, dev)
        y = torch.empty((T, w.d_model), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, tw.decode_workspace_bytes(tw.TWELL_BF16, T, w.d_model, w.d_ff,
                                                           w.width)),
                         dtype=torch.uint8, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)

        def sparse(tm=None):
            tw.decode_fwd(x, wg, wu, wd, width=w.width, out=out, y=y, workspace=ws, status=st,
                          timing=tm)
        sp_us = graph_us(torch, sparse)
        if int(st.item()) != 0:
            raise SystemExit(f"decode T={T}: device status {int(st.item())}")
        kms = kernel_ms(torch, tw, [sparse], 20)
        gu_t = torch.cat([wg, wu], 0).t().contiguous()
        wd_c = wd.contiguous()
        de_us = graph_us(torch, lambda: _dense_small(torch, x, gu_t, wd_c, w.d_ff))
        keep = (torch.arange(w.width, device=dev)[None, None, :]
                < out.count.clamp(max=w.width)[:, :, None])
        distinct = int(torch.unique(out.col[keep].long()).numel())
        touched = w.d_ff * w.d_model * 2 + distinct * 2 * w.d_model * 2
        rows.append({"T": T, "sparse_us": round(sp_us, 2), "dense_us": round(de_us, 2),
                     "speedup": round(de_us / sp_us, 3), "weight_bytes_touched": touched,
                     "touched_GBps": round(touched / (sp_us * 1e-6) / 1e9, 1),
                     "touched_frac_hbm": round(touched / (sp_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernel_us": {k: round(v * 1e3, 2) for k, v in kms.items()},
                     "nnz": int(out.count.clamp(max=w.width).sum())})
    return {"workload": "2b-decode", "d_model": 2304, "d_ff": 6144, "density": 0.01,
            "width": 32, "call": "twell_decode_fwd (gate partials, pack + up, down: 3 launches)",
            "timing": "HIP graph of 10 calls, replayed 20 times; kernel_us from events",
            "by_T": rows}


def tiny_leg(torch, tw, synth, dev, steps):
    """The tiny float32 configuration (T 64, d_model 256, d_ff 1024, 2%: the
    float32 MFMA gate and the few-token kernels): the inference forward
    (gate_pack + ffn_fwd, and twell_decode_fwd: the same layer in one call)
    and the training step (gate, TwELL->hybrid, forward
    over the hybrid, backward) against the dense float32 layer in torch. The
    forwards are graph-timed; the training steps are event-timed on both sides
    (torch's autograd is not captured), launches included."""
    w = synth.TINY_F32.with_(K=64, max_ovf=16)
    L = Layer(torch, tw, synth, w, dev, with_dy=True)
    fwd_us = graph_us(torch, L.fwd_step)
    L.check_status("tiny forward")
    dws = torch.empty(max(1, tw.decode_workspace_bytes(tw.TWELL_F32, w.T, w.d_model, w.d_ff,
                                                       w.width)), dtype=torch.uint8, device=dev)
    dec_us = graph_us(torch, lambda: tw.decode_fwd(L.x, L.wg, L.wu, L.wd, width=w.width,
                                                   out=L.twl, y=L.y, workspace=dws,
                                                   status=L.st))
    L.check_status("tiny forward in one call")
    tr_ms = event_ms(torch, L.train_step, steps)
    L.check_status("tiny training step")
    kms = kernel_ms(torch, tw, [L.gate, L.ffn], 20)
    fwd, _, train, _ = dense_fns(torch, L)
    with torch.no_grad():
        de_fwd_us = graph_us(torch, fwd)
    de_tr_ms = event_ms(torch, train, steps)
    c = L.counts(torch)
    return {"workload": "tiny-fp32", "T": w.T, "d_model": w.d_model, "d_ff": w.d_ff,
            "density": w.density, "dtype": "f32", "nnz": c["nnz"], "n_ovf": c["n_ovf"],
            "forward_us": round(fwd_us, 2), "dense_forward_us": round(de_fwd_us, 2),
            "forward_speedup": round(de_fwd_us / fwd_us, 3),
            "forward_one_call_us": round(dec_us, 2),
            "forward_one_call_speedup": round(de_fwd_us / dec_us, 3),
            "forward_kernel_us": {k: round(v * 1e3, 2) for k, v in kms.items()},
            "train_us": round(tr_ms * 1e3, 2), "dense_train_us": round(de_tr_ms * 1e3, 2),
            "train_speedup": round(de_tr_ms / tr_ms, 3),
            "timing": "forwards: HIP graph of 10 calls, replayed 20 times; training steps: "
                      "events around back-to-back steps"}


def sweep_leg(torch, tw, synth, dev):
    """The 1.5B-scale forward (T 8192, d_model 2048, d_ff 5632) at gate
    densities 0.5, 1, 2, 5 and 20%: gate GEMM + TwELL pack, then the fused
    up/down, against the dense bf16 forward of the same shape, both
    graph-timed. The TwELL width is 32 slots per tile up to 5% and 64 at 20%
    (about 26 nonzeros per 128-column tile there)."""
    rows = []
    for dens in synth.SWEEP_1P5B:
        w = synth.sweep_workload(dens)
        L = Layer(torch, tw, synth, w, dev)
        sp_us = graph_us(torch, L.fwd_step, calls=4, replays=10)
        L.check_status(f"sweep density {dens}")
        nnz = int(L.twl.count.clamp(max=w.width).sum())
        kms = kernel_ms(torch, tw, [L.gate, L.ffn], 5)
        fwd, _, _, _ = dense_fns(torch, L)
        with torch.no_grad():
            de_us = graph_us(torch, fwd, calls=4, replays=10)
        rows.append({"density": dens, "measured_density": round(nnz / (w.T * w.d_ff), 5),
                     "width": w.width, "sparse_us": round(sp_us, 1), "dense_us": round(de_us, 1),
                     "sparse_tokens_per_s": round(w.T / (sp_us * 1e-6), 1),
                     "dense_tokens_per_s": round(w.T / (de_us * 1e-6), 1),
                     "speedup": round(de_us / sp_us, 3),
                     "kernel_us": {k: round(v * 1e3, 1) for k, v in kms.items()}})
        del L, fwd
        torch.cuda.empty_cache()
    return {"workload": "1.5b-fwd", "T": 8192, "d_model": 2048, "d_ff": 5632,
            "call": "twell_gate_pack + twell_ffn_fwd (inference forward)",
            "timing": "HIP graph of 4 calls, replayed 10 times", "by_density": rows}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(synth, w, budget_s=12.0):
    """The float64 CPU oracle on this host, on a bounded sample of the headline
    workload (rows are independent, so a token subset is an exact share of
    the work): the sparse forward (gate, TwELL pack, sparse up/down) and the
    dense forward, then the tiny fp32 layer on all threads and on one."""
    import numpy as np
    import torch
    from oracle import oracle as orc
    d = synth.make_inputs(w)
    f64 = lambda t: t.double().numpy()
    X, WG, WU, WD = (f64(d[k]) for k in ("x", "wg_t", "wu_t", "wd"))
    threads = orc.num_threads()

    def run(fn, n_tok, budget):
        reps, el = 0, 0.0
        while el < budget and reps < 200:
            t1 = time.perf_counter()
            fn(reps, n_tok)
            el += time.perf_counter() - t1
            reps += 1
        return reps, el

    def sparse(rep, n):
        s = slice((rep * n) % w.T, (rep * n) % w.T + n)
        tws = orc.twell_pack(orc.gate(X[s], WG), W=w.width)
        tws["val"] = f64(torch.from_numpy(tws["val"]).to(torch.bfloat16))
        orc.ffn_twell(X[s], tws, WU, WD)

    def dense(rep, n):
        s = slice((rep * n) % w.T, (rep * n) % w.T + n)
        orc.ffn_dense(X[s], WG, WU, WD)

    n_sp, n_de = 256, 128
    r_sp, e_sp = run(sparse, n_sp, budget_s)
    r_de, e_de = run(dense, n_de, budget_s / 2)
    tiny = synth.TINY_F32
    dt = synth.make_inputs(tiny)
    Xt, WGt, WUt, WDt = (f64(dt[k]) for k in ("x", "wg_t", "wu_t", "wd"))

    def tiny_fwd(rep, n):
        tws = orc.twell_pack(orc.gate(Xt, WGt))
        orc.ffn_twell(Xt, tws, WUt, WDt)
    r_t, e_t = run(tiny_fwd, tiny.T, 1.0)
    orc.set_num_threads(1)
    try:
        r_t1, e_t1 = run(tiny_fwd, tiny.T, 1.0)
    finally:
        orc.set_num_threads(threads)
    return {"value": round(r_sp * n_sp / e_sp, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{r_sp} x {n_sp} consecutive tokens of the {w.name} workload (gate, "
                      f"TwELL pack, sparse up/down in float64), {e_sp:.1f} s",
            "threads_used": threads, "affinity_cpus": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "dense": {"value": round(r_de * n_de / e_de, 1), "unit": "tokens/s",
                      "sample": f"{r_de} x {n_de} tokens, dense float64 forward, {e_de:.1f} s"},
            "tiny_fp32": {"tokens_per_s": round(r_t * tiny.T / e_t, 1),
                          "tokens_per_s_1thread": round(r_t1 * tiny.T / e_t1, 1),
                          "sample": f"{tiny.name}: T {tiny.T}, {tiny.d_model} -> {tiny.d_ff}, "
                                    f"sparse forward, {r_t} and {r_t1} runs"}}


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

    WL = workloads(synth)
    w, kind = WL[a.workload]
    w = w.with_(name=a.workload)
    L = Layer(torch, tw, synth, w, dev, with_dy=(kind == "train"))
    step = L.fwd_step if kind == "fwd" else (lambda: L.train_step(a.l1))
    # clock settle: the part's clocks ramp for tens of milliseconds after an
    # idle spell (the gate GEMM runs ~10% slower meanwhile), so the step runs
    # for SETTLE_S seconds before the W warmup steps; nothing is timed here
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n_settle += 10
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    L.check_status(a.workload)

    # ---- timed region: K steps back to back, bracketed by synchronisation
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

    if kind == "fwd":
        head, _, _ = forward_leg(torch, tw, L, a.steps, a.workload, dense=not a.no_dense)
        step_desc = "gate GEMM + TwELL pack (twell_gate_pack), fused up/down over the TwELL " \
                    "(twell_ffn_fwd)"
    else:
        head = train_leg(torch, tw, L, a.steps, a.workload, a.l1, dense=not a.no_dense)
        step_desc = head["step"]
    roofline = head.pop("roofline")
    kernels = head.pop("kernels")

    extra = {}
    if not a.no_train and a.workload != "1.5b-train-skewed":
        Lt = Layer(torch, tw, synth, WL["1.5b-train-skewed"][0], dev, with_dy=True)
        extra["training_skewed"] = train_leg(torch, tw, Lt, a.steps, "1.5b-train-skewed",
                                             a.l1, dense=not a.no_dense)
        del Lt
        torch.cuda.empty_cache()
    if not a.no_small:
        if a.workload != "0.5b-fwd-1pct":
            Ls = Layer(torch, tw, synth, WL["0.5b-fwd-1pct"][0], dev)
            r, _, _ = forward_leg(torch, tw, Ls, a.steps, "0.5b-fwd-1pct",
                                  dense=not a.no_dense)
            extra["fwd_0p5b"] = r
            del Ls
        if a.workload != "0.5b-train-1pct":
            Ls = Layer(torch, tw, synth, WL["0.5b-train-1pct"][0].with_(name="0.5b-train-1pct"),
                       dev, with_dy=True)
            extra["train_0p5b"] = train_leg(torch, tw, Ls, a.steps, "0.5b-train-1pct", a.l1,
                                            dense=not a.no_dense)
            del Ls
        torch.cuda.empty_cache()
    if not a.no_cold and kind == "fwd":
        extra["cold"] = cold_leg(torch, tw, synth, L)
    if not a.no_decode:
        extra["decode"] = decode_leg(torch, tw, synth, dev)
    if not a.no_tiny:
        extra["tiny_fp32"] = tiny_leg(torch, tw, synth, dev, a.steps)
    if not a.no_sweep:
        extra["density_sweep"] = sweep_leg(torch, tw, synth, dev)
    cpu = None if a.no_cpu else cpu_leg(synth, w)

    T = w.T
    out = {
        "metric": METRIC,
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "settle": {"seconds": SETTLE_S, "steps": n_settle,
                   "note": "untimed steps before the warmup while the clocks ramp"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs and weights, gate offset for the target "
                "density)",
        "config": {"workload": a.workload, "step": step_desc, "T": T, "d_model": w.d_model,
                   "d_ff": w.d_ff, "density": w.density,
                   "measured_density": head.get("measured_density"), "nnz": head.get("nnz"),
                   "twell_width": w.width},
        "speedup_vs_dense": head.get("speedup_vs_dense"),
        "dense_bf16": head.get("dense_bf16"),
        "roofline": roofline,
        "kernels": kernels,
        "headline_detail": head,
        **extra,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
