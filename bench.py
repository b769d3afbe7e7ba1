"""Benchmark of EAGLE-3 mixed attention (forward + backward) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dense]

One step = one pass of the whole hot path over one batch: the forward (block-0
causal attention + TTT diagonals + merge) and the backward (delta, dK/dV, dQ +
closed-form diagonal gradients). Inputs are seeded synthetic tensors already
resident in HBM. Prints ONE JSON line with the throughput in TFLOP/s counted
with causal FLOPs (F_fwd = 4*B*H*D*P0 over the attended block-0 pairs P0,
F_bwd = 2.5*F_fwd; the diagonal FLOPs are not counted), the per-kernel times
measured with HIP events on the launch stream, the roofline of the dominant
kernel and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "EAGLE-3 mixed attn fwd+bwd TFLOP/s (causal) + % bf16 MFMA peak, T=4096 H=32 D=128"
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}   # MI355X dense MFMA (bf16) / fp32 vector
PEAK_GBS = 8000.0                               # MI355X HBM3E
# Stages timed with the events the library records per call (see
# eagle3_set_timing_events): forward e0 | fwd | e1; backward e0 | dq | e1, side
# stream e2 | diag_bwd | e3, main e1 | dkdv | e4 | the wait for the side stream | e5.
NFWD_EV, NBWD_EV = 2, 6
STAGE_EVENTS = {"fwd": ("f", 0, 1), "dq": ("b", 0, 1), "diag_bwd": ("b", 2, 3),
                "dkdv": ("b", 1, 4), "bwd_tail": ("b", 4, 5)}
KERNELS = list(STAGE_EVENTS)
KERNEL_NAMES = {"fwd": "fwd_kernel", "dq": "dq_kernel", "dkdv": "dkdv_kernel",
                "diag_bwd": "diag_bwd_kernel", "bwd_tail": "(join)"}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sources_sha256():
    """Hash of the kernel sources (the HIP files, the C ABI and its header)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "eagle_draft_amd", "csrc", "*")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` at the Dense workload from the counter
    summary in profiles/ (FETCH_SIZE and WRITE_SIZE, each divided by the factor the
    same counter reads on a plain copy of known size), or None when there is none
    for this kernel or workload, or the kernel sources changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", "dense_traffic.txt")
    if workload != "dense" or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^- ([\w.]+): (\S+)", line.strip())
            if m:
                kv[m.group(1)] = m.group(2)
    try:
        if kv.get("sources_sha256") != sources_sha256():
            return None
        fetch = float(kv[f"{kernel}.fetch_bytes_per_launch"]) / float(kv["copy_fetch_factor"])
        write = float(kv[f"{kernel}.write_bytes_per_launch"]) / float(kv["copy_write_factor"])
    except (KeyError, ValueError):
        return None
    return round(fetch + write)


def kernel_work(w, P0):
    """Algorithmic FLOPs and HBM bytes per launch of each stage. u = B*T*H*D*esz
    (one local [T,H,D] tensor), ukv = B*T_kv*H*D*esz, f32 = B*T*H*D*4."""
    esz = 2 if w.dtype == "bf16" else 4
    B, T, Tkv, H, D, N = w.B, w.T, w.T_kv, w.H, w.D, w.N
    u = B * T * H * D * esz
    ukv = B * Tkv * H * D * esz
    f32 = B * T * H * D * 4
    rowf = B * H * T * 4                      # one float per (b, h, row): lse or delta
    pf = B * H * D * P0                       # one D-long dot per attended pair
    diagf = B * H * D * T * N
    return {
        # q, k0, v0, kd, vd read; out, lse written
        "fwd": dict(flop=4 * pf, diag_flop=4 * diagf, bytes=u + 2 * ukv + 2 * N * u + u + rowf),
        # q, dO, O, k0, v0, lse read; delta, lse*log2(e) and dq (or its float32
        # partial) written; S, dP, dQ = 3 products
        "dq": dict(flop=6 * pf, diag_flop=0, bytes=3 * u + (f32 if N else u) + 2 * ukv + 3 * rowf),
        # q, dO, k0, v0, lse, delta read; dk0, dv0 written; S, dP, dV, dK = 4 products
        "dkdv": dict(flop=8 * pf, diag_flop=0, bytes=2 * u + 4 * ukv + 2 * rowf),
        # side stream (beside dK/dV): q, dO, kd, vd, the float32 dq partial, lse*log2(e),
        # delta read; dq, dkd, dvd written
        "diag_bwd": dict(flop=0, diag_flop=10 * diagf,
                         bytes=(2 * u + 2 * N * u + f32 + 2 * rowf + u + 2 * N * u) if N else 0),
        # the wait for the side stream after dK/dV: time only
        "bwd_tail": dict(flop=0, diag_flop=0, bytes=0),
    }


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            rc = self.rt.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            arr[i] = e.value
        return arr

    def elapsed_ms(self, a, b):
        t = ctypes.c_float()
        rc = self.rt.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(t.value)

    def destroy(self, arr):
        for e in arr:
            self.rt.hipEventDestroy(ctypes.c_void_p(e))


def cpu_baseline(w, inp, P0_per_head, budget_s):
    """The CPU oracle (float64) on whole heads of the same workload until about
    `budget_s` seconds of work; throughput on the same counted FLOPs."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    f = {k: v.double().numpy() for k, v in inp.items()}
    cu = w.cu_seqlens()
    ocp = w.cp if w.layout in ("contiguous", "zigzag") else 1
    done, secs = 0, 0.0
    for h in range(w.H):
        t0 = time.perf_counter()
        out, lse = oracle.forward(f["q"], f["k0"], f["v0"], f["kd"], f["vd"], w.scale, cu,
                                  w.layout, ocp, w.rank, heads=[h])
        oracle.backward(f["dout"], f["q"], f["k0"], f["v0"], f["kd"], f["vd"], w.scale, cu,
                        w.layout, ocp, w.rank, out=out, lse=lse, heads=[h])
        secs += time.perf_counter() - t0
        done += 1
        if secs >= budget_s:
            break
    flop = 3.5 * 4 * w.B * w.D * P0_per_head * done
    cores = len(os.sched_getaffinity(0))
    return {
        "value": flop / secs / 1e12, "unit": "TFLOP/s", "cores": blas_threads or cores,
        "kind": "oracle",
        "sample": f"{done} of {w.H} heads (all {w.T} rows, fwd+bwd, float64 NumPy), "
                  f"{secs:.1f} s; host has {cores} cores available",
        "seconds": secs,
    }


def _median_us(fn, n=20, warm=3):
    """Median duration of fn() in microseconds, torch events on the current stream
    (every entry point timed here launches on it)."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return statistics.median(ts)


def _roof(kind, amount, us):
    """Roofline record: kind "mfma" (amount = FLOP, bf16 peak) or "hbm" (bytes)."""
    if kind == "mfma":
        ach = amount / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS["bf16"], 4)}
    ach = amount / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_GBS, 4)}


def run_extras(args, dev):
    """The paths beside the headline, each at a full-size shape, one JSON line each:
    ring-step mode and the one-pass shard on the last rank of a contiguous ring
    (cp = 8 of a 32768-token sequence, H = 32, D = 128, num_blocks = 8), the
    frozen-target forward on the same share (num_blocks = 1, head-major), and the
    four Ulysses transforms at the Ulysses sequence shard (S_local = 4096 of 32768,
    H = 32, D = 128, uly = 8). FLOP are counted as in the headline (4*B*H*D*P0
    forward, 2.5x that backward); bytes are those each kernel must move."""
    import torch
    import eagle_draft_amd as e3
    import synth

    def emit(rec):
        print(json.dumps(rec), flush=True)

    # ---- ring-step mode against the one-pass shard -----------------------------
    w = synth.Workload("ring_contig_r7", "bf16", 1, 32768, 32, 128, 8, layout="contiguous",
                       cp=8, rank=7, seed=args.seed)
    log(f"[extras] {w}")
    d = {k: v.to(dev) for k, v in synth.make_inputs(w).items()}
    prob = e3.Problem(w.B, w.T, w.T_kv, w.H, w.D, w.num_blocks, w.scale, dtype=w.torch_dtype,
                      layout=w.layout, cp=w.cp, rank=w.rank, device=dev)
    P0 = prob.pair_count()
    ffwd = 4.0 * w.B * w.H * w.D * P0
    out, lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
    ws = torch.empty(max(prob.workspace_bytes(), 256), dtype=torch.uint8, device=dev)
    g = e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse, workspace=ws)
    t_fwd = _median_us(lambda: e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out=out, lse=lse))
    t_bwd = _median_us(lambda: e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out,
                                      lse, grads=g, workspace=ws))
    B, T, H, D = w.B, w.T, w.H, w.D
    acc_o = torch.empty(B, T, H, D, dtype=torch.float32, device=dev)
    acc_l = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    so = torch.empty_like(acc_o)
    sl = torch.empty_like(acc_l)
    o2, l2 = torch.empty_like(out), torch.empty_like(lse)
    dq_acc = torch.empty(B, T, H, D, dtype=torch.float32, device=dev)
    dk_acc = torch.empty(B, w.T_kv, H, D, dtype=torch.float32, device=dev)
    dv_acc = torch.empty_like(dk_acc)
    gd = (torch.empty_like(d["q"]), torch.empty_like(d["kd"]), torch.empty_like(d["vd"]))

    def ring_fwd():
        acc_o.zero_()
        acc_l.fill_(float("-inf"))
        for j in range(w.cp):
            e3.ring_fwd_step(prob, j, d["q"], d["k0"], d["v0"], out_step=so, lse_step=sl)
            e3.lse_merge(acc_o, acc_l, so, sl)
        e3.diag_merge_fwd(prob, d["q"], d["kd"], d["vd"], acc_o, acc_l, out=o2, lse=l2)

    def ring_bwd():
        dq_acc.zero_()
        dk_acc.zero_()
        dv_acc.zero_()
        for j in range(w.cp):
            e3.ring_bwd_step(prob, j, d["dout"], d["q"], d["k0"], d["v0"], out, lse, dq_acc, dk_acc,
                             dv_acc, workspace=ws)
        e3.diag_bwd(prob, d["dout"], d["q"], d["kd"], d["vd"], out, lse, dq_acc, grads=gd)

    t_rf = _median_us(ring_fwd, n=10)
    t_rb = _median_us(ring_bwd, n=10)
    # the HBM-bound pieces of the chain, alone
    ring_fwd()
    t_merge = _median_us(lambda: e3.lse_merge(acc_o, acc_l, so, sl))
    t_dmerge = _median_us(lambda: e3.diag_merge_fwd(prob, d["q"], d["kd"], d["vd"], acc_o, acc_l, out=o2,
                                                    lse=l2))
    t_dbwd = _median_us(lambda: e3.diag_bwd(prob, d["dout"], d["q"], d["kd"], d["vd"], out, lse, dq_acc,
                                            grads=gd))
    u = B * T * H * D
    N = w.N
    merge_bytes = 3 * u * 4 + 3 * B * H * T * 4
    dmerge_bytes = u * 2 + 2 * N * u * 2 + u * 4 + B * H * T * 4 + u * 2 + B * H * T * 4
    dbwd_bytes = 3 * u * 2 + 2 * N * u * 2 + u * 4 + B * H * T * 4 + u * 2 + 2 * N * u * 2
    cfg = {"workload": w.name, "B": B, "T": T, "T_kv": w.T_kv, "H": H, "D": D, "num_blocks": w.num_blocks,
           "layout": w.layout, "cp": w.cp, "rank": w.rank}
    emit({"extra": "ring_step_mode", "metric": "fwd+bwd TFLOP/s (causal), ring steps chained",
          "value": round(3.5 * ffwd / ((t_rf + t_rb) * 1e-6) / 1e12, 2), "unit": "TFLOP/s",
          "ms_fwd": round(t_rf / 1e3, 3), "ms_bwd": round(t_rb / 1e3, 3),
          "one_pass": {"value": round(3.5 * ffwd / ((t_fwd + t_bwd) * 1e-6) / 1e12, 2),
                       "ms_fwd": round(t_fwd / 1e3, 3), "ms_bwd": round(t_bwd / 1e3, 3)},
          "roofline": _roof("mfma", 3.5 * ffwd, t_rf + t_rb), "config": cfg, "pairs_P0": P0,
          "pieces": {"lse_merge": {"us": round(t_merge, 1), "roofline": _roof("hbm", merge_bytes, t_merge)},
                     "diag_merge_fwd": {"us": round(t_dmerge, 1),
                                        "roofline": _roof("hbm", dmerge_bytes, t_dmerge)},
                     "diag_bwd": {"us": round(t_dbwd, 1), "roofline": _roof("hbm", dbwd_bytes, t_dbwd)}},
          "dtype": "bf16", "data": "synthetic (seeded N(0,1) inputs, resident in HBM)"})

    # ---- frozen-target forward (head-major, num_blocks = 1) ---------------------
    p1 = e3.Problem(B, T, w.T_kv, H, D, 1, w.scale, dtype=w.torch_dtype, layout=w.layout, cp=w.cp,
                    rank=w.rank, device=dev)
    hm = lambda t: t.permute(0, 2, 1, 3).contiguous()
    qh, kh, vh = hm(d["q"]), hm(d["k0"]), hm(d["v0"])
    oh, lh = e3.target_cp_fwd(p1, qh, kh, vh)
    t_tcp = _median_us(lambda: e3.target_cp_fwd(p1, qh, kh, vh, out=oh, lse=lh))
    emit({"extra": "target_cp_fwd", "metric": "forward TFLOP/s (causal), head-major, num_blocks = 1",
          "value": round(ffwd / (t_tcp * 1e-6) / 1e12, 2), "unit": "TFLOP/s", "ms": round(t_tcp / 1e3, 3),
          "roofline": _roof("mfma", ffwd, t_tcp), "config": dict(cfg, num_blocks=1), "pairs_P0": P0,
          "dtype": "bf16", "data": "synthetic (seeded N(0,1) inputs, resident in HBM)"})
    del d, out, lse, g, ws, acc_o, acc_l, so, sl, o2, l2, dq_acc, dk_acc, dv_acc, gd, qh, kh, vh, oh, lh
    torch.cuda.empty_cache()

    # ---- Ulysses transforms -------------------------------------------------------
    uly, Sl = 8, 4096
    gen = torch.Generator(device="cpu").manual_seed(args.seed)
    x = torch.randn(B, Sl, H, D, generator=gen).to(torch.bfloat16).to(dev)
    lx = torch.randn(B, H, Sl, generator=gen).to(dev)
    recs = {}
    for kind, stage, src, nbytes in (
            ("seq_to_head", 0, x, x.numel() * 2), ("seq_to_head", 1, None, x.numel() * 2),
            ("head_to_seq", 0, None, x.numel() * 2), ("head_to_seq", 1, None, x.numel() * 2),
            ("lse_gather", 0, lx, lx.numel() * 4), ("lse_gather", 1, None, lx.numel() * 4),
            ("lse_scatter", 0, None, lx.numel() * 4), ("lse_scatter", 1, None, lx.numel() * 4)):
        if src is None:
            src = prev
        D_ = D if not kind.startswith("lse") else 1
        o_ = e3.ulysses(kind, stage, src, uly, B, Sl, H, D_)
        t = _median_us(lambda: e3.ulysses(kind, stage, src, uly, B, Sl, H, D_, out=o_))
        recs[f"{kind}/{stage}"] = {"us": round(t, 2), "roofline": _roof("hbm", 2 * nbytes, t)}
        prev = o_
    tot_b = 2 * (4 * x.numel() * 2 + 4 * lx.numel() * 4)
    tot_t = sum(r["us"] for r in recs.values())
    emit({"extra": "ulysses_transforms", "metric": "re-sharding GB/s (read + write)",
          "value": round(tot_b / (tot_t * 1e-6) / 1e9, 1), "unit": "GB/s",
          "roofline": _roof("hbm", tot_b, tot_t), "pieces": recs,
          "config": {"workload": "ulysses_shard", "B": B, "S_local": Sl, "S_full": Sl * uly, "H": H, "D": D,
                     "uly": uly},
          "dtype": "bf16", "data": "synthetic (seeded N(0,1) inputs, resident in HBM)"})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU oracle work for the baseline (0 = skip)")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--extras", action="store_true",
                    help="instead of the headline: time the ring-step mode, the frozen-target "
                         "forward and the Ulysses transforms (one JSON line each)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (a known-size "
                         "kernel for calibrating the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU's share on one GPU only; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: the library runs one GPU's share "
              "(full sequence, Ulysses head shard or zig-zag rank) and has no collectives.", file=sys.stderr)
        sys.exit(2)

    import torch
    import eagle_draft_amd as e3
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.extras:
        run_extras(args, dev)
        return
    w = synth.workload(args.workload, seed=args.seed)
    log(f"[bench] workload {w}")
    prob = e3.Problem(w.B, w.T, w.T_kv, w.H, w.D, w.num_blocks, w.scale, dtype=w.torch_dtype,
                      layout=w.layout, cp=w.cp, rank=w.rank, cu_seqlens=w.cu_seqlens(), device=dev)
    if w.layout == "zigzag" and w.doc_lens is not None and len(w.doc_lens) > 1:
        # a zig-zag share of several documents: its rows of the virtual global
        # tensors, at the positions the library's layout tables give
        inp_cpu = synth.make_inputs(w, positions=prob.query_positions())
    else:
        inp_cpu = synth.make_inputs(w)
    d = {k: v.to(dev) for k, v in inp_cpu.items()}
    P0 = prob.pair_count()                      # per (batch row, head)
    out = torch.empty_like(d["q"])
    lse = torch.empty(w.B, w.H, w.T, dtype=torch.float32, device=dev)
    grads = (torch.empty_like(d["q"]), torch.empty_like(d["k0"]), torch.empty_like(d["v0"]),
             torch.empty_like(d["kd"]), torch.empty_like(d["vd"]))
    ws = torch.empty(max(prob.workspace_bytes(), 256), dtype=torch.uint8, device=dev)
    lib = e3.lib()

    def step():
        e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out=out, lse=lse)
        e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse,
               grads=grads, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")
    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")

    # (1) the timed region: exactly K back-to-back steps, synchronized on both sides
    ev = HipEvents()
    se = ev.create(2)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ev.rt.hipEventRecord(ctypes.c_void_p(se[0]), stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    ev.rt.hipEventRecord(ctypes.c_void_p(se[1]), stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    total_ms = ev.elapsed_ms(se[0], se[1])
    ms_per_step = total_ms / args.steps
    log(f"[bench] {args.steps} steps: {total_ms:.3f} ms ({ms_per_step:.4f} ms/step, wall {wall_ms:.1f} ms)")

    # (2) per-kernel times: events recorded by the library around each kernel
    nfwd, nbwd = NFWD_EV, NBWD_EV
    per = {k: [] for k in KERNELS}
    fwd_ms, bwd_ms, flushed = [], [], []
    flush_buf = None if args.no_flush else torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    reps = max(args.steps, 5)
    evf = ev.create(nfwd * reps)
    evb = ev.create(nbwd * reps)
    for r in range(reps):
        if flush_buf is not None:
            flush_buf.zero_()     # evict L2 and MALL between steps (outside the events)
        psz = ctypes.sizeof(ctypes.c_void_p)
        lib.eagle3_set_timing_events(ctypes.c_void_p(ctypes.addressof(evf) + r * nfwd * psz), nfwd)
        e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out=out, lse=lse)
        assert lib.eagle3_timing_events_recorded() == nfwd
        lib.eagle3_set_timing_events(ctypes.c_void_p(ctypes.addressof(evb) + r * nbwd * psz), nbwd)
        e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse,
               grads=grads, workspace=ws)
        assert lib.eagle3_timing_events_recorded() == nbwd
        lib.eagle3_set_timing_events(None, 0)
    torch.cuda.synchronize()
    for r in range(reps):
        f0 = r * nfwd
        b0 = r * nbwd
        for k, (which, i, j) in STAGE_EVENTS.items():
            arr, base = (evf, f0) if which == "f" else (evb, b0)
            per[k].append(ev.elapsed_ms(arr[base + i], arr[base + j]))
        fwd_ms.append(ev.elapsed_ms(evf[f0], evf[f0 + nfwd - 1]))
        bwd_ms.append(ev.elapsed_ms(evb[b0], evb[b0 + nbwd - 1]))
        flushed.append(fwd_ms[-1] + bwd_ms[-1])
    ev.destroy(se)
    ev.destroy(evf)
    ev.destroy(evb)
    del flush_buf

    work = kernel_work(w, P0)
    kern = {}
    for k in KERNELS:
        t_us = statistics.mean(per[k]) * 1e3
        kw = work[k]
        kern[k] = {
            "us_mean": round(t_us, 2), "us_median": round(statistics.median(per[k]) * 1e3, 2),
            "tflops": round(kw["flop"] / (t_us * 1e-6) / 1e12, 2) if kw["flop"] and t_us > 0 else None,
            "gbs": round(kw["bytes"] / (t_us * 1e-6) / 1e9, 1) if kw["bytes"] and t_us > 0 else None,
            "flop": kw["flop"], "bytes": kw["bytes"], "kernel": KERNEL_NAMES[k],
        }
    kern["diag_bwd"]["stream"] = "side (overlaps dkdv)"
    kern["bwd_tail"]["note"] = "time only: the wait for diag_bwd after dkdv"
    # the dominant kernel: the longest of the kernels on the critical path
    dom = max(("fwd", "dq", "dkdv", "diag_bwd"), key=lambda k: kern[k]["us_mean"])
    dk = kern[dom]
    t_dom = dk["us_mean"] * 1e-6
    peak_t = PEAK_TFLOPS[w.dtype]
    mfma_time = dk["flop"] / (peak_t * 1e12)
    hbm_time = dk["bytes"] / (PEAK_GBS * 1e9)
    if mfma_time >= hbm_time and dk["flop"] > 0:
        roof = {"bound": "mfma", "achieved": round(dk["flop"] / t_dom / 1e12, 2), "peak": peak_t,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(dk["bytes"] / t_dom / 1e9, 1), "peak": PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(KERNEL_NAMES[dom], w.name)
    roof["kernel"] = KERNEL_NAMES[dom]
    roof["stage"] = dom
    roof["algorithmic"] = {"flop": dk["flop"], "bytes": dk["bytes"]}

    counted = 3.5 * 4 * w.B * w.H * w.D * P0
    value = counted / (ms_per_step * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(dev)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "T_kv": w.T_kv, "H": w.H, "D": w.D,
                   "num_blocks": w.num_blocks, "layout": w.layout, "cp": w.cp, "rank": w.rank,
                   "num_docs": len(w.doc_lens) if w.doc_lens else 1, "seed": w.seed},
        "pct_peak": round(100.0 * value / PEAK_TFLOPS[w.dtype], 2),
        "counted_flop": counted,
        "pairs_P0": P0,
        "flushed_ms_per_step_median": round(statistics.median(flushed), 4),
        "fwd_ms_median": round(statistics.median(fwd_ms), 4),
        "bwd_ms_median": round(statistics.median(bwd_ms), 4),
        "kernels": kern,
        "roofline": roof,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count},
        "sources_sha256": sources_sha256(),
    }
    if args.cpu_budget > 0:
        log("[bench] timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(w, inp_cpu, P0, args.cpu_budget)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
