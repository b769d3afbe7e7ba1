"""Helpers of the GPU parity tests: run the HIP path (through the C ABI) and the
CPU oracle on the same seeded inputs and compare them."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import eagle_draft_amd as e3
import oracle
import synth

# Tolerances: bf16 -- out max-abs 2e-2, lse max-abs 1e-2, dq/dk/dv relative
# Frobenius 3e-2 (dk and dv over all blocks together, and each of dk0, dv0, dkd,
# dvd on its own); fp32 -- 1e-5 on all.
TOL = {"bf16": dict(out=2e-2, lse=1e-2, grad=3e-2), "f32": dict(out=1e-5, lse=1e-5, grad=1e-5)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(w: synth.Workload) -> dict:
    """Seeded inputs of a share. A zig-zag share of several documents takes its
    rows of the virtual global tensors at the oracle's positions."""
    if w.layout == "zigzag" and w.doc_lens is not None and len(w.doc_lens) > 1:
        pos = oracle.query_positions("zigzag", w.T, w.cp, w.rank, w.cu_seqlens())
        return synth.make_inputs(w, positions=pos)
    return synth.make_inputs(w)


def problem(w: synth.Workload, device="cuda") -> e3.Problem:
    return e3.Problem(w.B, w.T, w.T_kv, w.H, w.D, w.num_blocks, w.scale, dtype=w.torch_dtype,
                      layout=w.layout, cp=w.cp, rank=w.rank, cu_seqlens=w.cu_seqlens(),
                      device=device)


def run_hip(w: synth.Workload, inp: dict, device="cuda"):
    """Forward + backward through the C ABI."""
    prob = problem(w, device)
    d = {k: v.to(device) for k, v in inp.items()}
    out, lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
    grads = e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), [g.cpu() for g in grads]


def oracle_cp(w):
    return w.cp if w.layout in ("contiguous", "zigzag") else 1


def stored_out(w: synth.Workload, o: np.ndarray) -> np.ndarray:
    """The forward output as the backward receives it: in q's dtype (ulysses_attention
    page, `cached_ulysses_attention` returns q's dtype; `_block0_backward` takes the
    merged out_g in q's dtype), so delta = <dO, out> is formed from the rounded out.
    The oracle's backward is given its own exact out rounded the same way (to
    nearest even); in rows where one key takes almost all the probability,
    ds = pi (dpi - delta) nearly cancels and this rounding alone moves the
    gradient by several percent, for any implementation of that interface."""
    if w.dtype != "bf16":
        return o
    return torch.from_numpy(o).to(torch.bfloat16).double().numpy()


def run_oracle(w: synth.Workload, inp: dict, heads=None, rows=256):
    """Oracle forward + backward for the requested heads (all by default). Inputs
    are converted to float64 one head at a time to bound host memory."""
    hs = list(range(w.H)) if heads is None else list(heads)
    B, T, N, D = w.B, w.T, w.N, w.D
    cu = w.cu_seqlens()
    qpos = oracle.query_positions(w.layout, T, oracle_cp(w), w.rank, cu)
    out = np.zeros((B, T, len(hs), D))
    lse = np.zeros((B, len(hs), T))
    dq = np.zeros((B, T, len(hs), D))
    dk0 = np.zeros((B, w.T_kv, len(hs), D))
    dv0 = np.zeros((B, w.T_kv, len(hs), D))
    dkd = np.zeros((B, N, T, len(hs), D))
    dvd = np.zeros((B, N, T, len(hs), D))
    f = lambda t: t.double().numpy()
    for b in range(B):
        for j, h in enumerate(hs):
            q, k0, v0 = f(inp["q"][b, :, h]), f(inp["k0"][b, :, h]), f(inp["v0"][b, :, h])
            kd, vd, do = f(inp["kd"][b, :, :, h]), f(inp["vd"][b, :, :, h]), f(inp["dout"][b, :, h])
            o, l = oracle.forward_head(q, k0, v0, kd, vd, w.scale, qpos, cu, rows)
            g = oracle.backward_head(do, q, k0, v0, kd, vd, w.scale, qpos, cu,
                                     out=stored_out(w, o), lse=l, rows=rows)
            out[b, :, j], lse[b, j] = o, l
            dq[b, :, j], dk0[b, :, j], dv0[b, :, j], dkd[b, :, :, j], dvd[b, :, :, j] = g
    return out, lse, (dq, dk0, dv0, dkd, dvd)


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def compare(w, hip, ref, heads=None):
    """Returns the error metrics of the HIP result against the oracle."""
    out, lse, (dq, dk0, dv0, dkd, dvd) = hip
    rout, rlse, (rdq, rdk0, rdv0, rdkd, rdvd) = ref
    if heads is not None:
        hs = list(heads)
        out, dq, dk0, dv0 = out[:, :, hs], dq[:, :, hs], dk0[:, :, hs], dv0[:, :, hs]
        dkd, dvd = dkd[:, :, :, hs], dvd[:, :, :, hs]
        lse = lse[:, hs]
    f = lambda t: t.double().numpy()
    m = {
        "out": float(np.abs(f(out) - rout).max()) if rout.size else 0.0,
        "lse": float(np.abs(f(lse) - rlse).max()) if rlse.size else 0.0,
        "dq": rel(f(dq), rdq),
        "dk": rel(np.concatenate([f(dk0).ravel(), f(dkd).ravel()]),
                  np.concatenate([rdk0.ravel(), rdkd.ravel()])),
        "dv": rel(np.concatenate([f(dv0).ravel(), f(dvd).ravel()]),
                  np.concatenate([rdv0.ravel(), rdvd.ravel()])),
    }
    # Each gradient block on its own as well: the diagonal blocks are N times larger
    # than block 0 and would dilute a block-0-only error in the combined norms.
    m["dk0"] = rel(f(dk0), rdk0)
    m["dv0"] = rel(f(dv0), rdv0)
    if w.N > 0:
        m["dkd"] = rel(f(dkd), rdkd)
        m["dvd"] = rel(f(dvd), rdvd)
    for k, v in m.items():
        assert np.isfinite(v), (k, v)
    return m


GRAD_KEYS = ("dq", "dk", "dv", "dk0", "dv0", "dkd", "dvd")


def assert_within(w, m):
    t = TOL[w.dtype]
    assert m["out"] <= t["out"], m
    assert m["lse"] <= t["lse"], m
    for k in GRAD_KEYS:
        if k in m:
            assert m[k] <= t["grad"], (k, m)
