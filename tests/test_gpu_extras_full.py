"""GPU parity of the widened paths at the full size `bench.py --extras` times them: the
last rank of a contiguous ring (cp = 8 of a 32768-token sequence, 4096 local rows against
32768 keys, H = 32, D = 128, num_blocks = 8).

- the one-pass shard forward and backward, and ring-step mode (every step's partial
  merged by lse_merge, then the diagonal merge; the backward step by step into float32
  accumulators, then the closed-form diagonal gradients): out, lse, dq, dkd and dvd on a
  row sample of all heads against the oracle (a row's values need only its own score
  row); the ring chain's dK0 / dV0 accumulators against the one-pass gradients;
- the frozen-target forward (head-major, num_blocks = 1) on the same rows against the
  oracle with no diagonal blocks."""
import numpy as np
import pytest
import torch

import eagle_draft_amd as e3
import oracle
import synth
from tests.parity import TOL, rel, say, stored_out
from tests.test_gpu_workloads import oracle_rows, sample_rows

pytestmark = pytest.mark.gpu

W = synth.Workload("ring_contig_r7", "bf16", 1, 32768, 32, 128, 8, layout="contiguous", cp=8, rank=7)


def row_metrics(w, rows, ref, out, lse, dq=None, dkd=None, dvd=None, heads_major=False):
    f = lambda x: x.double().cpu().numpy()
    m = {"out": 0.0, "lse": 0.0}
    if dq is not None:
        m.update({"dq": 0.0, "dkd": 0.0, "dvd": 0.0})
    for h in range(w.H):
        o = out[0, h, rows] if heads_major else out[0, rows, h]
        m["out"] = max(m["out"], float(np.abs(f(o) - ref["out"][h]).max()))
        m["lse"] = max(m["lse"], float(np.abs(f(lse[0, h, rows]) - ref["lse"][h]).max()))
        if dq is not None:
            m["dq"] = max(m["dq"], rel(f(dq[0, rows, h]), ref["dq"][h]))
            m["dkd"] = max(m["dkd"], rel(f(dkd[0][:, rows][:, :, h]), ref["dkd"][h]))
            m["dvd"] = max(m["dvd"], rel(f(dvd[0][:, rows][:, :, h]), ref["dvd"][h]))
    return m


def check(m, t):
    assert m["out"] <= t["out"] and m["lse"] <= t["lse"], m
    for k in ("dq", "dkd", "dvd"):
        if k in m:
            assert m[k] <= t["grad"], (k, m)


@pytest.mark.timeout(900)
def test_one_pass_and_ring_step_mode_at_the_extras_size():
    w = W
    say(f"[extras] generating inputs {w}")
    inp = synth.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    prob = e3.Problem(w.B, w.T, w.T_kv, w.H, w.D, w.num_blocks, w.scale, dtype=torch.bfloat16,
                      layout=w.layout, cp=w.cp, rank=w.rank, device="cuda")
    out, lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
    dq, dk0, dv0, dkd, dvd = e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse)

    B, T, H, D = w.B, w.T, w.H, w.D
    acc_o = torch.zeros(B, T, H, D, dtype=torch.float32, device="cuda")
    acc_l = torch.full((B, H, T), float("-inf"), dtype=torch.float32, device="cuda")
    for j in range(w.cp):
        so, sl = e3.ring_fwd_step(prob, j, d["q"], d["k0"], d["v0"])
        e3.lse_merge(acc_o, acc_l, so, sl)
    rout, rlse = e3.diag_merge_fwd(prob, d["q"], d["kd"], d["vd"], acc_o, acc_l)
    dq_acc = torch.zeros(B, T, H, D, dtype=torch.float32, device="cuda")
    dk_acc = torch.zeros(B, w.T_kv, H, D, dtype=torch.float32, device="cuda")
    dv_acc = torch.zeros_like(dk_acc)
    for j in range(w.cp):
        e3.ring_bwd_step(prob, j, d["dout"], d["q"], d["k0"], d["v0"], out, lse, dq_acc, dk_acc, dv_acc)
    rdq, rdkd, rdvd = e3.diag_bwd(prob, d["dout"], d["q"], d["kd"], d["vd"], out, lse, dq_acc)
    torch.cuda.synchronize()
    for name, x in (("out", out), ("lse", lse), ("dq", dq), ("dk0", dk0), ("dv0", dv0), ("dkd", dkd),
                    ("dvd", dvd), ("ring out", rout), ("ring dq", rdq), ("ring dk0", dk_acc)):
        assert torch.isfinite(x.float()).all(), name

    # the ring chain's block-0 key gradients (float32) against the one-pass ones (bf16)
    t = TOL[w.dtype]
    for name, a, b in (("dk0", dk_acc, dk0), ("dv0", dv_acc, dv0)):
        e = rel(a.double().cpu().numpy(), b.double().cpu().numpy())
        say(f"[extras] ring {name} vs one pass: {e:.3g}")
        assert e <= t["grad"], (name, e)

    rows = torch.from_numpy(sample_rows(w))
    say(f"[extras] oracle on {len(rows)} rows x {w.H} heads")
    ref = oracle_rows(w, inp, rows)
    m1 = row_metrics(w, rows, ref, out.cpu(), lse.cpu(), dq.cpu(), dkd.cpu(), dvd.cpu())
    m2 = row_metrics(w, rows, ref, rout.cpu(), rlse.cpu(), rdq.cpu(), rdkd.cpu(), rdvd.cpu())
    say(f"[extras] one pass (worst head): {m1}")
    say(f"[extras] ring steps (worst head): {m2}")
    check(m1, t)
    check(m2, t)


@pytest.mark.timeout(900)
def test_frozen_target_forward_at_the_extras_size():
    w = W
    say(f"[extras] frozen-target forward: generating inputs {w}")
    inp = synth.make_inputs(w)
    p1 = e3.Problem(w.B, w.T, w.T_kv, w.H, w.D, 1, w.scale, dtype=torch.bfloat16, layout=w.layout,
                    cp=w.cp, rank=w.rank, device="cuda")
    hm = lambda x: x.permute(0, 2, 1, 3).contiguous().cuda()
    oh, lh = e3.target_cp_fwd(p1, hm(inp["q"]), hm(inp["k0"]), hm(inp["v0"]))
    torch.cuda.synchronize()
    assert torch.isfinite(oh.float()).all() and torch.isfinite(lh).all()
    rows = sample_rows(w)
    qpos = oracle.query_positions(w.layout, w.T, w.cp, w.rank)[rows]
    f = lambda x: x.double().numpy()
    ref = {"out": [], "lse": []}
    empty = np.zeros((0, len(rows), w.D))
    for h in range(w.H):
        o, l = oracle.forward_head(f(inp["q"][0, rows, h]), f(inp["k0"][0, :, h]), f(inp["v0"][0, :, h]),
                                   empty, empty, w.scale, qpos, None, rows=len(rows))
        ref["out"].append(o)
        ref["lse"].append(l)
    m = row_metrics(w, torch.from_numpy(rows), ref, oh.cpu(), lh.cpu(), heads_major=True)
    say(f"[extras] frozen-target forward (worst head): {m}")
    check(m, TOL[w.dtype])
