"""GPU parity of ring-step mode, the single-GPU half of the ring protocol
(ring_attention page, `ring_flash_attn_forward` / `ring_flash_attn_backward`,
`_update_out_and_lse`, `_merge_diag`; zigzag_ring_attention page,
`zigzag_ring_flash_attn_varlen_forward` / `_backward`, `RingComm`):

  * every ring step's partial (out, lse) equals the oracle's attention of the
    share's rows over exactly that step's keys (rows that see none: out = 0,
    lse = -inf);
  * the steps chained through the lse_merge kernel, then the diagonal merge,
    equal the oracle's joint softmax and the one-pass shard forward;
  * the backward run step by step for EVERY rank of the ring, with the K/V
    gradients of each step added into accumulators that stand for the rotated
    dK/dV buffers, gives each rank's dq, dkd, dvd and, summed over ranks, the
    full-sequence dk0, dv0 of the oracle;

on fixed shares and on seeded random ones (layout, degree, rank, documents,
num_blocks, head dim, dtype)."""
import dataclasses
import random

import numpy as np
import pytest
import torch

import eagle_draft_amd as e3
import oracle
import synth
from tests.parity import TOL, compare, inputs, problem, rel, run_hip, run_oracle, say, stored_out

pytestmark = pytest.mark.gpu

W = synth.small_workload
CASES = {
    "contig_cp4": W(S=1024, H=2, D=128, num_blocks=3, layout="contiguous", cp=4, rank=2, chunk=256),
    "contig_docs_cp3": W(S=900, H=2, D=128, num_blocks=4, layout="contiguous", cp=3, rank=1,
                         doc_lens=[100, 350, 450], chunk=300),
    "zigzag_cp4": W(S=1024, H=2, D=128, num_blocks=3, layout="zigzag", cp=4, rank=1),
    "zigzag_docs_cp4": W(S=1024, H=2, D=128, num_blocks=3, layout="zigzag", cp=4, rank=3,
                         doc_lens=[8, 400, 0, 616]),
    "zigzag_f32": W(dtype="f32", S=480, H=2, D=64, num_blocks=3, layout="zigzag", cp=3, rank=0,
                    doc_lens=[60, 6, 414]),
    "zigzag_d64": W(S=512, H=2, D=64, num_blocks=3, layout="zigzag", cp=2, rank=0),
    # no diagonal blocks: the diagonal kernel only turns the float32 dq into q's dtype
    "contig_nb1": W(S=512, H=3, D=128, num_blocks=1, layout="contiguous", cp=2, rank=1, chunk=256),
}


def ring_fuzz_case(i):
    """Seeded random ring shares: contiguous (random documents) or zig-zag (documents
    whose lengths are multiples of 2cp), cp 2..4, any rank, num_blocks 1..5, both
    head dims and dtypes, lengths that match no tile size."""
    rng = random.Random(7000 + i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    D = rng.choice([64, 128])
    cp = rng.randint(2, 4)
    kw = dict(dtype=dtype, D=D, H=rng.randint(1, 3), num_blocks=rng.randint(1, 5), seed=100 + i, cp=cp,
              rank=rng.randrange(cp))
    if i % 2 == 0:
        t = rng.randint(33, 260)
        S = cp * t
        docs = None
        if rng.random() < 0.6:
            docs, acc = [], 0
            while acc < S:
                n = min(rng.choice([0, 1, rng.randint(2, 90), rng.randint(60, 500)]), S - acc)
                docs.append(n)
                acc += n
        return W(S=S, layout="contiguous", chunk=t, doc_lens=docs, **kw)
    docs = [2 * cp * rng.choice([0, 1, rng.randint(2, 12), rng.randint(10, 60)]) for _ in range(rng.randint(1, 4))]
    if sum(docs) == 0:
        docs[0] = 2 * cp
    return W(S=sum(docs), layout="zigzag", doc_lens=docs if len(docs) > 1 else None, **kw)


CASES.update({f"fuzz{i}": ring_fuzz_case(i) for i in range(8)})


def step_keys(w, step):
    """Global positions of the block-0 keys held at ring step `step` (rank
    (rank - step) mod cp's K/V: its contiguous shard, or chunks src and
    2cp-1-src of every document)."""
    src = (w.rank - step) % w.cp
    if w.layout == "contiguous":
        return np.arange(src * w.T, (src + 1) * w.T)
    cu = w.cu_seqlens()
    bounds = [(0, w.S)] if cu is None else list(zip(cu[:-1], cu[1:]))
    keys = []
    for lo, hi in bounds:
        c = (hi - lo) // (2 * w.cp)
        for ch in (src, 2 * w.cp - 1 - src):
            keys.append(lo + ch * c + np.arange(c))
    return np.concatenate(keys)


def tol(w):
    return TOL[w.dtype]


@pytest.mark.parametrize("name", list(CASES))
def test_ring_steps_forward(name):
    w = CASES[name]
    say(f"[ring] forward {name}: {w}")
    inp = inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    prob = problem(w)
    cu = w.cu_seqlens()
    qpos = oracle.query_positions(w.layout, w.T, w.cp, w.rank, cu)
    f = lambda t: t.double().numpy()
    out_acc = torch.zeros(w.B, w.T, w.H, w.D, device="cuda")
    lse_acc = torch.full((w.B, w.H, w.T), float("-inf"), device="cuda")
    t = tol(w)
    for j in range(w.cp):
        o_j, l_j = e3.ring_fwd_step(prob, j, d["q"], d["k0"], d["v0"])
        torch.cuda.synchronize()
        keys = step_keys(w, j)
        mask = oracle.visible_mask(qpos, keys, cu)
        for h in range(w.H):
            ro, rl = oracle.block_attention(f(inp["q"][0, :, h]), f(inp["k0"][0, keys, h]),
                                            f(inp["v0"][0, keys, h]), mask, w.scale)
            go, gl = f(o_j[0, :, h].cpu()), f(l_j[0, h].cpu())
            empty = ~np.isfinite(rl)
            assert np.array_equal(empty, ~np.isfinite(gl)), (j, h)
            assert np.all(go[empty] == 0.0)
            assert np.abs(go - ro).max() <= t["out"], (j, h, np.abs(go - ro).max())
            if (~empty).any():
                assert np.abs(gl[~empty] - rl[~empty]).max() <= t["lse"], (j, h)
        e3.lse_merge(out_acc, lse_acc, o_j, l_j)
    out, lse = e3.diag_merge_fwd(prob, d["q"], d["kd"], d["vd"], out_acc, lse_acc)
    one_out, one_lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
    torch.cuda.synchronize()
    ref = run_oracle(w, inp)
    m_out = float(np.abs(f(out.cpu()) - ref[0]).max())
    m_lse = float(np.abs(f(lse.cpu()) - ref[1]).max())
    say(f"[ring] forward {name}: chained vs oracle out {m_out:.3g} lse {m_lse:.3g}; "
        f"vs one pass out {(out.float() - one_out.float()).abs().max().item():.3g}")
    assert m_out <= t["out"] and m_lse <= t["lse"]
    assert (out.float() - one_out.float()).abs().max().item() <= t["out"]
    assert (lse - one_lse).abs().max().item() <= t["lse"]


@pytest.mark.parametrize("name", list(CASES))
def test_ring_steps_backward_all_ranks(name):
    w0 = CASES[name]
    say(f"[ring] backward {name}: every rank of cp={w0.cp}")
    full_w = dataclasses.replace(w0, layout="full", cp=1, rank=0, chunk=w0.gen_chunk())
    full_inp = synth.make_inputs(w0, layout="full")
    ref_full = run_oracle(full_w, full_inp)
    dk0_acc = torch.zeros(w0.B, w0.S, w0.H, w0.D, device="cuda")
    dv0_acc = torch.zeros_like(dk0_acc)
    t = tol(w0)
    worst = {}
    for r in range(w0.cp):
        w = dataclasses.replace(w0, rank=r)
        inp = inputs(w)
        d = {k: v.cuda() for k, v in inp.items()}
        prob = problem(w)
        out, lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
        dq_acc = torch.zeros(w.B, w.T, w.H, w.D, device="cuda")
        ws = torch.empty(max(prob.workspace_bytes(), 256), dtype=torch.uint8, device="cuda")
        for j in range(w.cp):
            e3.ring_bwd_step(prob, j, d["dout"], d["q"], d["k0"], d["v0"], out, lse, dq_acc,
                             dk0_acc, dv0_acc, workspace=ws)
        dq, dkd, dvd = e3.diag_bwd(prob, d["dout"], d["q"], d["kd"], d["vd"], out, lse, dq_acc)
        torch.cuda.synchronize()
        ref = run_oracle(w, inp)
        for k, a, b in (("dq", dq, ref[2][0]), ("dkd", dkd, ref[2][3]), ("dvd", dvd, ref[2][4])):
            if b.size:
                worst[k] = max(worst.get(k, 0.0), rel(a.double().cpu().numpy(), b))
    m = {"dk0": rel(dk0_acc.double().cpu().numpy(), ref_full[2][1]),
         "dv0": rel(dv0_acc.double().cpu().numpy(), ref_full[2][2]), **worst}
    say(f"[ring] backward {name}: {m}")
    for k, v in m.items():
        assert v <= t["grad"], (k, m)
