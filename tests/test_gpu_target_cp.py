"""GPU parity of the frozen-target context-parallel forward (target_cp page,
`attach_cp_kv_gather_hooks`): a rank's contiguous local queries against the
all-gathered K/V, masked causally by global position, head-major [B, nH, S, D] tensors,
forward only. It is the contiguous share with num_blocks = 1, so it is compared
with the oracle's forward of that share, and with the token-major shard
forward of the library (the same kernel over other strides: bitwise equal)."""
import random

import numpy as np
import pytest
import torch

import eagle_draft_amd as e3
import oracle
import synth
from tests.parity import TOL, problem, say

pytestmark = pytest.mark.gpu

W = synth.small_workload
CASES = {
    "cp4_r0": W(S=1024, H=2, D=128, num_blocks=1, layout="contiguous", cp=4, rank=0, chunk=256),
    "cp4_r3": W(S=1024, H=3, D=128, num_blocks=1, layout="contiguous", cp=4, rank=3, chunk=256),
    "cp3_docs": W(S=900, H=2, D=128, num_blocks=1, layout="contiguous", cp=3, rank=2,
                  doc_lens=[100, 350, 450], chunk=300),
    "full_ragged": W(S=517, H=2, D=128, num_blocks=1),
    "cp2_b2_d64": W(B=2, S=600, H=2, D=64, num_blocks=1, layout="contiguous", cp=2, rank=1, chunk=300),
    "f32_cp4": W(dtype="f32", S=512, H=2, D=64, num_blocks=1, layout="contiguous", cp=4, rank=2, chunk=128),
}


def _fuzz(i):
    """Seeded random contiguous shares: degree, rank, batch rows or documents,
    head dim, dtype, lengths that match no tile size."""
    rng = random.Random(8000 + i)
    cp = rng.randint(1, 5)
    t = rng.randint(1, 300)
    S = cp * t
    kw = dict(dtype="f32" if i % 3 == 2 else "bf16", D=rng.choice([64, 128]), H=rng.randint(1, 3), num_blocks=1,
              seed=200 + i, layout="contiguous", cp=cp, rank=rng.randrange(cp), chunk=t)
    if rng.random() < 0.5:
        docs, acc = [], 0
        while acc < S:
            n = min(rng.choice([0, 1, rng.randint(2, 120), rng.randint(100, 600)]), S - acc)
            docs.append(n)
            acc += n
        return W(S=S, doc_lens=docs, **kw)
    return W(S=S, B=rng.randint(1, 2), **kw)


CASES.update({f"fuzz{i}": _fuzz(i) for i in range(6)})


@pytest.mark.parametrize("name", list(CASES))
def test_target_cp_forward(name):
    w = CASES[name]
    say(f"[target-cp] {name}: {w}")
    inp = synth.make_inputs(w)
    prob = problem(w)
    hm = lambda t: t.permute(0, 2, 1, 3).contiguous().cuda()      # [B,T,H,D] -> [B,H,T,D]
    out, lse = e3.target_cp_fwd(prob, hm(inp["q"]), hm(inp["k0"]), hm(inp["v0"]))
    out_nolse, none = e3.target_cp_fwd(prob, hm(inp["q"]), hm(inp["k0"]), hm(inp["v0"]), want_lse=False)
    tok_out, tok_lse = e3.fwd(prob, inp["q"].cuda(), inp["k0"].cuda(), inp["v0"].cuda())
    torch.cuda.synchronize()
    assert none is None and torch.equal(out_nolse, out)
    assert torch.equal(out.permute(0, 2, 1, 3).cpu(), tok_out.cpu())
    assert torch.equal(lse.cpu(), tok_lse.cpu())
    cu = w.cu_seqlens()
    qpos = oracle.query_positions(w.layout, w.T, w.cp, w.rank, cu)
    f = lambda t: t.double().numpy()
    worst_o = worst_l = 0.0
    for b in range(w.B):
        for h in range(w.H):
            empty = np.zeros((0, w.T, w.D))
            ro, rl = oracle.forward_head(f(inp["q"][b, :, h]), f(inp["k0"][b, :, h]), f(inp["v0"][b, :, h]),
                                         empty, empty, w.scale, qpos, cu)
            worst_o = max(worst_o, float(np.abs(f(out[b, h].cpu()) - ro).max()))
            worst_l = max(worst_l, float(np.abs(f(lse[b, h].cpu()) - rl).max()))
    say(f"[target-cp] {name}: out {worst_o:.3g} lse {worst_l:.3g}")
    t = TOL[w.dtype]
    assert worst_o <= t["out"] and worst_l <= t["lse"]
