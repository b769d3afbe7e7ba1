"""The backward that allocates nothing (eagle3_bwd_noalloc, for callers that cannot
allocate device memory) against the backward with a workspace whose kernels it
shares (eagle3_shard_bwd): two calls in a row,
the second with a smaller input, each compared at the parity tolerances; the
K/V and diagonal gradients come from the same kernels and must be bitwise equal,
dq differs only by the rounding of its block-0 part to q's dtype. The same holds on
a float32 contiguous share with documents, a multi-document zig-zag share at D = 64,
a head shard and num_blocks = 12."""
import pytest
import torch

import eagle_draft_amd as e3
import synth
from tests.parity import TOL, inputs, problem, rel, say

pytestmark = pytest.mark.gpu

W = synth.small_workload


def run_both(w):
    inp = inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    prob = problem(w)
    out, lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
    ref = e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse)
    grads = tuple(torch.full_like(g, float("nan")) for g in ref)
    got = e3.bwd_noalloc(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse, grads)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_backward_matches_the_workspace_backward_twice():
    big = W(S=1200, H=3, D=128, num_blocks=4, doc_lens=[500, 1, 699], seed=2)
    small = W(S=256, H=2, D=128, num_blocks=3, layout="zigzag", cp=2, rank=1, seed=3)
    for w in (big, small):
        say(f"[noalloc] {w}")
        ref, got = run_both(w)
        t = TOL[w.dtype]
        names = ("dq", "dk0", "dv0", "dkd", "dvd")
        for n, a, b in zip(names, ref, got):
            assert torch.isfinite(b.float()).all(), n          # every element written
        for n, a, b in zip(names[1:], ref[1:], got[1:]):
            assert torch.equal(a, b), n
        err = rel(got[0].double().cpu().numpy(), ref[0].double().cpu().numpy())
        say(f"[noalloc] dq relative difference {err:.3g}")
        assert err <= t["grad"]


@pytest.mark.parametrize("w", [
    W(dtype="f32", S=300, H=2, D=64, num_blocks=3, layout="contiguous", cp=3, rank=2, chunk=100,
      doc_lens=[40, 1, 259], seed=5),
    W(S=960, H=2, D=64, num_blocks=4, layout="zigzag", cp=2, rank=1, doc_lens=[260, 4, 696], seed=6),
    W(S=768, H=3, D=128, num_blocks=5, layout="headshard", cp=4, doc_lens=[500, 268], seed=7),
    W(S=200, H=2, D=128, num_blocks=12, seed=8),
], ids=["f32_contig_docs", "zigzag_docs_d64", "headshard", "nb12"])
def test_noalloc_backward_on_more_shares(w):
    say(f"[noalloc] {w}")
    ref, got = run_both(w)
    t = TOL[w.dtype]
    names = ("dq", "dk0", "dv0", "dkd", "dvd")
    for n, b in zip(names, got):
        assert torch.isfinite(b.float()).all(), n
    for n, a, b in zip(names[1:], ref[1:], got[1:]):
        assert torch.equal(a, b), n
    assert rel(got[0].double().cpu().numpy(), ref[0].double().cpu().numpy()) <= t["grad"]


def test_noalloc_backward_replays_under_graph_capture():
    """The callers this entry point is for capture it in a HIP graph: captured once
    (after one eager call, which looks the scratch address up), replayed three times
    with new dout values copied in eagerly between the replays, and every replay
    bitwise equal to an eager call on the same inputs."""
    w = W(S=640, H=2, D=128, num_blocks=4, doc_lens=[300, 340], seed=9)
    inp = inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    prob = problem(w)
    out, lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
    dout = d["dout"].clone()
    args = lambda: (prob, dout, d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse)
    grads = (torch.empty_like(d["q"]), torch.empty_like(d["k0"]), torch.empty_like(d["v0"]),
             torch.empty_like(d["kd"]), torch.empty_like(d["vd"]))
    e3.bwd_noalloc(*args(), grads)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        e3.bwd_noalloc(*args(), grads)
    torch.cuda.synchronize()
    for r in range(3):
        dout.copy_(d["dout"] * (0.5 + r))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = e3.bwd_noalloc(*args(), tuple(torch.empty_like(x) for x in grads))
        torch.cuda.synchronize()
        for n, a, b in zip(("dq", "dk0", "dv0", "dkd", "dvd"), grads, ref):
            assert torch.equal(a, b), (r, n)
        say(f"[noalloc] graph replay {r}: bitwise equal to the eager call")
