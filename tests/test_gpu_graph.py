"""The forward and the split backward captured in one HIP graph, as a training step
that is replayed: the library allocates nothing, synchronises nothing and issues no
memset, and the backward's side stream (fork after dQ, join after dK/dV) joins the
capture through its events. After one eager step (which creates the side stream), a
step is captured once and replayed three times with new q and dout copied in eagerly
between the replays; every output of every replay is compared bitwise with an eager
step on the same inputs (the kernels are deterministic)."""
import pytest
import torch

import eagle_draft_amd as e3
import synth
from tests.parity import inputs, problem, say

pytestmark = pytest.mark.gpu

W = synth.small_workload


@pytest.mark.parametrize("w", [
    W(S=900, H=3, D=128, num_blocks=4, doc_lens=[300, 1, 599], seed=31),
    W(S=1024, H=2, D=64, num_blocks=3, layout="zigzag", cp=2, rank=1, seed=32),
], ids=["docs_d128", "zigzag_d64"])
def test_forward_and_backward_replay_under_graph_capture(w):
    d = {k: v.cuda() for k, v in inputs(w).items()}
    prob = problem(w)
    q, dout = d["q"].clone(), d["dout"].clone()
    out, lse = torch.empty_like(q), torch.empty(w.B, w.H, w.T, dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(d["k0"]), torch.empty_like(d["v0"]),
             torch.empty_like(d["kd"]), torch.empty_like(d["vd"]))
    ws = torch.empty(max(prob.workspace_bytes(), 256), dtype=torch.uint8, device="cuda")

    def step(o, l, g):
        e3.fwd(prob, q, d["k0"], d["v0"], d["kd"], d["vd"], out=o, lse=l)
        e3.bwd(prob, dout, q, d["k0"], d["v0"], d["kd"], d["vd"], o, l, grads=g, workspace=ws)

    step(out, lse, grads)                       # eager: creates the side stream and its events
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out, lse, grads)
    torch.cuda.synchronize()
    names = ("out", "lse", "dq", "dk0", "dv0", "dkd", "dvd")
    for r in range(3):
        q.copy_(d["q"] * (1.0 + 0.25 * r))
        dout.copy_(d["dout"] * (0.5 + r))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [out.clone(), lse.clone()] + [x.clone() for x in grads]
        ref_out, ref_lse = torch.empty_like(out), torch.empty_like(lse)
        ref_g = tuple(torch.empty_like(x) for x in grads)
        step(ref_out, ref_lse, ref_g)
        torch.cuda.synchronize()
        for n, a, b in zip(names, got, [ref_out, ref_lse] + list(ref_g)):
            assert torch.equal(a, b), (r, n)
        say(f"[graph] {w}: replay {r} bitwise equal to an eager step")
