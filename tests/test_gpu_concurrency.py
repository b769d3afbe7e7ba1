"""Calls from several host threads at once, each on its own stream: the library keeps
its per-call state per host thread (error text, timing events, the backward's side
stream and its fork/join events), so concurrent callers must get exactly the
results of serial calls. Two threads run five forward + backward steps each on two
different problems (bf16 D=128 with documents, bf16 D=64 zig-zag) while the other
runs; every output of every step is compared bitwise with a serial run (the kernels
are deterministic)."""
import threading

import pytest
import torch

import eagle_draft_amd as e3
import synth
from tests.parity import inputs, problem, say

pytestmark = pytest.mark.gpu

W = synth.small_workload
CASES = {
    "docs_d128": W(S=900, H=3, D=128, num_blocks=4, doc_lens=[300, 1, 599], seed=21),
    "zigzag_d64": W(S=1024, H=2, D=64, num_blocks=3, layout="zigzag", cp=2, rank=1, seed=22),
}
STEPS = 5


def step(prob, d):
    out, lse = e3.fwd(prob, d["q"], d["k0"], d["v0"], d["kd"], d["vd"])
    g = e3.bwd(prob, d["dout"], d["q"], d["k0"], d["v0"], d["kd"], d["vd"], out, lse)
    return (out, lse) + tuple(g)


def test_two_host_threads_on_their_own_streams_match_serial_calls():
    data = {n: ({k: v.cuda() for k, v in inputs(w).items()}, problem(w)) for n, w in CASES.items()}
    ref = {}
    for n, (d, prob) in data.items():
        ref[n] = [x.clone() for x in step(prob, d)]
    torch.cuda.synchronize()

    results, errors = {}, []

    def worker(n):
        try:
            d, prob = data[n]
            s = torch.cuda.Stream()
            got = []
            with torch.cuda.stream(s):
                for _ in range(STEPS):
                    got.append([x.clone() for x in step(prob, d)])
            s.synchronize()
            results[n] = got
        except Exception as exc:   # re-raised in the main thread
            errors.append((n, exc))

    threads = [threading.Thread(target=worker, args=(n,)) for n in CASES]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    names = ("out", "lse", "dq", "dk0", "dv0", "dkd", "dvd")
    for n in CASES:
        assert len(results[n]) == STEPS
        for i, got in enumerate(results[n]):
            for name, a, b in zip(names, ref[n], got):
                assert torch.equal(a, b), (n, i, name)
        say(f"[threads] {n}: {STEPS} concurrent steps bitwise equal to the serial call")
