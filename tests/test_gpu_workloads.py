"""GPU parity on the five workloads at their real sizes, in the launch
configuration bench.py times (the same entry points, grids and tiles): tiny,
dense, packed varlen, Ulysses head share and zig-zag ring rank 3 of cp=8.

Every head is compared with the oracle element by element, except for the
zig-zag share, where two heads (0 and 21) are compared in full -- each costs
about 1.07e9 attended pairs on the host -- and, for all 32 heads, the per-row
outputs (out, lse, dq, dkd, dvd) are compared on a sample of rows (the starts,
middles and ends of both chunks, the rows around query-tile edges and seeded
random rows), whose oracle values need only those rows' score rows. All heads
are also checked for the properties that hold at any size (finite outputs, exact
zeros for the K/V rows no local query sees, the softmax bounds of lse). The
zig-zag share of eight documents that the benchmark also times gets the same
row-sample comparison and property checks."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import TOL, assert_within, compare, rel, run_hip, run_oracle, say, stored_out
from tests.parity import inputs as tinputs

pytestmark = pytest.mark.gpu

CASES = [("tiny", None), ("dense", None), ("packed", None), ("ulysses", None), ("zigzag", [0, 21])]


def check_properties(w, hip):
    out, lse, (dq, dk0, dv0, dkd, dvd) = hip
    for name, t in (("out", out), ("lse", lse), ("dq", dq), ("dk0", dk0), ("dv0", dv0),
                    ("dkd", dkd), ("dvd", dvd)):
        assert torch.isfinite(t.float()).all(), name
    # lse_t >= log(number of keys) + min score is not available without the
    # scores; the joint softmax does give lse_t >= max diagonal score, and
    # lse_t <= max score + log(n_t). Check the cheap lower bound on a sample.
    if w.N > 0:
        q = inp_cache["q"].float()
        kd = inp_cache["kd"].float()
        rows = torch.linspace(0, w.T - 1, 64).long()
        y = w.scale * (q[:, rows].unsqueeze(1) * kd[:, :, rows]).sum(-1)     # [B, N, r, H]
        ymax = y.max(dim=1).values.permute(0, 2, 1)                              # [B, H, r]
        assert (lse[:, :, rows] >= ymax - 1e-2).all()
    if w.layout in ("zigzag", "contiguous"):
        qpos = oracle.query_positions(w.layout, w.T, w.cp, w.rank)
        unseen = np.arange(w.T_kv) > qpos.max()
        idx = torch.from_numpy(np.nonzero(unseen)[0])
        if len(idx):
            assert torch.count_nonzero(dk0[:, idx]) == 0
            assert torch.count_nonzero(dv0[:, idx]) == 0


inp_cache = {}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,heads", CASES)
def test_workload_parity_full_size(name, heads):
    w = synth.workload(name)
    say(f"[workload] {name}: generating inputs {w}")
    inp = synth.make_inputs(w)
    inp_cache.clear()
    inp_cache.update(inp)
    say(f"[workload] {name}: HIP forward + backward")
    hip = run_hip(w, inp)
    check_properties(w, hip)
    say(f"[workload] {name}: oracle on heads {heads if heads is not None else 'all'}")
    ref = run_oracle(w, inp, heads=heads)
    m = compare(w, hip, ref, heads)
    say(f"[workload] {name}: {m}")
    assert_within(w, m)
    inp_cache.clear()


def share_runs(w):
    """Lengths of the share's local runs in local order: the two zig-zag chunks of
    every document (doc_len / 2cp rows each), else the whole share."""
    if w.layout != "zigzag":
        return [w.T]
    docs = w.doc_lens if w.doc_lens is not None else [w.S]
    return [n // (2 * w.cp) for n in docs for _ in range(2)]


def sample_rows(w, n_random=16, seed=0):
    """Row sample of a share: the first, middle and last rows of each run (the
    zig-zag chunks), the rows on both sides of 64- and 128-row tile edges, and
    seeded random rows."""
    rows = set()
    r0 = 0
    for c in share_runs(w):
        for o in (0, 1, 2, 63, 64, 127, 128, 129, c // 2 - 1, c // 2, c - 129, c - 128, c - 65,
                  c - 64, c - 2, c - 1):
            if 0 <= o < c:
                rows.add(r0 + o)
        r0 += c
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, w.T, n_random))
    return np.array(sorted(rows))


def oracle_rows(w, inp, rows):
    """Oracle out, lse, dq, dkd, dvd of the sampled rows for every head; a row's
    values depend only on its own score row, so the oracle runs on those rows
    alone (their global positions passed explicitly)."""
    cu = w.cu_seqlens()
    qpos = oracle.query_positions(w.layout, w.T, w.cp, w.rank, cu)[rows.numpy()]
    f = lambda t: t.double().numpy()
    res = {k: [] for k in ("out", "lse", "dq", "dkd", "dvd")}
    for h in range(w.H):
        q, do = f(inp["q"][0, rows, h]), f(inp["dout"][0, rows, h])
        k0, v0 = f(inp["k0"][0, :, h]), f(inp["v0"][0, :, h])
        kd, vd = f(inp["kd"][0][:, rows][:, :, h]), f(inp["vd"][0][:, rows][:, :, h])
        o, l = oracle.forward_head(q, k0, v0, kd, vd, w.scale, qpos, cu, rows=len(rows))
        dq, _, _, dkd, dvd = oracle.backward_head(do, q, k0, v0, kd, vd, w.scale, qpos, cu,
                                                  out=stored_out(w, o), lse=l, rows=len(rows))
        for k, v in (("out", o), ("lse", l), ("dq", dq), ("dkd", dkd), ("dvd", dvd)):
            res[k].append(v)
    return res


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["zigzag", "zigzag_docs"])
def test_zigzag_share_all_heads_on_sampled_rows(name):
    """zigzag: one 131072-token document; zigzag_docs: eight 16384-token documents,
    each cut into 2cp chunks (the bench's multi-document share). For the latter all
    heads are also checked for the properties that hold at any size."""
    w = synth.workload(name)
    say(f"[workload] {name} row sample: generating inputs {w}")
    inp = tinputs(w)
    say(f"[workload] {name} row sample: HIP forward + backward")
    out, lse, (dq, dk0, dv0, dkd, dvd) = run_hip(w, inp)
    if w.doc_lens is not None:
        for nm, x in (("out", out), ("lse", lse), ("dq", dq), ("dk0", dk0), ("dv0", dv0), ("dkd", dkd),
                      ("dvd", dvd)):
            assert torch.isfinite(x.float()).all(), nm
        cu = w.cu_seqlens()
        qpos = oracle.query_positions(w.layout, w.T, w.cp, w.rank, cu)
        seen = np.zeros(w.T_kv, dtype=bool)
        for lo, hi in zip(cu[:-1], cu[1:]):
            mine = qpos[(qpos >= lo) & (qpos < hi)]
            if len(mine):
                seen[lo:mine.max() + 1] = True
        unseen = torch.from_numpy(np.nonzero(~seen)[0])
        assert len(unseen) > 0
        assert torch.count_nonzero(dk0[:, unseen]) == 0 and torch.count_nonzero(dv0[:, unseen]) == 0
    del dk0, dv0
    rows = torch.from_numpy(sample_rows(w))
    say(f"[workload] {name} row sample: oracle on {len(rows)} rows x {w.H} heads")
    ref = oracle_rows(w, inp, rows)
    t = TOL[w.dtype]
    f = lambda x: x.double().numpy()
    m = {"out": 0.0, "lse": 0.0, "dq": 0.0, "dkd": 0.0, "dvd": 0.0}
    for h in range(w.H):
        m["out"] = max(m["out"], float(np.abs(f(out[0, rows, h]) - ref["out"][h]).max()))
        m["lse"] = max(m["lse"], float(np.abs(f(lse[0, h, rows]) - ref["lse"][h]).max()))
        m["dq"] = max(m["dq"], rel(f(dq[0, rows, h]), ref["dq"][h]))
        m["dkd"] = max(m["dkd"], rel(f(dkd[0][:, rows][:, :, h]), ref["dkd"][h]))
        m["dvd"] = max(m["dvd"], rel(f(dvd[0][:, rows][:, :, h]), ref["dvd"][h]))
    say(f"[workload] {name} row sample (worst head): {m}")
    assert m["out"] <= t["out"] and m["lse"] <= t["lse"], m
    for k in ("dq", "dkd", "dvd"):
        assert m[k] <= t["grad"], (k, m)
