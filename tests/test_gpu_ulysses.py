"""GPU tests of the Ulysses re-sharding transforms (ulysses_attention page:
`_gather_seq_scatter_heads`, `_scatter_seq_gather_heads`, `_gather_lse`,
`_scatter_lse`, around `_all_to_all_single`), with the all-to-all itself
emulated on one GPU by indexing (part i of rank r's send buffer is part r of
rank i's receive buffer):

  * each transform gives exactly the re-sharded tensor and the pairs invert each
    other (bit-exact copies);
  * the whole Ulysses path run for every rank -- gather q, k0, v0 to head
    shards, block 0 over the full sequence on the head shard, out and lse back
    to the sequence shard, the diagonal blocks merged there; backward likewise
    with the merged out/lse -- equals the oracle's joint softmax and gradients."""
import random

import numpy as np
import pytest
import torch

import eagle_draft_amd as e3
import oracle
import synth
from tests.parity import TOL, rel, run_oracle, say

pytestmark = pytest.mark.gpu


def a2a(sends):
    """Emulated all_to_all_single over dim 0 with equal splits: rank r receives
    part r of every rank's send buffer, in rank order."""
    uly = len(sends)
    return [torch.stack([sends[i][r] for i in range(uly)], 0).contiguous() for r in range(uly)]


def _random_shapes(n):
    """Seeded random transform shapes: odd lengths, head counts that divide by the
    degree, and head dims whose rows are not 16-byte multiples (the 4-byte copies)."""
    rng = random.Random(9000)
    out = []
    for _ in range(n):
        uly = rng.randint(1, 8)
        out.append((rng.randint(1, 2), rng.randint(1, 97), uly * rng.randint(1, 4), rng.choice([2, 6, 64, 128]),
                    uly))
    return out + [(1, 9, 6, 3, 2)]       # a row of 3 elements: float32 copies it, bf16 is refused


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("B,S_local,H,D,uly", [(1, 64, 8, 128, 4), (2, 37, 6, 64, 3), (1, 5, 4, 128, 1),
                                               (1, 130, 16, 128, 8),
                                               (1, 4096, 32, 128, 8)]    # the size bench.py --extras times
                         + _random_shapes(6))
def test_transforms_are_exact_and_invert(dtype, B, S_local, H, D, uly):
    if dtype == torch.bfloat16 and (H // uly * D) % 2:
        x = torch.zeros(B, S_local, H, D, dtype=dtype, device="cuda")
        with pytest.raises(e3.E3Error, match="multiple of 4 bytes"):
            e3.ulysses("seq_to_head", 0, x, uly, B, S_local, H, D)
        return
    g = torch.Generator().manual_seed(B * 1000 + S_local)
    Sf, Hl = uly * S_local, H // uly
    X = torch.randn(B, Sf, H, D, generator=g).to(dtype).cuda()
    L = torch.randn(B, H, Sf, generator=g).cuda()
    xs = [X[:, r * S_local:(r + 1) * S_local].contiguous() for r in range(uly)]
    ys = [e3.ulysses("seq_to_head", 1, rv, uly, B, S_local, H, D)
          for rv in a2a([e3.ulysses("seq_to_head", 0, x, uly, B, S_local, H, D) for x in xs])]
    for r in range(uly):
        assert torch.equal(ys[r], X[:, :, r * Hl:(r + 1) * Hl])
    back = [e3.ulysses("head_to_seq", 1, rv, uly, B, S_local, H, D)
            for rv in a2a([e3.ulysses("head_to_seq", 0, y, uly, B, S_local, H, D) for y in ys])]
    for r in range(uly):
        assert torch.equal(back[r], xs[r])
    ls = [L[:, :, r * S_local:(r + 1) * S_local].contiguous() for r in range(uly)]
    lg = [e3.ulysses("lse_gather", 1, rv, uly, B, S_local, H)
          for rv in a2a([e3.ulysses("lse_gather", 0, l, uly, B, S_local, H) for l in ls])]
    for r in range(uly):
        assert lg[r].is_contiguous() and torch.equal(lg[r], L[:, r * Hl:(r + 1) * Hl])
    lb = [e3.ulysses("lse_scatter", 1, rv, uly, B, S_local, H)
          for rv in a2a([e3.ulysses("lse_scatter", 0, l, uly, B, S_local, H) for l in lg])]
    for r in range(uly):
        assert torch.equal(lb[r], ls[r])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ulysses_path_end_to_end(dtype):
    uly, H, D = 4, 8, 128 if dtype == "bf16" else 64
    Sf = 4 * 192
    Sl, Hl, N = Sf // uly, H // uly, 3
    w = synth.small_workload(dtype=dtype, S=Sf, H=H, D=D, num_blocks=N + 1, seed=41,
                             doc_lens=[300, 5, 463])
    say(f"[ulysses] end to end {dtype}: uly={uly} {w}")
    inp = synth.make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    cu = w.cu_seqlens()
    tdt = w.torch_dtype
    seq = lambda t, r: t[:, r * Sl:(r + 1) * Sl].contiguous()          # sequence shard of rank r
    seq_d = lambda t, r: t[:, :, r * Sl:(r + 1) * Sl].contiguous()     # of a [B, N, S, H, D] tensor

    def gather(t):               # sequence shards of every rank -> head shards
        sends = [e3.ulysses("seq_to_head", 0, seq(t, r), uly, 1, Sl, H, D) for r in range(uly)]
        return [e3.ulysses("seq_to_head", 1, rv, uly, 1, Sl, H, D) for rv in a2a(sends)]

    def scatter(parts):          # head shards of every rank -> sequence shards
        sends = [e3.ulysses("head_to_seq", 0, p, uly, 1, Sl, H, D) for p in parts]
        return [e3.ulysses("head_to_seq", 1, rv, uly, 1, Sl, H, D) for rv in a2a(sends)]

    qh, kh, vh = gather(d["q"]), gather(d["k0"]), gather(d["v0"])
    # block 0 on each head shard (the full sequence, H/uly heads), float32 (out, lse)
    o0, l0 = [], []
    for r in range(uly):
        ph = e3.Problem(1, Sf, Sf, Hl, D, 1, w.scale, dtype=tdt, layout="headshard", cp=uly, rank=r,
                        cu_seqlens=cu, device="cuda")
        o, l = e3.ring_fwd_step(ph, 0, qh[r], kh[r], vh[r])
        o0.append(o)
        l0.append(l)
    o0s = scatter(o0)
    lsends = [e3.ulysses("lse_scatter", 0, l, uly, 1, Sl, H) for l in l0]
    l0s = [e3.ulysses("lse_scatter", 1, rv, uly, 1, Sl, H) for rv in a2a(lsends)]
    # diagonal merge on each sequence shard (all heads): the sequence shard is the
    # contiguous share of rank r
    outs, lses, probs = [], [], []
    for r in range(uly):
        ps = e3.Problem(1, Sl, Sf, H, D, N + 1, w.scale, dtype=tdt, layout="contiguous", cp=uly, rank=r,
                        cu_seqlens=cu, device="cuda")
        o, l = e3.diag_merge_fwd(ps, seq(d["q"], r), seq_d(d["kd"], r), seq_d(d["vd"], r), o0s[r], l0s[r])
        outs.append(o)
        lses.append(l)
        probs.append(ps)
    out = torch.cat(outs, 1)
    lse = torch.cat(lses, 2)
    # backward: gather dout, out and lse to the head shards, block 0 there against
    # the merged out/lse, gradients back, diagonal gradients on the sequence shards
    doh, oh = gather(d["dout"]), gather(out)
    lg = [e3.ulysses("lse_gather", 1, rv, uly, 1, Sl, H)
          for rv in a2a([e3.ulysses("lse_gather", 0, lses[r], uly, 1, Sl, H) for r in range(uly)])]
    dqh, dkh, dvh = [], [], []
    for r in range(uly):
        ph = e3.Problem(1, Sf, Sf, Hl, D, 1, w.scale, dtype=tdt, layout="headshard", cp=uly, rank=r,
                        cu_seqlens=cu, device="cuda")
        dq_acc = torch.zeros(1, Sf, Hl, D, device="cuda")
        dk_acc = torch.zeros(1, Sf, Hl, D, device="cuda")
        dv_acc = torch.zeros(1, Sf, Hl, D, device="cuda")
        e3.ring_bwd_step(ph, 0, doh[r], qh[r], kh[r], vh[r], oh[r], lg[r], dq_acc, dk_acc, dv_acc)
        dqh.append(dq_acc)
        dkh.append(dk_acc)
        dvh.append(dv_acc)
    dq_s, dk0_s, dv0_s = scatter(dqh), scatter(dkh), scatter(dvh)
    dqs, dkds, dvds = [], [], []
    for r in range(uly):
        dq, dkd, dvd = e3.diag_bwd(probs[r], seq(d["dout"], r), seq(d["q"], r), seq_d(d["kd"], r),
                                   seq_d(d["vd"], r), outs[r], lses[r], dq_s[r])
        dqs.append(dq)
        dkds.append(dkd)
        dvds.append(dvd)
    torch.cuda.synchronize()
    ref = run_oracle(w, inp)
    f = lambda t: t.double().cpu().numpy()
    m = {"out": float(np.abs(f(out) - ref[0]).max()), "lse": float(np.abs(f(lse) - ref[1]).max()),
         "dq": rel(f(torch.cat(dqs, 1)), ref[2][0]), "dk0": rel(f(torch.cat(dk0_s, 1)), ref[2][1]),
         "dv0": rel(f(torch.cat(dv0_s, 1)), ref[2][2]), "dkd": rel(f(torch.cat(dkds, 2)), ref[2][3]),
         "dvd": rel(f(torch.cat(dvds, 2)), ref[2][4])}
    say(f"[ulysses] end to end {dtype}: {m}")
    t = TOL[dtype]
    assert m["out"] <= t["out"] and m["lse"] <= t["lse"], m
    for k in ("dq", "dk0", "dv0", "dkd", "dvd"):
        assert m[k] <= t["grad"], (k, m)
