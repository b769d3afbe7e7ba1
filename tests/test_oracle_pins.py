"""Pins for the CPU oracle: each test ties the oracle to something other than
itself (a library routine on a reduced problem, finite differences, brute force,
closed forms, invariants the mathematics fixes, and the layout statements of the
pages). A plausible mistake anywhere in the oracle (a dropped term, a wrong sign
or index, a transposed operand) fails at least one of these; the planted-mistake
tests at the bottom check that for a few such mistakes."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rand_problem(rng, B=1, T=24, Tkv=None, H=2, D=8, nb=3, scale=None):
    Tkv = T if Tkv is None else Tkv
    N = nb - 1
    p = dict(
        q=rng.standard_normal((B, T, H, D)),
        k0=rng.standard_normal((B, Tkv, H, D)),
        v0=rng.standard_normal((B, Tkv, H, D)),
        kd=rng.standard_normal((B, N, T, H, D)),
        vd=rng.standard_normal((B, N, T, H, D)),
        dout=rng.standard_normal((B, T, H, D)),
    )
    p["scale"] = 1.0 / math.sqrt(D) if scale is None else scale
    return p


# ---------------------------------------------------------------------------
# Library reduction: SDPA over an augmented key set with a boolean mask
# ---------------------------------------------------------------------------

def explicit_mask(qpos, Tkv, N, docs):
    """Boolean mask over the augmented keys [k0 (Tkv) | kd_1 (T) | ... | kd_N (T)],
    built with plain loops: block-0 key s is visible to query t iff s <= pos(t)
    and both lie in the same document; diagonal key (i, t') iff t' == t."""
    T = len(qpos)
    m = np.zeros((T, Tkv + N * T), dtype=bool)
    for t in range(T):
        g = int(qpos[t])
        for (a, b) in docs:
            if a <= g < b:
                for s in range(a, g + 1):
                    m[t, s] = True
        for i in range(N):
            m[t, Tkv + i * T + t] = True
    return m


def sdpa_reference(p, qpos, docs):
    """out, lse, dq, dk0, dv0, dkd, dvd via torch SDPA + autograd in float64."""
    q = torch.tensor(p["q"], requires_grad=True)
    k0 = torch.tensor(p["k0"], requires_grad=True)
    v0 = torch.tensor(p["v0"], requires_grad=True)
    kd = torch.tensor(p["kd"], requires_grad=True)
    vd = torch.tensor(p["vd"], requires_grad=True)
    B, T, H, D = q.shape
    N = kd.shape[1]
    Tkv = k0.shape[1]
    kaug = torch.cat([k0] + [kd[:, i] for i in range(N)], dim=1)   # [B, Tkv+N*T, H, D]
    vaug = torch.cat([v0] + [vd[:, i] for i in range(N)], dim=1)
    mask = torch.tensor(explicit_mask(qpos, Tkv, N, docs))
    qh, kh, vh = (x.transpose(1, 2) for x in (q, kaug, vaug))
    out = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=p["scale"])
    out = out.transpose(1, 2)
    scores = torch.matmul(qh, kh.transpose(-1, -2)) * p["scale"]
    lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)   # [B,H,T]
    (out * torch.tensor(p["dout"])).sum().backward()
    def g(t):
        return np.zeros(t.shape) if t.grad is None else t.grad.numpy()
    return (out.detach().numpy(), lse.detach().numpy(), g(q), g(k0), g(v0), g(kd), g(vd))


CASES = [
    # (layout, T_local, cp, rank, docs over the global sequence or None, nb, B)
    ("full", 24, 1, 0, None, 3, 1),
    ("full", 24, 1, 0, [5, 11, 8], 4, 1),
    ("full", 20, 1, 0, None, 1, 2),
    ("full", 17, 1, 0, [1, 16], 2, 2),
    ("contiguous", 8, 3, 1, None, 3, 1),
    ("contiguous", 8, 3, 2, [10, 14], 3, 1),
    ("zigzag", 8, 2, 1, None, 3, 1),
    ("zigzag", 6, 3, 0, None, 2, 1),
    ("zigzag", 12, 2, 1, [8, 16], 3, 1),          # each document cut into 2cp chunks
    ("zigzag", 12, 3, 2, [6, 0, 12, 18], 2, 1),
    ("headshard", 16, 2, 0, [9, 7], 3, 1),
]


def _docs_and_cu(S, doc_lens):
    if doc_lens is None:
        return [(0, S)], None
    cu = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32)
    return [(int(cu[i]), int(cu[i + 1])) for i in range(len(doc_lens))], cu


@pytest.mark.parametrize("layout,T,cp,rank,doc_lens,nb,B", CASES)
def test_oracle_matches_sdpa_augmented_mask(layout, T, cp, rank, doc_lens, nb, B):
    rng = np.random.default_rng(1234 + T + nb)
    S = T * cp if layout in ("contiguous", "zigzag") else T
    p = rand_problem(rng, B=B, T=T, Tkv=S, nb=nb)
    docs, cu = _docs_and_cu(S, doc_lens)
    qpos = oracle.query_positions(layout, T, cp, rank, cu)
    ref = sdpa_reference(p, qpos, docs)
    out, lse = oracle.forward(p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu,
                              layout, cp, rank, rows=5)
    grads = oracle.backward(p["dout"], p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"],
                            cu, layout, cp, rank, rows=7)
    np.testing.assert_allclose(out, ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref[1], rtol=0, atol=1e-12)
    for g, r in zip(grads, ref[2:]):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------
# Finite differences of L = sum(out * dO)
# ---------------------------------------------------------------------------

def test_oracle_gradients_match_finite_differences():
    rng = np.random.default_rng(7)
    p = rand_problem(rng, B=1, T=12, H=2, D=8, nb=3)
    cu = np.array([0, 5, 12], dtype=np.int32)

    def loss(q, k0, v0, kd, vd):
        out, _ = oracle.forward(q, k0, v0, kd, vd, p["scale"], cu)
        return float(np.sum(out * p["dout"]))

    names = ["q", "k0", "v0", "kd", "vd"]
    grads = oracle.backward(p["dout"], p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu)
    h = 1e-6
    for name, g in zip(names, grads):
        x = p[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {n: p[n] for n in names}
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args[name] = xp
            lp = loss(**args)
            args[name] = xm
            lm = loss(**args)
            fd[idx] = (lp - lm) / (2 * h)
        rel = np.linalg.norm(g - fd) / np.linalg.norm(fd)
        assert rel < 1e-6, (name, rel)


# ---------------------------------------------------------------------------
# num_blocks = 1 reduces to textbook causal attention
# ---------------------------------------------------------------------------

def test_single_block_is_causal_attention_brute_force():
    rng = np.random.default_rng(3)
    T, D = 10, 4
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    scale = 0.7
    ref = np.zeros((T, D))
    ref_lse = np.zeros(T)
    for t in range(T):                      # naive loops
        w = [math.exp(scale * sum(q[t, d] * k[s, d] for d in range(D))) for s in range(t + 1)]
        z = sum(w)
        ref_lse[t] = math.log(z)
        for d in range(D):
            ref[t, d] = sum(w[s] * v[s, d] for s in range(t + 1)) / z
    out, lse = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None],
                              np.zeros((1, 0, T, 1, D)), np.zeros((1, 0, T, 1, D)), scale)
    np.testing.assert_allclose(out[0, :, 0], ref, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], ref_lse, atol=1e-13)


def test_single_block_varlen_is_per_document_causal_sdpa():
    rng = np.random.default_rng(4)
    docs = [7, 3, 9]
    cu = np.concatenate([[0], np.cumsum(docs)])
    T, H, D = int(cu[-1]), 3, 16
    p = rand_problem(rng, T=T, H=H, D=D, nb=1)
    out, lse = oracle.forward(p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu)
    for i in range(len(docs)):
        a, b = int(cu[i]), int(cu[i + 1])
        qh = torch.tensor(p["q"][0, a:b]).transpose(0, 1)
        kh = torch.tensor(p["k0"][0, a:b]).transpose(0, 1)
        vh = torch.tensor(p["v0"][0, a:b]).transpose(0, 1)
        ref = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True, scale=p["scale"])
        np.testing.assert_allclose(out[0, a:b], ref.transpose(0, 1).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# Closed form at q = 0: every score is 0
# ---------------------------------------------------------------------------

def test_closed_form_zero_query():
    rng = np.random.default_rng(5)
    docs = [6, 10]
    cu = np.concatenate([[0], np.cumsum(docs)])
    T, H, D, nb = 16, 2, 8, 4
    N = nb - 1
    p = rand_problem(rng, T=T, H=H, D=D, nb=nb)
    p["q"][:] = 0.0
    out, lse = oracle.forward(p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu)
    dq, dk0, dv0, dkd, dvd = oracle.backward(p["dout"], p["q"], p["k0"], p["v0"], p["kd"],
                                            p["vd"], p["scale"], cu)
    start = np.repeat(cu[:-1], docs)
    n = (np.arange(T) - start + 1) + N                       # keys per row
    np.testing.assert_allclose(lse[0], np.log(n)[None, :].repeat(H, 0), atol=1e-14)
    for t in range(T):
        s0 = int(start[t])
        expect = (p["v0"][0, s0:t + 1].sum(0) + p["vd"][0, :, t].sum(0)) / n[t]
        np.testing.assert_allclose(out[0, t], expect, atol=1e-14)
    np.testing.assert_allclose(dk0, 0.0, atol=0)
    np.testing.assert_allclose(dkd, 0.0, atol=0)
    for s in range(T):
        end = int(cu[np.searchsorted(cu, s, side="right")])
        expect = sum(p["dout"][0, t] / n[t] for t in range(s, end))
        np.testing.assert_allclose(dv0[0, s], expect, atol=1e-14)
    expect = np.broadcast_to(p["dout"][0][None] / n[None, :, None, None], dvd[0].shape)
    np.testing.assert_allclose(dvd[0], expect, atol=1e-14)


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def test_invariants():
    rng = np.random.default_rng(6)
    T, H, D, nb = 20, 2, 8, 3
    cu = np.array([0, 9, 20])
    p = rand_problem(rng, T=T, H=H, D=D, nb=nb)
    sc = p["scale"]
    out, lse = oracle.forward(p["q"], p["k0"], p["v0"], p["kd"], p["vd"], sc, cu)
    # probabilities sum to one: values all equal to 1 give out = 1
    ones = np.ones_like(p["v0"])
    o1, _ = oracle.forward(p["q"], p["k0"], ones, p["kd"], np.ones_like(p["vd"]), sc, cu)
    np.testing.assert_allclose(o1, 1.0, atol=1e-13)
    # max score <= lse <= max score + ln(n)
    qpos = np.arange(T)
    lo = oracle.doc_start(cu, qpos)
    for h in range(H):
        for t in range(T):
            xs = [sc * p["q"][0, t, h] @ p["k0"][0, s, h] for s in range(lo[t], t + 1)]
            ys = [sc * p["q"][0, t, h] @ p["kd"][0, i, t, h] for i in range(nb - 1)]
            mx = max(xs + ys)
            n = len(xs) + len(ys)
            assert mx - 1e-12 <= lse[0, h, t] <= mx + math.log(n) + 1e-12
    # translating every key by c leaves out unchanged and shifts lse by scale*<q,c>
    c = rng.standard_normal(D)
    out2, lse2 = oracle.forward(p["q"], p["k0"] + c, p["v0"], p["kd"] + c, p["vd"], sc, cu)
    np.testing.assert_allclose(out2, out, atol=1e-12)
    shift = sc * np.einsum("bthd,d->bht", p["q"], c)
    np.testing.assert_allclose(lse2, lse + shift, atol=1e-12)
    # translating every value by c adds c to out
    out3, _ = oracle.forward(p["q"], p["k0"], p["v0"] + c, p["kd"], p["vd"] + c, sc, cu)
    np.testing.assert_allclose(out3, out + c, atol=1e-12)
    # per (b, h): sum of all key grads is 0; sum of all value grads is sum_t dO_t
    dq, dk0, dv0, dkd, dvd = oracle.backward(p["dout"], p["q"], p["k0"], p["v0"], p["kd"],
                                            p["vd"], sc, cu)
    ksum = dk0.sum(axis=1) + dkd.sum(axis=(1, 2))
    np.testing.assert_allclose(ksum, 0.0, atol=1e-12)
    vsum = dv0.sum(axis=1) + dvd.sum(axis=(1, 2))
    np.testing.assert_allclose(vsum, p["dout"].sum(axis=1), atol=1e-12)


# ---------------------------------------------------------------------------
# Merge invariant: any split of the keys merged in any order = the unsplit softmax
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_merge_of_split_blocks_in_any_order(seed):
    rng = np.random.default_rng(100 + seed)
    T, D, N = 16, 8, 3
    cu = np.array([0, 7, 16])
    q = rng.standard_normal((T, D))
    k0 = rng.standard_normal((T, D))
    v0 = rng.standard_normal((T, D))
    kd = rng.standard_normal((N, T, D))
    vd = rng.standard_normal((N, T, D))
    sc = 0.4
    qpos = np.arange(T)
    full_out, full_lse = oracle.forward_head(q, k0, v0, kd, vd, sc, qpos, cu)
    vis = oracle.visible_mask(qpos, np.arange(T), cu)
    # random split of the block-0 keys into segments (some rows see none of a segment)
    cuts = np.sort(rng.choice(np.arange(1, T), size=4, replace=False))
    bounds = [0] + list(cuts) + [T]
    blocks = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        m = np.zeros_like(vis)
        m[:, a:b] = vis[:, a:b]
        blocks.append(oracle.block_attention(q, k0, v0, m, sc))
    for i in range(N):                       # each diagonal is a one-key block
        blocks.append((vd[i], sc * np.sum(q * kd[i], axis=1)))
    order = rng.permutation(len(blocks))
    out = np.zeros((T, D))
    lse = np.full(T, -np.inf)
    for j in order:
        out, lse, _ = oracle.lse_merge(out, lse, *blocks[j])
    np.testing.assert_allclose(out, full_out, atol=1e-12)
    np.testing.assert_allclose(lse, full_lse, atol=1e-12)


def test_merge_special_cases():
    rng = np.random.default_rng(9)
    out = rng.standard_normal((4, 3))
    lse = rng.standard_normal(4)
    bo = rng.standard_normal((4, 3))
    # empty block is a no-op
    o, l, w = oracle.lse_merge(out, lse, bo, np.full(4, -np.inf))
    np.testing.assert_array_equal(o, out)
    np.testing.assert_array_equal(l, lse)
    # merging into an empty state takes the block
    o, l, _ = oracle.lse_merge(np.zeros((4, 3)), np.full(4, -np.inf), bo, lse)
    np.testing.assert_array_equal(o, bo)
    np.testing.assert_array_equal(l, lse)
    # two equal-lse blocks average; lse grows by ln 2
    o, l, w = oracle.lse_merge(out, lse, bo, lse.copy())
    np.testing.assert_allclose(o, 0.5 * (out + bo), atol=1e-15)
    np.testing.assert_allclose(l, lse + math.log(2), atol=1e-15)
    np.testing.assert_allclose(w, 0.5)
    # far-apart lse values do not overflow
    o, l, _ = oracle.lse_merge(out, np.full(4, 800.0), bo, np.full(4, -800.0))
    np.testing.assert_allclose(o, out, atol=1e-300)
    np.testing.assert_allclose(l, 800.0)


# ---------------------------------------------------------------------------
# Layouts: shares re-assembled equal the full-sequence result
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layout,doc_lens", [("contiguous", None), ("zigzag", None),
                                             ("contiguous", [5, 20, 7]),
                                             ("zigzag", [8, 0, 16, 8])])
def test_ring_layout_shares_reassemble_to_full(layout, doc_lens):
    rng = np.random.default_rng(11)
    cp, S, H, D, nb = 4, 32, 2, 8, 3
    T = S // cp
    _, cu = _docs_and_cu(S, doc_lens)
    full = rand_problem(rng, T=S, H=H, D=D, nb=nb)
    f_out, f_lse = oracle.forward(full["q"], full["k0"], full["v0"], full["kd"], full["vd"],
                                  full["scale"], cu)
    f_grads = oracle.backward(full["dout"], full["q"], full["k0"], full["v0"], full["kd"],
                              full["vd"], full["scale"], cu)
    dk0 = np.zeros_like(f_grads[1])
    dv0 = np.zeros_like(f_grads[2])
    seen = np.zeros(S, dtype=int)
    for r in range(cp):
        pos = oracle.query_positions(layout, T, cp, r, cu)
        seen[pos] += 1
        sh = {k: full[k][:, pos] for k in ("q", "dout")}
        sh.update({k: full[k][:, :, pos] for k in ("kd", "vd")})
        out, lse = oracle.forward(sh["q"], full["k0"], full["v0"], sh["kd"], sh["vd"],
                                  full["scale"], cu, layout, cp, r)
        np.testing.assert_allclose(out, f_out[:, pos], atol=1e-12)
        np.testing.assert_allclose(lse, f_lse[:, :, pos], atol=1e-12)
        dq, a, b, dkd, dvd = oracle.backward(sh["dout"], sh["q"], full["k0"], full["v0"], sh["kd"],
                                             sh["vd"], full["scale"], cu, layout, cp, r)
        np.testing.assert_allclose(dq, f_grads[0][:, pos], atol=1e-12)
        np.testing.assert_allclose(dkd, f_grads[3][:, :, pos], atol=1e-12)
        np.testing.assert_allclose(dvd, f_grads[4][:, :, pos], atol=1e-12)
        dk0 += a
        dv0 += b
    assert np.all(seen == 1)                 # the shares partition the sequence
    np.testing.assert_allclose(dk0, f_grads[1], atol=1e-12)
    np.testing.assert_allclose(dv0, f_grads[2], atol=1e-12)


def test_headshard_equals_full_restricted_to_heads():
    rng = np.random.default_rng(12)
    uly, S, H, D, nb = 4, 24, 8, 8, 3
    cu = np.array([0, 10, 24])
    p = rand_problem(rng, T=S, H=H, D=D, nb=nb)
    f_out, f_lse = oracle.forward(p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu)
    f_g = oracle.backward(p["dout"], p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu)
    hl = H // uly
    for r in range(uly):
        hs = slice(r * hl, (r + 1) * hl)
        sh = {k: p[k][:, :, hs] if k in ("q", "k0", "v0", "dout") else p[k][:, :, :, hs]
              for k in ("q", "k0", "v0", "kd", "vd", "dout")}
        out, lse = oracle.forward(sh["q"], sh["k0"], sh["v0"], sh["kd"], sh["vd"], p["scale"], cu,
                                  "headshard", uly, r)
        np.testing.assert_allclose(out, f_out[:, :, hs], atol=1e-13)
        np.testing.assert_allclose(lse, f_lse[:, hs], atol=1e-13)
        g = oracle.backward(sh["dout"], sh["q"], sh["k0"], sh["v0"], sh["kd"], sh["vd"],
                            p["scale"], cu, "headshard", uly, r)
        for a, b, ax in zip(g, f_g, (2, 2, 2, 3, 3)):
            idx = [slice(None)] * b.ndim
            idx[ax] = hs
            np.testing.assert_allclose(a, b[tuple(idx)], atol=1e-13)


# ---------------------------------------------------------------------------
# Pair counts (the load-balance statements of the pages)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cp,c", [(2, 3), (4, 5), (8, 16)])
def test_zigzag_every_rank_does_equal_work(cp, c):
    # zigzag_ring_attention page, module text: pairing an early and a late
    # chunk gives every rank equal causal work. Count: 2cp*c^2 + c pairs.
    T = 2 * c
    counts = [oracle.pair_count("zigzag", T, cp, r) for r in range(cp)]
    assert counts == [2 * cp * c * c + c] * cp
    S = 2 * cp * c
    assert sum(counts) == S * (S + 1) // 2
    # brute force from the mask
    for r in range(cp):
        qpos = oracle.query_positions("zigzag", T, cp, r)
        assert oracle.visible_mask(qpos, np.arange(S)).sum() == counts[r]


@pytest.mark.parametrize("cp,doc_lens", [(2, [4, 12, 0, 8]), (4, [8, 24, 96]), (8, [16, 4096, 32])])
def test_zigzag_several_documents_equal_work_and_halves(cp, doc_lens):
    """Several documents (zigzag_ring_attention page, `get_half_index`: the front
    and back half of each varlen document): every rank does equal causal work in
    every document (the page's load-balance statement, per document: 2cp*c^2 + c
    pairs for chunks of c), the shares partition the sequence, and each local
    document is [front half | back half] with every front position before every
    back position; local documents follow the global order with local
    boundaries cu / cp."""
    S = sum(doc_lens)
    T = S // cp
    cu = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32)
    seen = np.zeros(S, dtype=int)
    want = sum(2 * cp * (L // (2 * cp)) ** 2 + L // (2 * cp) for L in doc_lens)
    for r in range(cp):
        qpos = oracle.query_positions("zigzag", T, cp, r, cu)
        seen[qpos] += 1
        assert oracle.pair_count("zigzag", T, cp, r, cu) == want
        vis = oracle.visible_mask(qpos, np.arange(S), cu)
        assert vis.sum() == want                                  # brute force from the mask
        for d, L in enumerate(doc_lens):
            a, b = cu[d] // cp, cu[d + 1] // cp                    # local document d
            loc = qpos[a:b]
            assert np.all((loc >= cu[d]) & (loc < cu[d + 1]))
            front, back = loc[: (b - a) // 2], loc[(b - a) // 2:]
            if len(front):
                assert front.max() < back.min()
                assert np.all(np.diff(front) == 1) and np.all(np.diff(back) == 1)
    assert np.all(seen == 1)
    assert sum(oracle.pair_count("zigzag", T, cp, r, cu) for r in range(cp)) == \
        sum(L * (L + 1) // 2 for L in doc_lens)


@pytest.mark.parametrize("cp,L", [(2, 4), (8, 16), (8, 1024)])
def test_contiguous_last_rank_does_about_twice_the_mean(cp, L):
    # ring_attention page, `_CachedZigZagRingAttention`: with contiguous shards the
    # last rank carries close to double the mean load. Rank r: r*L^2 + L(L+1)/2.
    counts = [oracle.pair_count("contiguous", L, cp, r) for r in range(cp)]
    assert counts == [r * L * L + L * (L + 1) // 2 for r in range(cp)]
    S = cp * L
    assert sum(counts) == S * (S + 1) // 2
    ratio = counts[-1] / (sum(counts) / cp)
    assert 1.0 < ratio < 2.0                      # close to double; tends to 2 - 1/cp
    assert abs(ratio - (2.0 - 1.0 / cp)) < 1.0 / L
    if L >= 1024 and cp == 8:
        assert abs(ratio - 1.875) < 2e-3


def test_ring_order_and_per_step_visibility():
    # zigzag_ring_attention page, `RingComm`: each step K/V move one rank up the
    # ring, so step j holds rank (r-j) mod cp's K/V.
    steps = oracle.ring_steps("zigzag", 8, 3)
    assert [s for s, _ in steps] == [3, 2, 1, 0, 7, 6, 5, 4]
    assert steps[4][1] == [7, 8]
    # ring_attention page, `ring_flash_attn_forward`: a causal contiguous share
    # skips the K/V of higher ranks.
    assert [s for s, _ in oracle.ring_steps("contiguous", 4, 2)] == [2, 1, 0]
    # per-step visibility of the zig-zag share (early half = rows [0,c), late = [c,2c))
    cp, r, c = 4, 1, 4
    T = 2 * c
    qpos = oracle.query_positions("zigzag", T, cp, r)
    for src, chunks in oracle.ring_steps("zigzag", cp, r):
        keys = np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in chunks])
        vis = oracle.visible_mask(qpos, keys)
        early, late = vis[:c], vis[c:]
        front, back = vis[:, :c], vis[:, c:]
        if src == r:     # own block: causal over the local [early | late]
            assert early[:, :c].sum() == c * (c + 1) // 2 and not early[:, c:].any()
            assert late[:, :c].all() and late[:, c:].sum() == c * (c + 1) // 2
        elif src < r:    # all local rows see the front (early) chunk only
            assert front.all() and not back.any()
        else:            # only the late rows see the block, all of it
            assert not early.any() and late.all()
    # the same rule inside every document of a packed sequence (the early and late
    # halves of each document, addressed with cu_seqlens divided by two:
    # zigzag_ring_attention page, `_block_forward`)
    doc_lens = [16, 32, 8]
    cu = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32)
    S = int(cu[-1])
    qpos = oracle.query_positions("zigzag", S // cp, cp, r, cu)
    for d, L in enumerate(doc_lens):
        c = L // (2 * cp)
        rows = qpos[cu[d] // cp: cu[d + 1] // cp]
        for src, chunks in oracle.ring_steps("zigzag", cp, r):
            keys = np.concatenate([cu[d] + np.arange(ch * c, (ch + 1) * c) for ch in chunks])
            vis = oracle.visible_mask(rows, keys, cu)
            early, late = vis[:c], vis[c:]
            if src == r:
                assert early[:, :c].sum() == c * (c + 1) // 2 and not early[:, c:].any()
                assert late[:, :c].all() and late[:, c:].sum() == c * (c + 1) // 2
            elif src < r:
                assert vis[:, :c].all() and not vis[:, c:].any()
            else:
                assert not early.any() and late.all()
            # keys of other documents are never visible to these rows
            other = np.setdiff1d(np.arange(S), np.arange(cu[d], cu[d + 1]))
            assert not oracle.visible_mask(rows, other, cu).any()


# ---------------------------------------------------------------------------
# Negative test: the backward needs the MERGED lse
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nb", [1, 3])
def test_backward_with_block0_only_lse_is_wrong_when_diagonals_exist(nb):
    rng = np.random.default_rng(21)
    T, D = 12, 8
    q, k0, v0, dout = (rng.standard_normal((T, D)) for _ in range(4))
    kd, vd = (rng.standard_normal((nb - 1, T, D)) for _ in range(2))
    sc = 0.35
    qpos = np.arange(T)
    out, lse = oracle.forward_head(q, k0, v0, kd, vd, sc, qpos)
    _, lse0 = oracle.block_attention(q, k0, v0, oracle.visible_mask(qpos, qpos), sc)
    good = oracle.backward_head(dout, q, k0, v0, kd, vd, sc, qpos, out=out, lse=lse)
    bad = oracle.backward_head(dout, q, k0, v0, kd, vd, sc, qpos, out=out, lse=lse0)
    diff = max(np.abs(a - b).max() for a, b in zip(good[:3], bad[:3]))
    if nb == 1:
        assert diff < 1e-13
    else:
        assert diff > 1e-3


# ---------------------------------------------------------------------------
# Planted mistakes: a broken copy of the oracle must fail the pins above
# ---------------------------------------------------------------------------

MUTATIONS = [
    ("y = scale * np.einsum(\"rd,nrd->rn\", Q, kd[:, a:b])      # diagonal scores",
     "y = np.einsum(\"rd,nrd->rn\", Q, kd[:, a:b])"),                      # dropped diag scale
    ("(ks[None, :] <= qp[:, None])\n        Q = q[a:b]\n        x = scale",
     "(ks[None, :] < qp[:, None])\n        Q = q[a:b]\n        x = scale"),  # causal not inclusive
    ("dS = p * ((dO @ V.T) - dl[:, None])", "dS = p * ((dO @ V.T) + dl[:, None])"),   # sign
    ("dvd[:, a:b] = pi.T[:, :, None] * dO[None]", "dvd[:, a:b] = pi.T[:, :, None] * Q[None]"),
    ("dk0[kmin:kmax] += scale * (dS.T @ Q)", "dk0[kmin:kmax] += scale * (dS.T @ dO)"),
    ("out[a:b] = p @ v0[kmin:kmax] + np.einsum(\"rn,nrd->rd\", pi, vd[:, a:b])",
     "out[a:b] = p @ v0[kmin:kmax]"),                                         # dropped term
]


def _mutant(src_from, src_to):
    import importlib.util
    import types
    spec = importlib.util.find_spec("oracle.eagle3_oracle")
    text = open(spec.origin).read()
    assert src_from in text, src_from
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(src_from, src_to, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("i", range(len(MUTATIONS)))
def test_planted_mistake_is_caught_by_sdpa_pin(i):
    mod = _mutant(*MUTATIONS[i])
    rng = np.random.default_rng(77)
    T, nb = 12, 3
    p = rand_problem(rng, T=T, nb=nb)
    cu = np.array([0, 5, 12])
    docs = [(0, 5), (5, 12)]
    ref = sdpa_reference(p, np.arange(T), docs)
    out, lse = mod.forward(p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu)
    grads = mod.backward(p["dout"], p["q"], p["k0"], p["v0"], p["kd"], p["vd"], p["scale"], cu)
    errs = [np.abs(out - ref[0]).max(), np.abs(lse - ref[1]).max()]
    errs += [np.abs(g - r).max() for g, r in zip(grads, ref[2:])]
    assert max(errs) > 1e-6
