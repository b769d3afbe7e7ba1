"""CPU oracle for EAGLE-3 mixed attention (forward and backward).

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously correct
definition the HIP kernels are checked against. Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it. The product path never
calls it, and it shares no code with the HIP path (it imports nothing from the
product package).

What it computes (pages: nemo_automodel ... speculative.eagle.ring_attention,
class `_CachedRingAttention`; ...eagle.ulysses_attention, class
`_CachedUlyssesAttention`; ...eagle.zigzag_ring_attention, module text):

  For every query row t (global position g_t) the row holds one joint softmax
  over
    * block 0: the step-0 sequence keys k0_s that lie in the same document as
      g_t with position s <= g_t (causal, inclusive of self), score
      x_{t,s} = scale * <q_t, k0_s>, value v0_s;
    * blocks i = 1..N (TTT steps): one key per row, at the same position,
      score y_{t,i} = scale * <q_t, kd_{i,t}>, value vd_{i,t}.
  lse_t = log( sum_s exp(x_{t,s}) + sum_i exp(y_{t,i}) ), natural log;
  out_t = sum_s p_{t,s} v0_s + sum_i pi_{t,i} vd_{i,t},
  with p = exp(x - lse), pi = exp(y - lse).

  The backward is the gradient of that joint softmax: with delta_t = <dO_t, out_t>
    dS_{t,s} = p_{t,s} (<dO_t, v0_s> - delta_t),  ds_{t,i} = pi_{t,i} (<dO_t, vd_{i,t}> - delta_t)
    dq_t  = scale (sum_s dS_{t,s} k0_s + sum_i ds_{t,i} kd_{i,t})
    dk0_s = scale sum_t dS_{t,s} q_t,   dv0_s = sum_t p_{t,s} dO_t
    dkd_{i,t} = scale ds_{t,i} q_t,     dvd_{i,t} = pi_{t,i} dO_t
  (ring_attention page, `_CachedRingAttention`: block 0's gradient is taken with
  the out/lse of all blocks together, and the diagonal terms have a closed form;
  zigzag_ring_attention page, `zigzag_ring_flash_attn_varlen_backward`: every
  block's backward is given that final out/lse.)

Everything is float64. The score rows are materialised explicitly, a block of
rows at a time (rows are independent, so the grouping is only for memory); the
keys offered to a row block are limited to the window that can be visible to
any row of it, which drops only keys whose scores are -inf.

Shapes (FlashAttention layout, as on the pages):
  q, dout, out, dq          [B, T, H, D]
  k0, v0, dk0, dv0          [B, T_kv, H, D]   block 0, full sequence, global order
  kd, vd, dkd, dvd          [B, N, T, H, D]   blocks 1..N, the local rows
  lse                       [B, H, T]
"""
from __future__ import annotations

import numpy as np

LAYOUTS = ("full", "contiguous", "zigzag", "headshard")


# ---------------------------------------------------------------------------
# Layout: global positions of the local query rows, document starts, masks
# ---------------------------------------------------------------------------

def query_positions(layout: str, T: int, cp: int = 1, rank: int = 0, cu_seqlens=None) -> np.ndarray:
    """Global sequence position of each local query row.

    full / headshard: the whole sequence is local (ulysses_attention page,
      module text: once the all-to-all has run, every rank has all positions,
      for H/uly of the heads).
    contiguous: rank r holds positions [r*T, (r+1)*T) (ring_attention page,
      module text: the r-th run of S/cp consecutive positions).
    zigzag: every document is cut into 2*cp chunks; rank r holds chunk r
      (early) then chunk 2*cp-1-r (late) of each document, documents one after
      the other (zigzag_ring_attention page, module text: the 2*cp chunks and
      their ownership; `get_half_index`: the front and back half of EACH varlen
      document; ring_attention page, `_CachedZigZagRingAttention`). With one
      document (cu_seqlens None) the chunks are c = T/2 rows of the sequence
      S = cp*T. Every document length must divide by 2*cp.
    """
    if layout in ("full", "headshard"):
        return np.arange(T, dtype=np.int64)
    if layout == "contiguous":
        return rank * T + np.arange(T, dtype=np.int64)
    if layout == "zigzag":
        assert T % 2 == 0
        S = cp * T
        if cu_seqlens is None:
            bounds = [(0, S)]
        else:
            cu = [int(x) for x in cu_seqlens]
            assert cu[0] == 0 and cu[-1] == S
            bounds = list(zip(cu[:-1], cu[1:]))
        parts = []
        for lo, hi in bounds:
            assert (hi - lo) % (2 * cp) == 0, "document length must divide by 2*cp"
            c = (hi - lo) // (2 * cp)
            parts.append(lo + rank * c + np.arange(c, dtype=np.int64))
            parts.append(lo + (2 * cp - 1 - rank) * c + np.arange(c, dtype=np.int64))
        return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    raise ValueError(layout)


def doc_start(cu_seqlens, pos: np.ndarray) -> np.ndarray:
    """First position of the document that holds each position. `cu_seqlens`
    holds global document boundaries [0, ..., S] (ulysses_attention page,
    `cached_ulysses_attention`: GLOBAL packed-document boundaries); None means a
    single document."""
    pos = np.asarray(pos, dtype=np.int64)
    if cu_seqlens is None:
        return np.zeros_like(pos)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    idx = np.searchsorted(cu, pos, side="right") - 1
    return cu[idx]


def visible_mask(qpos: np.ndarray, kpos: np.ndarray, cu_seqlens=None) -> np.ndarray:
    """bool [len(qpos), len(kpos)]: key s is visible to query t iff both are in
    the same document and s <= t (block-0 causal attention within documents)."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    lo = doc_start(cu_seqlens, qpos)
    return (kpos[None, :] >= lo[:, None]) & (kpos[None, :] <= qpos[:, None])


def pair_count(layout: str, T: int, cp: int = 1, rank: int = 0, cu_seqlens=None) -> int:
    """Number of attended block-0 (query, key) pairs of one share, counted
    row by row from the visibility rule."""
    qpos = query_positions(layout, T, cp, rank, cu_seqlens)
    lo = doc_start(cu_seqlens, qpos)
    return int(np.sum(qpos - lo + 1))


def ring_steps(layout: str, cp: int, rank: int) -> list:
    """Ring order of the block-0 K/V segments a rank attends.

    At ring step j a rank holds the K/V of rank (rank - j) mod cp (the ring
    sends to rank+1 and receives from rank-1: zigzag_ring_attention page,
    `RingComm`). Returns [(src, [chunk ids])] with chunk ids in units of the
    layout's chunk: contiguous -> [src]; zigzag -> [src, 2cp-1-src].
    For contiguous causal attention only steps with src <= rank contribute
    (ring_attention page, `ring_flash_attn_forward`); the zig-zag steps all
    contribute to some rows.
    """
    steps = []
    for j in range(cp):
        src = (rank - j) % cp
        if layout == "contiguous":
            if src <= rank:
                steps.append((src, [src]))
        elif layout == "zigzag":
            steps.append((src, [src, 2 * cp - 1 - src]))
        else:
            raise ValueError(layout)
    return steps


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------

def _row_blocks(T: int, rows: int):
    for a in range(0, T, rows):
        yield a, min(T, a + rows)


def _window(qpos, lo):
    """Key window [kmin, kmax) that can hold a visible key for these rows."""
    return int(lo.min()), int(qpos.max()) + 1


def forward_head(q, k0, v0, kd, vd, scale, qpos, cu_seqlens=None, rows=256):
    """One (batch row, head): q [T,D], k0/v0 [T_kv,D], kd/vd [N,T,D].
    Returns out [T,D], lse [T] (float64)."""
    q = np.asarray(q, np.float64)
    k0 = np.asarray(k0, np.float64)
    v0 = np.asarray(v0, np.float64)
    kd = np.asarray(kd, np.float64)
    vd = np.asarray(vd, np.float64)
    T, D = q.shape
    out = np.zeros((T, D))
    lse = np.zeros(T)
    lo_all = doc_start(cu_seqlens, qpos)
    for a, b in _row_blocks(T, rows):
        qp, lo = qpos[a:b], lo_all[a:b]
        kmin, kmax = _window(qp, lo)
        ks = np.arange(kmin, kmax)
        vis = (ks[None, :] >= lo[:, None]) & (ks[None, :] <= qp[:, None])
        Q = q[a:b]
        x = scale * (Q @ k0[kmin:kmax].T)                       # block-0 scores
        x = np.where(vis, x, -np.inf)
        y = scale * np.einsum("rd,nrd->rn", Q, kd[:, a:b])      # diagonal scores
        m = np.maximum(x.max(axis=1), y.max(axis=1) if y.size else -np.inf)
        z = np.exp(x - m[:, None]).sum(axis=1) + np.exp(y - m[:, None]).sum(axis=1)
        L = m + np.log(z)
        p = np.exp(x - L[:, None])
        pi = np.exp(y - L[:, None])
        out[a:b] = p @ v0[kmin:kmax] + np.einsum("rn,nrd->rd", pi, vd[:, a:b])
        lse[a:b] = L
    return out, lse


def _heads(H, heads):
    return list(range(H)) if heads is None else list(heads)


def forward(q, k0, v0, kd, vd, scale, cu_seqlens=None, layout="full", cp=1, rank=0,
            heads=None, rows=256):
    """Full forward over [B, T, H, D] tensors (any array-likes; bf16 torch
    tensors should be upcast by the caller). Returns out [B,T,h,D] and
    lse [B,h,T] for the requested heads (all by default)."""
    q = np.asarray(q, np.float64)
    B, T, H, D = q.shape
    hs = _heads(H, heads)
    qpos = query_positions(layout, T, cp, rank, cu_seqlens)
    out = np.zeros((B, T, len(hs), D))
    lse = np.zeros((B, len(hs), T))
    for b in range(B):
        for j, h in enumerate(hs):
            o, l = forward_head(q[b, :, h], np.asarray(k0)[b, :, h], np.asarray(v0)[b, :, h],
                                np.asarray(kd)[b, :, :, h], np.asarray(vd)[b, :, :, h],
                                scale, qpos, cu_seqlens, rows)
            out[b, :, j] = o
            lse[b, j] = l
    return out, lse


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def backward_head(dout, q, k0, v0, kd, vd, scale, qpos, cu_seqlens=None, out=None,
                  lse=None, rows=256):
    """Gradient of sum(out * dout) for one (batch row, head).

    `out`/`lse` default to this oracle's own forward (out and lse of the joint
    softmax over all blocks). Passing another lse (e.g. the block-0-only lse) reproduces the
    backward that the zigzag_ring_attention page warns against.
    Returns dq [T,D], dk0 [T_kv,D], dv0 [T_kv,D], dkd [N,T,D], dvd [N,T,D].
    """
    q = np.asarray(q, np.float64)
    k0 = np.asarray(k0, np.float64)
    v0 = np.asarray(v0, np.float64)
    kd = np.asarray(kd, np.float64)
    vd = np.asarray(vd, np.float64)
    dout = np.asarray(dout, np.float64)
    if out is None or lse is None:
        o2, l2 = forward_head(q, k0, v0, kd, vd, scale, qpos, cu_seqlens, rows)
        out = o2 if out is None else out
        lse = l2 if lse is None else lse
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    T, D = q.shape
    dq = np.zeros_like(q)
    dk0 = np.zeros_like(k0)
    dv0 = np.zeros_like(v0)
    dkd = np.zeros_like(kd)
    dvd = np.zeros_like(vd)
    lo_all = doc_start(cu_seqlens, qpos)
    delta = np.sum(dout * out, axis=1)                         # <dO_t, out_t>
    for a, b in _row_blocks(T, rows):
        qp, lo = qpos[a:b], lo_all[a:b]
        kmin, kmax = _window(qp, lo)
        ks = np.arange(kmin, kmax)
        vis = (ks[None, :] >= lo[:, None]) & (ks[None, :] <= qp[:, None])
        Q, dO, L, dl = q[a:b], dout[a:b], lse[a:b], delta[a:b]
        K, V = k0[kmin:kmax], v0[kmin:kmax]
        x = np.where(vis, scale * (Q @ K.T), -np.inf)
        p = np.exp(x - L[:, None])                              # joint-softmax probs
        y = scale * np.einsum("rd,nrd->rn", Q, kd[:, a:b])
        pi = np.exp(y - L[:, None])
        dS = p * ((dO @ V.T) - dl[:, None])
        ds = pi * (np.einsum("rd,nrd->rn", dO, vd[:, a:b]) - dl[:, None])
        dq[a:b] = scale * (dS @ K + np.einsum("rn,nrd->rd", ds, kd[:, a:b]))
        dk0[kmin:kmax] += scale * (dS.T @ Q)
        dv0[kmin:kmax] += p.T @ dO
        dkd[:, a:b] = scale * ds.T[:, :, None] * Q[None]
        dvd[:, a:b] = pi.T[:, :, None] * dO[None]
    return dq, dk0, dv0, dkd, dvd


def backward(dout, q, k0, v0, kd, vd, scale, cu_seqlens=None, layout="full", cp=1,
             rank=0, out=None, lse=None, heads=None, rows=256):
    """Backward over [B, T, H, D] tensors for the requested heads. `out` and
    `lse` (if given) are indexed like the returned forward, i.e. [B,T,h,D] and
    [B,h,T] over the requested heads. Returns dq, dk0, dv0, dkd, dvd with the
    head axis restricted to those heads."""
    q = np.asarray(q, np.float64)
    B, T, H, D = q.shape
    k0 = np.asarray(k0)
    v0 = np.asarray(v0)
    kd = np.asarray(kd)
    vd = np.asarray(vd)
    dout = np.asarray(dout)
    hs = _heads(H, heads)
    qpos = query_positions(layout, T, cp, rank, cu_seqlens)
    Tkv = k0.shape[1]
    N = kd.shape[1]
    dq = np.zeros((B, T, len(hs), D))
    dk0 = np.zeros((B, Tkv, len(hs), D))
    dv0 = np.zeros((B, Tkv, len(hs), D))
    dkd = np.zeros((B, N, T, len(hs), D))
    dvd = np.zeros((B, N, T, len(hs), D))
    for b in range(B):
        for j, h in enumerate(hs):
            o = None if out is None else np.asarray(out)[b, :, j]
            l = None if lse is None else np.asarray(lse)[b, j]
            r = backward_head(dout[b, :, h], q[b, :, h], k0[b, :, h], v0[b, :, h],
                              kd[b, :, :, h], vd[b, :, :, h], scale, qpos, cu_seqlens,
                              o, l, rows)
            dq[b, :, j], dk0[b, :, j], dv0[b, :, j], dkd[b, :, :, j], dvd[b, :, :, j] = r
    return dq, dk0, dv0, dkd, dvd


# ---------------------------------------------------------------------------
# Partial blocks and the log-sum-exp merge
# ---------------------------------------------------------------------------

def block_attention(q, k, v, mask, scale):
    """Attention of rows q [T,D] over keys k/v [S,D] restricted by mask [T,S].
    Returns (out [T,D], lse [T]); a row with no visible key gets out = 0 and
    lse = -inf (an empty block)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    x = np.where(mask, scale * (q @ k.T), -np.inf)
    m = x.max(axis=1) if x.shape[1] else np.full(q.shape[0], -np.inf)
    empty = ~np.isfinite(m)
    msafe = np.where(empty, 0.0, m)
    z = np.exp(x - msafe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, msafe + np.log(np.where(empty, 1.0, z)))
    p = np.exp(x - np.where(empty, 0.0, lse)[:, None])
    out = np.where(empty[:, None], 0.0, p @ v)
    return out, lse


def _log_sigmoid(x):
    """log(1 / (1 + exp(-x))), evaluated without overflow."""
    x = np.asarray(x, np.float64)
    return np.where(x >= 0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))


def _sigmoid(x):
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def lse_merge(out, lse, block_out, block_lse):
    """Folds one block's (block_out, block_lse) into the running (out, lse),
    in the sigmoid form of the ring_attention page (`_update_out_and_lse`,
    `_merge_diag`) and the zigzag_ring_attention page (`update_out_and_lse`):
        out' = out - sigmoid(block_lse - lse) * (out - block_out)
        lse' = lse - logsigmoid(lse - block_lse)
    out [..., D] and lse [...] share leading axes. An empty block
    (block_lse = -inf) leaves the state unchanged; an empty state
    (lse = -inf) takes the block.
    Returns new arrays (also the sigmoid weight, as the zig-zag page does)."""
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    bo = np.asarray(block_out, np.float64)
    bl = np.asarray(block_lse, np.float64)
    b_empty = ~np.isfinite(bl)
    s_empty = ~np.isfinite(lse) & ~b_empty
    with np.errstate(invalid="ignore"):
        w = _sigmoid(bl - lse)
        new_out = out - w[..., None] * (out - bo)
        new_lse = lse - _log_sigmoid(lse - bl)
    new_out = np.where(b_empty[..., None], out, np.where(s_empty[..., None], bo, new_out))
    new_lse = np.where(b_empty, lse, np.where(s_empty, bl, new_lse))
    w = np.where(b_empty, 0.0, np.where(s_empty, 1.0, w))
    return new_out, new_lse, w
