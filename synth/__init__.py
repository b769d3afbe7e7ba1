"""Seeded synthetic inputs for EAGLE-3 mixed attention.

This module is shared by the tests, the benchmark and the smoke check. It holds
no attention arithmetic: it only names the workloads, draws document lengths and
draws normal random tensors. Both the CPU oracle and the HIP path consume the
exact bits produced here (bf16 values are upcast for the oracle).

Workloads (all synthetic; the pages name no dataset or benchmark suite, so these
stand in for packed EAGLE-3 training batches):

  tiny     fp32, B=1, T=256,  H=4,  D=64,  num_blocks=3, one document
  dense    bf16, B=1, T=4096, H=32, D=128, num_blocks=8, one document, x0.5
  packed   bf16, B=1, T=16384, H=32, D=128, num_blocks=8, documents with
           lengths uniform on [256, 4096] (last one truncated)
  ulysses  bf16, head shard of a Ulysses degree-8 run: S=32768, H=4, D=128,
           num_blocks=8, four 8192-token documents
  zigzag   bf16, zig-zag ring rank 3 of cp=8: S=131072 in 16 chunks of 8192,
           local Q = chunks 3 and 12, K0/V0 = the whole sequence, H=32, D=128,
           num_blocks=8, one document

Every tensor is generated per (tensor, block, batch row, chunk) from its own
derived seed, so a rank's share is a slice of one consistent full-sequence
("virtual global") tensor and the full sequence or any other rank can be
regenerated bit-identically.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

LAYOUT_FULL = 0
LAYOUT_CONTIGUOUS = 1
LAYOUT_ZIGZAG = 2
LAYOUT_HEADSHARD = 3
LAYOUT_NAMES = {"full": LAYOUT_FULL, "contiguous": LAYOUT_CONTIGUOUS,
                "zigzag": LAYOUT_ZIGZAG, "headshard": LAYOUT_HEADSHARD}


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str            # "bf16" or "f32"
    B: int
    S: int                # full (global) sequence length
    H: int                # heads held by this share
    D: int
    num_blocks: int
    layout: str = "full"  # full | contiguous | zigzag | headshard
    cp: int = 1
    rank: int = 0
    gen_scale: float = 1.0
    doc_lens: Optional[list] = None   # None = one document spanning S
    seed: int = 0
    chunk: Optional[int] = None       # rows per generator chunk (default below)

    @property
    def T(self) -> int:
        """Local query rows."""
        if self.layout in ("contiguous", "zigzag"):
            return self.S // self.cp
        return self.S

    @property
    def T_kv(self) -> int:
        return self.S

    @property
    def N(self) -> int:
        return self.num_blocks - 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def cu_seqlens(self) -> Optional[np.ndarray]:
        if self.doc_lens is None:
            return None
        return np.concatenate([[0], np.cumsum(self.doc_lens)]).astype(np.int32)

    def gen_chunk(self) -> int:
        """Rows per generator chunk: explicit, else the zig-zag chunk S/(2cp),
        else the contiguous shard S/cp, else S. It depends on the workload only,
        never on the layout a share is cut with, so every layout of one workload
        sees the same virtual global tensors."""
        if self.chunk is not None:
            return self.chunk
        if self.layout == "zigzag":
            return self.S // (2 * self.cp)
        if self.layout == "contiguous":
            return self.S // self.cp
        return self.S


def draw_doc_lens(total: int, lo: int, hi: int, seed: int) -> list:
    """Document lengths uniform on [lo, hi] (inclusive) drawn until they cover
    `total`; the last one is truncated so the lengths sum to exactly `total`."""
    rng = np.random.default_rng(seed)
    lens = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def workload(name: str, seed: int = 0) -> Workload:
    if name == "tiny":
        return Workload("tiny", "f32", 1, 256, 4, 64, 3, seed=seed)
    if name == "dense":
        return Workload("dense", "bf16", 1, 4096, 32, 128, 8, gen_scale=0.5, seed=seed)
    if name == "packed":
        return Workload("packed", "bf16", 1, 16384, 32, 128, 8,
                        doc_lens=draw_doc_lens(16384, 256, 4096, seed), seed=seed)
    if name == "ulysses":
        return Workload("ulysses", "bf16", 1, 32768, 4, 128, 8, layout="headshard",
                        cp=8, doc_lens=[8192] * 4, seed=seed)
    if name == "zigzag":
        return Workload("zigzag", "bf16", 1, 131072, 32, 128, 8, layout="zigzag",
                        cp=8, rank=3, seed=seed)
    if name == "zigzag_docs":
        # the zig-zag share of a packed batch: eight 16384-token documents, each cut
        # into 2cp chunks (measurement only; not one of the parity workloads)
        return Workload("zigzag_docs", "bf16", 1, 131072, 32, 128, 8, layout="zigzag",
                        cp=8, rank=3, doc_lens=[16384] * 8, seed=seed, chunk=1024)
    raise KeyError(name)


WORKLOADS = ("tiny", "dense", "packed", "ulysses", "zigzag")

_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "dout": 4}


def _seed_for(base: int, tensor: str, block: int, batch: int, chunk: int, head0: int) -> int:
    x = (base * 1_000_003 + _TENSOR_IDS[tensor]) * 1_000_033 + block
    x = (x * 1_000_037 + batch) * 1_000_039 + chunk
    x = x * 1_000_081 + head0
    return x % (2 ** 62)


def _chunk_randn(seed: int, rows: int, H: int, D: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(rows, H, D, generator=g, dtype=torch.float32)


def global_rows(w: Workload, tensor: str, block: int, b: int, chunk_ids, head0: int = 0,
                dtype=None) -> torch.Tensor:
    """Rows of the virtual global tensor `tensor`[block] for batch row b,
    concatenated over the given generator chunks, shape [len*chunk, H, D]."""
    c = w.gen_chunk()
    dtype = dtype or w.torch_dtype
    parts = []
    for ci in chunk_ids:
        x = _chunk_randn(_seed_for(w.seed, tensor, block, b, ci, head0), c, w.H, w.D)
        if w.gen_scale != 1.0:
            x.mul_(w.gen_scale)
        parts.append(x.to(dtype))
    return torch.cat(parts, 0)


def local_chunks(w: Workload, cp: Optional[int] = None, rank: Optional[int] = None,
                 layout: Optional[str] = None) -> list:
    """Generator chunk ids that make up a share's local rows, in local order."""
    layout = layout or w.layout
    cp = w.cp if cp is None else cp
    rank = w.rank if rank is None else rank
    c = w.gen_chunk()
    nchunks = w.S // c
    if layout in ("full", "headshard"):
        return list(range(nchunks))
    if layout == "contiguous":
        L = w.S // cp
        assert L % c == 0, "contiguous shard must be a whole number of generator chunks"
        per = L // c
        return list(range(rank * per, (rank + 1) * per))
    if layout == "zigzag":
        zc = w.S // (2 * cp)
        assert zc % c == 0, "zig-zag chunk must be a whole number of generator chunks"
        per = zc // c
        early = [rank * per + i for i in range(per)]
        late = [(2 * cp - 1 - rank) * per + i for i in range(per)]
        return early + late
    raise KeyError(layout)


def make_inputs(w: Workload, device="cpu", with_dout: bool = True,
                cp: Optional[int] = None, rank: Optional[int] = None,
                layout: Optional[str] = None, positions=None) -> dict:
    """All inputs of one share:
         q    [B, T, H, D]
         k0,v0 [B, S, H, D]         (block 0, full sequence in global order)
         kd,vd [B, N, T, H, D]      (blocks 1..N, local rows)
         dout [B, T, H, D]
    The local rows are the share's generator chunks, or, when `positions` (the
    global position of every local row, in local order) is given, those rows of
    the virtual global tensors; a zig-zag share of several documents needs them."""
    layout = layout or w.layout
    allc = list(range(w.S // w.gen_chunk()))
    if positions is None:
        if layout == "zigzag" and w.doc_lens is not None and len(w.doc_lens) > 1:
            raise ValueError("a zig-zag share of several documents needs the positions of its rows")
        loc = local_chunks(w, cp, rank, layout)
        pick = lambda t: t
    else:
        # only the generator chunks that hold the requested rows
        ch = w.gen_chunk()
        pos = np.asarray(positions, dtype=np.int64)
        loc = sorted(set((pos // ch).tolist()))
        slot = {c: i for i, c in enumerate(loc)}
        idx = torch.as_tensor(np.array([slot[int(p) // ch] * ch + int(p) % ch for p in pos], dtype=np.int64))
        pick = lambda t: t.index_select(0, idx)
    out = {}

    def stack_b(fn):
        return torch.stack([fn(b) for b in range(w.B)], 0)

    out["q"] = stack_b(lambda b: pick(global_rows(w, "q", 0, b, loc)))
    out["k0"] = stack_b(lambda b: global_rows(w, "k", 0, b, allc))
    out["v0"] = stack_b(lambda b: global_rows(w, "v", 0, b, allc))
    if w.N > 0:
        out["kd"] = stack_b(lambda b: torch.stack(
            [pick(global_rows(w, "k", i, b, loc)) for i in range(1, w.num_blocks)], 0))
        out["vd"] = stack_b(lambda b: torch.stack(
            [pick(global_rows(w, "v", i, b, loc)) for i in range(1, w.num_blocks)], 0))
    else:
        T = out["q"].shape[1]
        out["kd"] = torch.zeros(w.B, 0, T, w.H, w.D, dtype=w.torch_dtype)
        out["vd"] = torch.zeros(w.B, 0, T, w.H, w.D, dtype=w.torch_dtype)
    if with_dout:
        out["dout"] = stack_b(lambda b: pick(global_rows(w, "dout", 0, b, loc)))
    if device != "cpu":
        out = {k: v.to(device) for k, v in out.items()}
    return out


def small_workload(name: str = "small", *, dtype="bf16", B=1, S=384, H=2, D=128,
                   num_blocks=3, layout="full", cp=1, rank=0, doc_lens=None,
                   gen_scale=1.0, seed=0, chunk=None) -> Workload:
    """A reduced-size workload for parity cases the oracle finishes quickly."""
    return Workload(name, dtype, B, S, H, D, num_blocks, layout=layout, cp=cp,
                    rank=rank, gen_scale=gen_scale, doc_lens=doc_lens, seed=seed,
                    chunk=chunk)
