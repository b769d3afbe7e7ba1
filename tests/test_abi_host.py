"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
rejects bad arguments before launching anything, and its shard driver (query
positions, pair counts, ring-ordered key tiles) agrees with the oracle. No GPU
is touched: only host-side entry points and validation failures are called."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import eagle_draft_amd as e3
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "eagle3_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = e3.lib()
    names = declared_functions()
    assert "eagle3_attn_fwd" in names and "lse_merge" in names and "eagle3_shard_bwd" in names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.eagle3_abi_version() == e3.ABI_VERSION


def prob(**kw):
    d = dict(B=1, T=256, T_kv=256, H=2, D=128, num_blocks=3, scale=0.088, dtype=torch.bfloat16)
    d.update(kw)
    return e3.Problem(**d)


BAD = [
    (dict(D=96), e3.E3_EUNSUPPORTED, "head dim"),
    (dict(num_blocks=0), e3.E3_EINVAL, "num_blocks"),
    (dict(num_blocks=17), e3.E3_EINVAL, "num_blocks"),
    (dict(scale=float("nan")), e3.E3_EINVAL, "scale"),
    (dict(scale=-1.0), e3.E3_EINVAL, "scale"),
    (dict(T_kv=128), e3.E3_EINVAL, "T_kv"),
    (dict(layout="headshard", cp=3, T=256, T_kv=256), e3.E3_EINVAL, "Ulysses"),
    (dict(layout="zigzag", cp=2, T=255, T_kv=510), e3.E3_EINVAL, "even"),
    (dict(layout="zigzag", cp=2, B=2, T=256, T_kv=512), e3.E3_EINVAL, "B must be 1"),
    (dict(layout="contiguous", cp=2, rank=2, T=256, T_kv=512), e3.E3_EINVAL, "rank"),
    (dict(layout="contiguous", cp=2, rank=0, T=256, T_kv=256), e3.E3_EINVAL, "cp*T"),
    (dict(cu_seqlens=[0, 100, 200]), e3.E3_EINVAL, "ends at"),
    (dict(cu_seqlens=[1, 100, 256]), e3.E3_EINVAL, "must be 0"),
    (dict(cu_seqlens=[0, 200, 100, 256]), e3.E3_EINVAL, "non-decreasing"),
    (dict(cu_seqlens=[0, 100, 256], B=2), e3.E3_EINVAL, "B == 1"),
    # zig-zag documents are each cut into 2cp chunks: lengths must divide by 2cp
    (dict(layout="zigzag", cp=2, T=256, T_kv=512, cu_seqlens=[0, 102, 512]), e3.E3_EINVAL, "multiple of 2*cp"),
    # strides under which batch rows or blocks would overlap (gradients are written through them)
    (dict(B=2, k0_batch_stride=256 * 2 * 128 - 8), e3.E3_EINVAL, "k0_batch_stride"),
    (dict(kd_block_stride=256 * 2 * 128 - 8), e3.E3_EINVAL, "kd_block_stride"),
    (dict(B=2, kd_batch_stride=2 * 256 * 2 * 128 - 8), e3.E3_EINVAL, "kd_batch_stride"),
    (dict(k0_batch_stride=12), e3.E3_EINVAL, "multiples of 8"),
]


@pytest.mark.parametrize("kw,code,msg", BAD)
def test_invalid_problems_are_rejected_before_launch(kw, code, msg):
    p = prob(**kw)
    lib = e3.lib()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    rc = lib.eagle3_shard_fwd(p.ref(), fake, fake, fake, fake, fake, fake, fake, None)
    assert rc == code
    assert msg in lib.eagle3_last_error().decode()
    rc = lib.eagle3_shard_bwd(p.ref(), *([fake] * 14), None)
    assert rc == code
    assert lib.eagle3_bwd_workspace_bytes(p.ref()) == 0


def test_null_and_misaligned_pointers_are_rejected():
    lib = e3.lib()
    p = prob()
    a = ctypes.c_void_p(0x1000)
    rc = lib.eagle3_attn_fwd(p.ref(), None, a, a, a, a, a, a, None)
    assert rc == e3.E3_EINVAL and "q is NULL" in lib.eagle3_last_error().decode()
    rc = lib.eagle3_attn_fwd(p.ref(), a, a, a, a, a, a, None, None)
    assert rc == e3.E3_EINVAL and "lse is NULL" in lib.eagle3_last_error().decode()
    rc = lib.eagle3_attn_fwd(p.ref(), a, a, a, ctypes.c_void_p(0x1008), a, a, a, None)
    assert rc == e3.E3_EINVAL and "kd is not 16-byte aligned" in lib.eagle3_last_error().decode()
    rc = lib.eagle3_attn_bwd(p.ref(), *([a] * 8), None, *([a] * 5), None)
    assert rc == e3.E3_EINVAL and "workspace is NULL" in lib.eagle3_last_error().decode()
    rc = lib.eagle3_attn_bwd(p.ref(), *([a] * 13), None, None)
    assert rc == e3.E3_EINVAL and "dvd is NULL" in lib.eagle3_last_error().decode()
    # the full-sequence entry points refuse a ring share
    q = prob(layout="zigzag", cp=2, T=256, T_kv=512)
    rc = lib.eagle3_attn_fwd(q.ref(), *([a] * 7), None)
    assert rc == e3.E3_EINVAL and "eagle3_shard_fwd" in lib.eagle3_last_error().decode()
    # lse_merge shape checks
    rc = lib.lse_merge(a, a, a, a, 1, 4, 2, 6, 0, None)
    assert rc == e3.E3_EINVAL
    rc = lib.lse_merge(a, a, a, a, 1, 4, 2, 8, 2, None)
    assert rc == e3.E3_EINVAL
    # an empty problem is a valid no-op
    z = prob(T=0, T_kv=0)
    assert lib.eagle3_attn_fwd(z.ref(), *([None] * 7), None) == e3.E3_OK
    assert lib.eagle3_attn_bwd(z.ref(), *([None] * 14), None) == e3.E3_OK
    assert lib.lse_merge(None, None, None, None, 1, 0, 2, 8, 0, None) == e3.E3_OK


def test_workspace_bytes():
    p = prob(B=1, T=1000, T_kv=1000, H=3)
    # backward: lse2 and delta (float32 [B, H, P]), P = T rounded up to 64 (one run),
    # and, with diagonal blocks, the block-0 part of dq (float32 [B, T, H, D])
    P = 1024
    assert p.workspace_bytes() == 2 * 1 * 3 * P * 4 + 1 * 1000 * 3 * 128 * 4
    assert prob(B=1, T=1000, T_kv=1000, H=3, num_blocks=1).workspace_bytes() == 2 * 3 * P * 4
    # zig-zag: each of the two local chunks is padded to 64 rows on its own
    # zig-zag: run i (of 150 rows) starts at roundup4(local start) + 68 i: 0 and
    # 152 + 68 = 220, and ends its padding at 220 + 192 = 412, rounded up to 448
    zz = e3.Problem(1, 300, 3 * 300, 3, 128, 3, 0.1, layout="zigzag", cp=3, rank=2)
    Pz = 448
    assert zz.workspace_bytes() == 2 * 3 * Pz * 4 + 300 * 3 * 128 * 4


SHARES = [
    ("full", 1000, 1, 0, None),
    ("full", 700, 1, 0, [0, 5, 300, 300, 700]),    # includes an empty document
    ("headshard", 1024, 4, 2, [0, 256, 1000, 1024]),
    ("contiguous", 320, 4, 0, None),
    ("contiguous", 320, 4, 3, None),
    ("contiguous", 300, 3, 1, [0, 100, 450, 900]),
    ("zigzag", 256, 4, 1, None),
    ("zigzag", 300, 3, 2, None),     # chunk 150: ragged tiles
    ("zigzag", 16384, 8, 3, None),   # the zig-zag workload's geometry
    # several documents, each cut into 2cp chunks (one empty, one of a single chunk row)
    ("zigzag", 256, 4, 1, [0, 8, 400, 400, 1024]),
    ("zigzag", 2048, 8, 3, [0, 4096, 4112, 12288, 16384]),
    ("zigzag", 90, 3, 0, [0, 30, 36, 270]),
]


def share_problem(layout, T, cp, rank, cu):
    Tkv = T * cp if layout in ("contiguous", "zigzag") else T
    return e3.Problem(1, T, Tkv, 2, 128, 3, 0.1, layout=layout, cp=cp if layout != "full" else 1,
                      rank=rank, cu_seqlens=cu)


def check_positions_and_pairs(layout, T, cp, rank, cu):
    p = share_problem(layout, T, cp, rank, cu)
    pos = p.query_positions()
    ocp = cp if layout in ("contiguous", "zigzag") else 1
    np.testing.assert_array_equal(pos, oracle.query_positions(layout, T, ocp, rank, cu))
    assert p.pair_count() == oracle.pair_count(layout, T, ocp, rank, cu)


@pytest.mark.parametrize("layout,T,cp,rank,cu", SHARES)
def test_shard_driver_positions_and_pair_counts(layout, T, cp, rank, cu):
    check_positions_and_pairs(layout, T, cp, rank, cu)


@pytest.mark.parametrize("layout,T,cp,rank,cu", SHARES)
def test_shard_driver_key_tiles_cover_exactly_the_visible_keys(layout, T, cp, rank, cu):
    """Every query row counts each visible block-0 key exactly once over the
    key tiles the kernel visits; unmasked tiles are fully visible to every row
    of their query tile; the tiles of a segment follow the ring order."""
    check_key_tile_coverage(layout, T, cp, rank, cu)


def check_key_tile_coverage(layout, T, cp, rank, cu):
    p = share_problem(layout, T, cp, rank, cu)
    ocp = cp if layout in ("contiguous", "zigzag") else 1
    qpos = oracle.query_positions(layout, T, ocp, rank, cu)
    lo = oracle.doc_start(cu, qpos)
    ntiles, BM = p.fwd_tiles()
    covered = np.zeros(T, dtype=bool)
    heavy = []
    if T > 4096:
        tiles = list(range(0, ntiles, max(1, ntiles // 16)))
    else:
        tiles = range(ntiles)
    for t in tiles:
        (r0, r1), segs = p.fwd_tile_segments(t)
        assert 0 < r1 - r0 <= BM
        covered[r0:r1] = True
        rows = np.arange(r0, r1)
        g, l = qpos[rows], lo[rows]
        assert np.all(np.diff(g) == 1)               # a tile is one run of positions
        counts = np.zeros((len(rows), ), dtype=np.int64)
        for (s0, s1, masked) in segs:
            ks = np.arange(s0, s1)
            vis = (ks[None, :] >= l[:, None]) & (ks[None, :] <= g[:, None])
            counts += vis.sum(axis=1)
            if not masked:
                assert vis.all()
        np.testing.assert_array_equal(counts, g - l + 1)
        # no key counted twice: the tiles' clipped ranges are disjoint
        spans = sorted((s0, s1) for (s0, s1, _) in segs)
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 <= b0
        heavy.append(int(g[0]))
        if layout in ("contiguous", "zigzag"):
            # the visited K/V chunks follow the ring: step j holds rank (r - j) mod cp
            # (zig-zag: chunks of the tile's document, 2cp of them)
            dlo = 0
            c = T if layout == "contiguous" else T // 2
            if layout == "zigzag" and cu is not None:
                d = int(np.searchsorted(cu, g[0], side="right")) - 1
                dlo, c = int(cu[d]), (int(cu[d + 1]) - int(cu[d])) // (2 * ocp)
            order = []
            for (s0, _, _) in segs:
                ch = (s0 - dlo) // c
                src = ch if ch < ocp else 2 * ocp - 1 - ch
                if not order or order[-1] != src:
                    order.append(src)
            ring = [s for s, _ in oracle.ring_steps(layout, ocp, rank)]
            assert order == [s for s in ring if s in order]
    if T <= 4096:
        assert covered.all()
    if cu is None and layout != "zigzag":
        assert heavy == sorted(heavy, reverse=True)    # latest positions (most keys) launch first



def random_share(i):
    """Seeded random share (layout, local T, cp, rank, cu_seqlens) within what the
    library accepts: any document list (empty documents included) for the full,
    head-shard and contiguous layouts; documents of whole 2cp chunks (one-row chunks
    and empty documents included) for the zig-zag layout."""
    rng = np.random.default_rng(7000 + i)
    layout = ("full", "headshard", "contiguous", "zigzag")[i % 4]
    cp = 1 if layout == "full" else int(rng.integers(1, 9))
    rank = int(rng.integers(0, cp))
    nd = int(rng.integers(1, 7))
    if layout == "zigzag":
        # a quarter of the documents empty, a quarter of one-row chunks
        kind = rng.integers(0, 4, size=nd)
        lens = [0 if k == 0 else 2 * cp if k == 1 else 2 * cp * int(rng.integers(1, 200 // cp + 2))
                for k in kind]
        if sum(lens) == 0:
            lens[0] = 2 * cp
        S = sum(lens)
        T = S // cp
    else:
        if layout == "full":
            T = S = int(rng.integers(1, 1500))
        elif layout == "headshard":
            S = T = cp * int(rng.integers(1, 300))
        else:
            T = int(rng.integers(1, 400))
            S = T * cp
        cuts = rng.integers(0, S + 1, size=nd - 1)
        if nd > 2:
            cuts[1] = cuts[0]                      # an empty document
        cuts = np.sort(cuts)
        lens = np.diff(np.concatenate([[0], cuts, [S]])).tolist()
    if nd == 1 and rng.random() < 0.5:
        return layout, T, cp, rank, None
    return layout, T, cp, rank, [0] + np.cumsum(lens).astype(int).tolist()


@pytest.mark.parametrize("i", range(48))
def test_shard_driver_on_seeded_random_shares(i):
    """Positions, pair counts and key-tile coverage of 48 seeded random shares
    (12 per layout) against the oracle: integer work, compared exactly."""
    layout, T, cp, rank, cu = random_share(i)
    check_positions_and_pairs(layout, T, cp, rank, cu)
    check_key_tile_coverage(layout, T, cp, rank, cu)

def test_workload_pair_counts_match_golden():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "pair_counts.json")))
    for name in synth.WORKLOADS:
        w = synth.workload(name)
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        p = e3.Problem(w.B, w.T, w.T_kv, w.H, w.D, w.num_blocks, w.scale, dtype=dt,
                       layout=w.layout, cp=w.cp, rank=w.rank, cu_seqlens=w.cu_seqlens())
        assert p.pair_count() == g[name]["P0"], name


def test_binding_checks_strides_against_the_problem():
    """The binding compares every k/v tensor's strides with the Problem's before
    calling the library (nothing is launched: it raises first)."""
    B, nb, T, H, D = 2, 3, 64, 2, 64
    cache = torch.zeros(B, nb, T, H, D)
    dense = e3.Problem(B, T, T, H, D, nb, 0.125, dtype=torch.float32)
    q = torch.zeros(B, T, H, D)
    with pytest.raises(ValueError, match="strides"):
        e3.fwd(dense, q, cache[:, 0], cache[:, 0], cache[:, 1:], cache[:, 1:])
    blk = nb * T * H * D
    strided = e3.Problem(B, T, T, H, D, nb, 0.125, dtype=torch.float32, k0_batch_stride=blk,
                         kd_batch_stride=blk, kd_block_stride=T * H * D)
    with pytest.raises(ValueError, match="strides"):
        e3.fwd(strided, q, cache[:, 0].contiguous(), cache[:, 0], cache[:, 1:], cache[:, 1:])
    assert strided.k0_strides == (blk, H * D, D, 1)
    assert strided.kd_strides == (blk, T * H * D, H * D, D, 1)
    g = e3._strided_empty((B, nb - 1, T, H, D), strided.kd_strides, torch.float32, "cpu")
    assert g.stride() == strided.kd_strides


def test_ring_step_entry_points_refuse_a_step_out_of_range():
    lib = e3.lib()
    a = ctypes.c_void_p(0x1000)        # never dereferenced: validation fails first
    for layout, cp, T, Tkv in (("contiguous", 4, 256, 1024), ("zigzag", 4, 256, 1024), ("full", 1, 256, 256)):
        p = prob(layout=layout, cp=cp, rank=0, T=T, T_kv=Tkv)
        for step in (-1, cp):
            rc = lib.eagle3_ring_fwd_step(p.ref(), step, a, a, a, a, a, None)
            assert rc == e3.E3_EINVAL and "ring step" in lib.eagle3_last_error().decode()
            rc = lib.eagle3_ring_bwd_step(p.ref(), step, *([a] * 10), None)
            assert rc == e3.E3_EINVAL and "ring step" in lib.eagle3_last_error().decode()


def test_target_cp_forward_refuses_what_it_does_not_compute():
    lib = e3.lib()
    a = ctypes.c_void_p(0x1000)        # never dereferenced: validation fails first
    p = prob(layout="contiguous", cp=4, rank=1, T=256, T_kv=1024, num_blocks=3)
    assert lib.eagle3_target_cp_fwd(p.ref(), a, a, a, a, a, None) == e3.E3_EINVAL
    assert "num_blocks must be 1" in lib.eagle3_last_error().decode()
    p = prob(layout="zigzag", cp=4, rank=1, T=256, T_kv=1024, num_blocks=1)
    assert lib.eagle3_target_cp_fwd(p.ref(), a, a, a, a, a, None) == e3.E3_EINVAL
    assert "FULL or CONTIGUOUS" in lib.eagle3_last_error().decode()
    p = prob(B=2, layout="contiguous", cp=4, rank=1, T=256, T_kv=1024, num_blocks=1,
             k0_batch_stride=4096 * 256)
    assert lib.eagle3_target_cp_fwd(p.ref(), a, a, a, a, a, None) == e3.E3_EINVAL
    assert "dense head-major" in lib.eagle3_last_error().decode()


def test_noalloc_backward_refuses_a_problem_larger_than_its_scratch():
    """The no-allocation backward's static scratch holds 2 x B*H*P floats; a larger
    problem is refused before anything is launched (no device is touched)."""
    lib = e3.lib()
    cap = lib.eagle3_bwd_noalloc_max_scratch_bytes()
    assert cap == 16 << 20
    H = 64
    T = cap // (2 * 4 * H) + 64
    p = e3.Problem(1, T, T, H, 128, 1, 0.088, dtype=torch.bfloat16)
    a = ctypes.c_void_p(0x1000)        # never dereferenced: the size check fails first
    rc = lib.eagle3_bwd_noalloc(p.ref(), *([a] * 13), None)
    assert rc == e3.E3_EINVAL and "scratch" in lib.eagle3_last_error().decode()


def test_ulysses_transforms_refuse_segments_that_are_not_whole_words():
    """The re-sharding copies move 4-byte words: a bf16 head-group row of an odd
    number of elements is refused (nothing is launched), float32 is accepted up to
    the launch and an even bf16 row passes validation too."""
    lib = e3.lib()
    a, b = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000)   # never dereferenced here
    for name in ("eagle3_ulysses_seq_to_head", "eagle3_ulysses_head_to_seq"):
        f = getattr(lib, name)
        for stage in (0, 1):
            rc = f(stage, e3.DTYPES[torch.bfloat16], 1, 5, 2, 3, 2, a, b, None)   # H/uly*D = 3
            assert rc == e3.E3_EUNSUPPORTED and "multiple of 4 bytes" in lib.eagle3_last_error().decode()
            rc = f(stage, e3.DTYPES[torch.bfloat16], 1, 0, 2, 4, 2, a, b, None)   # S_local = 0: nothing to do
            assert rc == e3.E3_OK


def test_backward_refuses_a_delta_offset_beyond_32_bits():
    """lse*log2(e) and delta sit B*H*P floats apart in the workspace and the kernels
    address one from the other with a 32-bit byte offset: a larger problem is refused
    before anything is launched."""
    lib = e3.lib()
    a = ctypes.c_void_p(0x1000)        # never dereferenced: the check fails first
    T = 1 << 20
    p = e3.Problem(1, T, T, 1100, 64, 1, 0.125, dtype=torch.bfloat16)      # 1100 * 2^20 * 4 B > 4 GiB
    rc = lib.eagle3_attn_bwd(p.ref(), *([a] * 9), a, a, a, None, None, None)
    assert rc == e3.E3_EUNSUPPORTED and "32-bit" in lib.eagle3_last_error().decode()
    rc = lib.eagle3_ring_bwd_step(p.ref(), 0, *([a] * 10), None)
    assert rc == e3.E3_EUNSUPPORTED and "32-bit" in lib.eagle3_last_error().decode()
