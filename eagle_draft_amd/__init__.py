"""Python binding of libeagle3_attn.so: EAGLE-3 mixed attention on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the library's
HIP kernels. PyTorch supplies device memory and the current HIP stream.

    import eagle_draft_amd as e3
    prob = e3.Problem(B, T, T_kv, H, D, num_blocks, scale, dtype=torch.bfloat16,
                      layout="full", cp=1, rank=0, cu_seqlens=None)
    out, lse = e3.fwd(prob, q, k0, v0, kd, vd)
    dq, dk0, dv0, dkd, dvd = e3.bwd(prob, dout, q, k0, v0, kd, vd, out, lse)
    out = e3.cached_attention(q, cache_k, cache_v, scale)   # autograd, list API

Shapes (FlashAttention layout of the pages):
    q, dout, out, dq     [B, T, H, D]
    k0, v0, dk0, dv0     [B, T_kv, H, D]   block 0, full sequence in global order
    kd, vd, dkd, dvd     [B, N, T, H, D]   blocks 1..N (N = num_blocks - 1)
    lse                  [B, H, T] float32
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch  # loaded first: the library then shares torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libeagle3_attn.so")
ABI_VERSION = 4

E3_OK, E3_EINVAL, E3_EUNSUPPORTED, E3_EHIP = 0, -1, -2, -3
LAYOUTS = {"full": 0, "contiguous": 1, "zigzag": 2, "headshard": 3}
DTYPES = {torch.bfloat16: 0, torch.float32: 1}


class E3Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"eagle3 error {code}: {msg}")
        self.code = code


class _Problem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("T", ctypes.c_int32),
        ("T_kv", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("scale", ctypes.c_float), ("layout", ctypes.c_int32),
        ("cp", ctypes.c_int32), ("rank", ctypes.c_int32), ("num_docs", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_dev", ctypes.c_void_p),
        ("k0_batch_stride", ctypes.c_int64), ("kd_batch_stride", ctypes.c_int64),
        ("kd_block_stride", ctypes.c_int64),
    ]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m eagle_draft_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_Problem)
    vp = ctypes.c_void_p
    lib.eagle3_abi_version.restype = ctypes.c_int
    lib.eagle3_last_error.restype = ctypes.c_char_p
    lib.eagle3_bwd_workspace_bytes.argtypes = [P]
    lib.eagle3_bwd_workspace_bytes.restype = ctypes.c_size_t
    for name in ("eagle3_attn_fwd", "eagle3_shard_fwd"):
        f = getattr(lib, name)
        f.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        f.restype = ctypes.c_int
    for name in ("eagle3_attn_bwd", "eagle3_shard_bwd"):
        f = getattr(lib, name)
        f.argtypes = [P] + [vp] * 14 + [vp]
        f.restype = ctypes.c_int
    lib.eagle3_bwd_noalloc.argtypes = [P] + [vp] * 13 + [vp]
    lib.eagle3_bwd_noalloc.restype = ctypes.c_int
    lib.eagle3_bwd_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
    lib.lse_merge.argtypes = [vp, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                              ctypes.c_int, ctypes.c_int, vp]
    lib.lse_merge.restype = ctypes.c_int
    lib.eagle3_query_positions.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    lib.eagle3_query_positions.restype = ctypes.c_int
    lib.eagle3_pair_count.argtypes = [P]
    lib.eagle3_pair_count.restype = ctypes.c_int64
    lib.eagle3_fwd_tiles.argtypes = [P, ctypes.POINTER(ctypes.c_int32)]
    lib.eagle3_fwd_tiles.restype = ctypes.c_int
    lib.eagle3_fwd_tile_segments.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int32),
                                             ctypes.POINTER(ctypes.c_int32), ctypes.c_int]
    lib.eagle3_fwd_tile_segments.restype = ctypes.c_int
    for name in ("eagle3_ulysses_seq_to_head", "eagle3_ulysses_head_to_seq"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_int] * 7 + [vp, vp, vp]
        f.restype = ctypes.c_int
    for name in ("eagle3_ulysses_lse_gather", "eagle3_ulysses_lse_scatter"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_int] * 5 + [vp, vp, vp]
        f.restype = ctypes.c_int
    lib.eagle3_target_cp_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.eagle3_target_cp_fwd.restype = ctypes.c_int
    lib.eagle3_ring_fwd_step.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    lib.eagle3_ring_fwd_step.restype = ctypes.c_int
    lib.eagle3_diag_merge_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.eagle3_diag_merge_fwd.restype = ctypes.c_int
    lib.eagle3_ring_bwd_step.argtypes = [P, ctypes.c_int] + [vp] * 10 + [vp]
    lib.eagle3_ring_bwd_step.restype = ctypes.c_int
    lib.eagle3_diag_bwd.argtypes = [P] + [vp] * 10 + [vp]
    lib.eagle3_diag_bwd.restype = ctypes.c_int
    lib.eagle3_set_timing_events.argtypes = [vp, ctypes.c_int]
    lib.eagle3_set_timing_events.restype = ctypes.c_int
    lib.eagle3_timing_events_recorded.restype = ctypes.c_int
    v = lib.eagle3_abi_version()
    if v != ABI_VERSION:
        raise RuntimeError(f"libeagle3_attn ABI version {v} != binding version {ABI_VERSION}")
    _lib = lib
    return lib


def lib():
    return _load()


def _check(rc: int):
    if rc != E3_OK:
        raise E3Error(rc, _load().eagle3_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Problem:
    """One problem shape: sizes, scale, layout and documents (host and device
    copies of cu_seqlens). Reusable across calls."""

    def __init__(self, B: int, T: int, T_kv: int, H: int, D: int, num_blocks: int, scale: float,
                 dtype=torch.bfloat16, layout: str = "full", cp: int = 1, rank: int = 0,
                 cu_seqlens=None, device=None, k0_batch_stride: int = 0,
                 kd_batch_stride: int = 0, kd_block_stride: int = 0):
        if dtype not in DTYPES:
            raise ValueError(f"dtype {dtype} not supported (bfloat16 or float32)")
        if layout not in LAYOUTS:
            raise ValueError(f"layout {layout!r} not one of {sorted(LAYOUTS)}")
        self.dtype = dtype
        self.B, self.T, self.T_kv, self.H, self.D = B, T, T_kv, H, D
        self.num_blocks = num_blocks
        self.N = num_blocks - 1
        self.scale = float(scale)
        self.layout, self.cp, self.rank = layout, cp, rank
        self._cu_host = None
        self._cu_dev = None
        nd = 0
        if cu_seqlens is not None:
            if isinstance(cu_seqlens, torch.Tensor):
                host = cu_seqlens.detach().to("cpu", torch.int32).numpy()
            else:
                host = np.asarray(cu_seqlens, dtype=np.int32)
            self._cu_host = np.ascontiguousarray(host, dtype=np.int32)
            nd = len(self._cu_host) - 1
            if nd > 1 and device is not None and torch.device(device).type == "cuda":
                self._cu_dev = torch.from_numpy(self._cu_host).to(device)
        self.num_docs = nd
        s = _Problem()
        s.dtype = DTYPES[dtype]
        s.B, s.T, s.T_kv, s.H, s.D = B, T, T_kv, H, D
        s.num_blocks = num_blocks
        s.scale = self.scale
        s.layout = LAYOUTS[layout]
        s.cp, s.rank = cp, rank
        s.num_docs = nd
        if self._cu_host is not None:
            s.cu_seqlens_host = self._cu_host.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        s.cu_seqlens_dev = None if self._cu_dev is None else self._cu_dev.data_ptr()
        s.k0_batch_stride = k0_batch_stride
        s.kd_batch_stride = kd_batch_stride
        s.kd_block_stride = kd_block_stride
        self._s = s
        # Element strides of the k/v tensors (block 0 and the diagonal blocks) and
        # of their gradients; 0 in the arguments means dense.
        HD = H * D
        k0_bs = k0_batch_stride or T_kv * HD
        kd_blk = kd_block_stride or T * HD
        kd_bs = kd_batch_stride or (num_blocks - 1) * T * HD
        self.k0_strides = (k0_bs, HD, D, 1)
        self.kd_strides = (kd_bs, kd_blk, HD, D, 1)
        self.dense_kv = (k0_bs == T_kv * HD and kd_blk == T * HD
                         and kd_bs == (num_blocks - 1) * T * HD)

    def ref(self):
        return ctypes.byref(self._s)

    # host-side inspection of the shard driver (no GPU needed)
    def query_positions(self) -> np.ndarray:
        out = np.zeros(self.T, dtype=np.int64)
        _check(_load().eagle3_query_positions(self.ref(), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))))
        return out

    def pair_count(self) -> int:
        n = _load().eagle3_pair_count(self.ref())
        if n < 0:
            _check(int(n))
        return int(n)

    def fwd_tiles(self):
        rows = ctypes.c_int32(0)
        n = _load().eagle3_fwd_tiles(self.ref(), ctypes.byref(rows))
        if n < 0:
            _check(n)
        return n, rows.value

    def fwd_tile_segments(self, tile: int):
        rows = (ctypes.c_int32 * 2)()
        n = _load().eagle3_fwd_tile_segments(self.ref(), tile, rows, None, 0)
        if n < 0:
            _check(n)
        seg = (ctypes.c_int32 * (3 * max(n, 1)))()
        n2 = _load().eagle3_fwd_tile_segments(self.ref(), tile, rows, seg, n)
        if n2 < 0:
            _check(n2)
        return (rows[0], rows[1]), [(seg[3 * i], seg[3 * i + 1], seg[3 * i + 2]) for i in range(n)]

    def workspace_bytes(self) -> int:
        """Backward workspace bytes."""
        n = _load().eagle3_bwd_workspace_bytes(self.ref())
        if n == 0 and self.T > 0:
            _check(E3_EINVAL)
        return int(n)


def _check_tensor(name, t, shape, dtype, device, strides=None):
    """Checks device, dtype and shape, and that the memory layout is the dense
    row-major one, or, for the k/v tensors, the one given by `strides` (in
    elements; dimensions of size 1 are not checked). The inner [rows, H, D]
    part must be dense either way."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if strides is None:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return
    for dim, (n, want, got) in enumerate(zip(t.shape, strides, t.stride())):
        if n > 1 and want != got:
            raise ValueError(f"{name} has strides {tuple(t.stride())}, expected {tuple(strides)} "
                             f"(dimension {dim}); pass the strides in the Problem")


def _strided_empty(shape, strides, dtype, device):
    """An uninitialised tensor of the given shape and element strides."""
    extent = 1 + sum((n - 1) * s for n, s in zip(shape, strides) if n > 0)
    if any(n == 0 for n in shape):
        extent = 0
    return torch.empty(max(extent, 1), dtype=dtype, device=device).as_strided(shape, strides)


def _entry(prob: Problem, kind: str):
    whole = prob.layout in ("full", "headshard")
    return getattr(_load(), f"eagle3_{'attn' if whole else 'shard'}_{kind}")


def fwd(prob: Problem, q, k0, v0, kd=None, vd=None, out=None, lse=None):
    """Forward: returns (out [B,T,H,D] in q's dtype, lse [B,H,T] float32)."""
    dev = q.device
    B, T, Tkv, H, D, N = prob.B, prob.T, prob.T_kv, prob.H, prob.D, prob.N
    _check_tensor("q", q, (B, T, H, D), prob.dtype, dev)
    _check_tensor("k0", k0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("v0", v0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    if N > 0:
        _check_tensor("kd", kd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
        _check_tensor("vd", vd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    _check_tensor("out", out, (B, T, H, D), prob.dtype, dev)
    _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    _check(_entry(prob, "fwd")(prob.ref(), _ptr(q), _ptr(k0), _ptr(v0),
                               _ptr(kd if N > 0 else None), _ptr(vd if N > 0 else None),
                               _ptr(out), _ptr(lse), _stream()))
    return out, lse


def bwd(prob: Problem, dout, q, k0, v0, kd, vd, out, lse, grads=None, workspace=None):
    """Backward against the merged out/lse: returns (dq, dk0, dv0, dkd, dvd)."""
    dev = q.device
    B, T, Tkv, H, D, N = prob.B, prob.T, prob.T_kv, prob.H, prob.D, prob.N
    for name, t, shp in (("dout", dout, (B, T, H, D)), ("q", q, (B, T, H, D)),
                         ("out", out, (B, T, H, D))):
        _check_tensor(name, t, shp, prob.dtype, dev)
    _check_tensor("k0", k0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("v0", v0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    if N > 0:
        _check_tensor("kd", kd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
        _check_tensor("vd", vd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
    if grads is None:
        # gradients take the strides of the tensors they differentiate
        grads = (torch.empty_like(q),
                 _strided_empty((B, Tkv, H, D), prob.k0_strides, prob.dtype, dev),
                 _strided_empty((B, Tkv, H, D), prob.k0_strides, prob.dtype, dev),
                 _strided_empty((B, N, T, H, D), prob.kd_strides, prob.dtype, dev),
                 _strided_empty((B, N, T, H, D), prob.kd_strides, prob.dtype, dev))
    dq, dk0, dv0, dkd, dvd = grads
    _check_tensor("dq", dq, (B, T, H, D), prob.dtype, dev)
    _check_tensor("dk0", dk0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("dv0", dv0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    if N > 0:
        _check_tensor("dkd", dkd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
        _check_tensor("dvd", dvd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
    if workspace is None:
        workspace = torch.empty(max(prob.workspace_bytes(), 256), dtype=torch.uint8, device=dev)
    _check(_entry(prob, "bwd")(prob.ref(), _ptr(dout), _ptr(q), _ptr(k0), _ptr(v0),
                               _ptr(kd if N > 0 else None), _ptr(vd if N > 0 else None),
                               _ptr(out), _ptr(lse), _ptr(workspace), _ptr(dq), _ptr(dk0),
                               _ptr(dv0), _ptr(dkd if N > 0 else None),
                               _ptr(dvd if N > 0 else None), _stream()))
    return dq, dk0, dv0, dkd, dvd


def bwd_noalloc(prob: Problem, dout, q, k0, v0, kd, vd, out, lse, grads):
    """The backward through eagle3_bwd_noalloc: no workspace, no allocation by the
    library; the caller passes the gradient buffers (dq, dk0, dv0, dkd, dvd)."""
    dev = q.device
    B, T, Tkv, H, D, N = prob.B, prob.T, prob.T_kv, prob.H, prob.D, prob.N
    for name, t in (("dout", dout), ("q", q), ("out", out)):
        _check_tensor(name, t, (B, T, H, D), prob.dtype, dev)
    _check_tensor("k0", k0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("v0", v0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    dq, dk0, dv0, dkd, dvd = grads
    _check_tensor("dq", dq, (B, T, H, D), prob.dtype, dev)
    _check_tensor("dk0", dk0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("dv0", dv0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    if N > 0:
        for name, t in (("kd", kd), ("vd", vd), ("dkd", dkd), ("dvd", dvd)):
            _check_tensor(name, t, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
    _check(_load().eagle3_bwd_noalloc(prob.ref(), _ptr(dout), _ptr(q), _ptr(k0), _ptr(v0),
                                      _ptr(kd if N > 0 else None), _ptr(vd if N > 0 else None),
                                      _ptr(out), _ptr(lse), _ptr(dq), _ptr(dk0), _ptr(dv0),
                                      _ptr(dkd if N > 0 else None), _ptr(dvd if N > 0 else None),
                                      _stream()))
    return grads


def lse_merge(out, lse, block_out, block_lse, block_lse_layout: int = 0):
    """In-place merge of (block_out, block_lse) into float32 (out [B,T,H,D], lse [B,H,T])."""
    B, T, H, D = out.shape
    for name, t in (("out", out), ("lse", lse), ("block_out", block_out), ("block_lse", block_lse)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != out.device:
            raise ValueError(f"{name} must be a contiguous float32 tensor on {out.device}")
    if tuple(block_out.shape) != (B, T, H, D) or tuple(lse.shape) != (B, H, T):
        raise ValueError("shape mismatch")
    want = (B, H, T) if block_lse_layout == 0 else (B, T, H)
    if tuple(block_lse.shape) != want:
        raise ValueError(f"block_lse has shape {tuple(block_lse.shape)}, expected {want}")
    _check(_load().lse_merge(_ptr(out), _ptr(lse), _ptr(block_out), _ptr(block_lse), B, T, H, D,
                             block_lse_layout, _stream()))
    return out, lse


def target_cp_fwd(prob: Problem, q, k, v, out=None, lse=None, want_lse: bool = True):
    """Frozen-target context-parallel forward (head-major): q [B,H,T,D] local
    contiguous queries, k/v [B,H,T_kv,D] the all-gathered K/V; returns (out [B,H,T,D],
    lse [B,H,T] float32 or None). prob: layout "contiguous" (or "full"), num_blocks 1."""
    dev = q.device
    B, T, Tkv, H, D = prob.B, prob.T, prob.T_kv, prob.H, prob.D
    _check_tensor("q", q, (B, H, T, D), prob.dtype, dev)
    _check_tensor("k", k, (B, H, Tkv, D), prob.dtype, dev)
    _check_tensor("v", v, (B, H, Tkv, D), prob.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, (B, H, T, D), prob.dtype, dev)
    if lse is None and want_lse:
        lse = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    if lse is not None:
        _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    _check(_load().eagle3_target_cp_fwd(prob.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                        _stream()))
    return out, lse


# ---- Ulysses re-sharding (the local halves around the all-to-all) ------------------

def _uly_shapes(kind, stage, B, S_local, H, D, uly):
    Hl, Sf = H // uly, uly * S_local
    send = (uly, B, S_local, Hl, D)
    if kind == "seq_to_head":
        return ((B, S_local, H, D), send) if stage == 0 else (send, (B, Sf, Hl, D))
    if kind == "head_to_seq":
        return ((B, Sf, Hl, D), send) if stage == 0 else (send, (B, S_local, H, D))
    lsend = (uly, B, Hl, S_local)
    if kind == "lse_gather":
        return ((B, H, S_local), lsend) if stage == 0 else (lsend, (B, Hl, Sf))
    return ((B, Hl, Sf), lsend) if stage == 0 else (lsend, (B, H, S_local))


def ulysses(kind: str, stage: int, src: torch.Tensor, uly: int, B: int, S_local: int, H: int,
            D: int = 1, out: Optional[torch.Tensor] = None):
    """One local half of a Ulysses transform (kind: seq_to_head, head_to_seq,
    lse_gather, lse_scatter; stage 0 = pack into the all-to-all send buffer,
    1 = unpack the receive buffer). H is the global head count."""
    if H % uly:
        raise ValueError(f"H={H} must divide by the Ulysses degree {uly}")
    sin, sout = _uly_shapes(kind, stage, B, S_local, H, D, uly)
    lse = kind.startswith("lse")
    dt = torch.float32 if lse else src.dtype
    if lse and src.dtype != torch.float32:
        raise ValueError("lse must be float32")
    if not lse and dt not in DTYPES:
        raise ValueError(f"dtype {dt} not supported")
    _check_tensor("src", src, sin, dt, src.device)
    if out is None:
        out = torch.empty(sout, dtype=dt, device=src.device)
    _check_tensor("out", out, sout, dt, src.device)
    lib = _load()
    if lse:
        _check(getattr(lib, f"eagle3_ulysses_{kind}")(stage, B, S_local, H, uly, _ptr(src), _ptr(out),
                                                      _stream()))
    else:
        _check(getattr(lib, f"eagle3_ulysses_{kind}")(stage, DTYPES[dt], B, S_local, H, D, uly, _ptr(src),
                                                      _ptr(out), _stream()))
    return out


# ---- ring-step mode (one ring step of one share on the local GPU) -------------------

def ring_fwd_step(prob: Problem, step: int, q, k0, v0, out_step=None, lse_step=None):
    """Block-0 attention over ring step `step`'s keys only: float32 (out [B,T,H,D],
    lse [B,H,T]); rows that see no key of the step get out = 0, lse = -inf."""
    dev = q.device
    B, T, Tkv, H, D = prob.B, prob.T, prob.T_kv, prob.H, prob.D
    _check_tensor("q", q, (B, T, H, D), prob.dtype, dev)
    _check_tensor("k0", k0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("v0", v0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    if out_step is None:
        out_step = torch.empty(B, T, H, D, dtype=torch.float32, device=dev)
    if lse_step is None:
        lse_step = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    _check_tensor("out_step", out_step, (B, T, H, D), torch.float32, dev)
    _check_tensor("lse_step", lse_step, (B, H, T), torch.float32, dev)
    _check(_load().eagle3_ring_fwd_step(prob.ref(), step, _ptr(q), _ptr(k0), _ptr(v0), _ptr(out_step),
                                        _ptr(lse_step), _stream()))
    return out_step, lse_step


def diag_merge_fwd(prob: Problem, q, kd, vd, out_acc, lse_acc, out=None, lse=None):
    """Merges the diagonal blocks into the chained float32 block-0 (out_acc, lse_acc):
    returns the final (out in q's dtype, lse float32)."""
    dev = q.device
    B, T, H, D, N = prob.B, prob.T, prob.H, prob.D, prob.N
    _check_tensor("q", q, (B, T, H, D), prob.dtype, dev)
    if N > 0:
        _check_tensor("kd", kd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
        _check_tensor("vd", vd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
    _check_tensor("out_acc", out_acc, (B, T, H, D), torch.float32, dev)
    _check_tensor("lse_acc", lse_acc, (B, H, T), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    _check_tensor("out", out, (B, T, H, D), prob.dtype, dev)
    _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    _check(_load().eagle3_diag_merge_fwd(prob.ref(), _ptr(q), _ptr(kd if N > 0 else None),
                                         _ptr(vd if N > 0 else None), _ptr(out_acc), _ptr(lse_acc),
                                         _ptr(out), _ptr(lse), _stream()))
    return out, lse


def ring_bwd_step(prob: Problem, step: int, dout, q, k0, v0, out, lse, dq_acc, dk0_acc, dv0_acc,
                  workspace=None):
    """Block-0 backward of ring step `step` against the merged out/lse: adds into the
    float32 accumulators dq_acc [B,T,H,D] and dk0_acc / dv0_acc [B,T_kv,H,D] (the rows
    of the step's keys). Returns the accumulators."""
    dev = q.device
    B, T, Tkv, H, D = prob.B, prob.T, prob.T_kv, prob.H, prob.D
    for name, t in (("dout", dout), ("q", q), ("out", out)):
        _check_tensor(name, t, (B, T, H, D), prob.dtype, dev)
    _check_tensor("k0", k0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("v0", v0, (B, Tkv, H, D), prob.dtype, dev, prob.k0_strides)
    _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    _check_tensor("dq_acc", dq_acc, (B, T, H, D), torch.float32, dev)
    _check_tensor("dk0_acc", dk0_acc, (B, Tkv, H, D), torch.float32, dev, prob.k0_strides)
    _check_tensor("dv0_acc", dv0_acc, (B, Tkv, H, D), torch.float32, dev, prob.k0_strides)
    if workspace is None:
        workspace = torch.empty(max(prob.workspace_bytes(), 256), dtype=torch.uint8, device=dev)
    _check(_load().eagle3_ring_bwd_step(prob.ref(), step, _ptr(dout), _ptr(q), _ptr(k0), _ptr(v0),
                                        _ptr(out), _ptr(lse), _ptr(workspace), _ptr(dq_acc),
                                        _ptr(dk0_acc), _ptr(dv0_acc), _stream()))
    return dq_acc, dk0_acc, dv0_acc


def diag_bwd(prob: Problem, dout, q, kd, vd, out, lse, dq_acc, grads=None):
    """Closed-form diagonal gradients and the final dq = dq_acc + diagonal part:
    returns (dq, dkd, dvd) in q's dtype."""
    dev = q.device
    B, T, H, D, N = prob.B, prob.T, prob.H, prob.D, prob.N
    for name, t in (("dout", dout), ("q", q), ("out", out)):
        _check_tensor(name, t, (B, T, H, D), prob.dtype, dev)
    _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    _check_tensor("dq_acc", dq_acc, (B, T, H, D), torch.float32, dev)
    if N > 0:
        _check_tensor("kd", kd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
        _check_tensor("vd", vd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
    if grads is None:
        grads = (torch.empty_like(q),
                 _strided_empty((B, N, T, H, D), prob.kd_strides, prob.dtype, dev),
                 _strided_empty((B, N, T, H, D), prob.kd_strides, prob.dtype, dev))
    dq, dkd, dvd = grads
    _check_tensor("dq", dq, (B, T, H, D), prob.dtype, dev)
    if N > 0:
        _check_tensor("dkd", dkd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
        _check_tensor("dvd", dvd, (B, N, T, H, D), prob.dtype, dev, prob.kd_strides)
    _check(_load().eagle3_diag_bwd(prob.ref(), _ptr(dout), _ptr(q), _ptr(kd if N > 0 else None),
                                   _ptr(vd if N > 0 else None), _ptr(out), _ptr(lse), _ptr(dq_acc),
                                   _ptr(dq), _ptr(dkd if N > 0 else None),
                                   _ptr(dvd if N > 0 else None), _stream()))
    return dq, dkd, dvd


class _CachedAttention(torch.autograd.Function):
    """List form: separate q, k0, v0, kd, vd tensors."""

    @staticmethod
    def forward(ctx, prob, q, k0, v0, kd, vd):
        out, lse = fwd(prob, q, k0, v0, kd, vd)
        ctx.prob = prob
        ctx.save_for_backward(q, k0, v0, kd, vd, out, lse)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k0, v0, kd, vd, out, lse = ctx.saved_tensors
        dq, dk0, dv0, dkd, dvd = bwd(ctx.prob, dout.contiguous(), q, k0, v0, kd, vd, out, lse)
        return None, dq, dk0, dv0, dkd, dvd


class _CachedAttentionStacked(torch.autograd.Function):
    """Stacked form: cache_k / cache_v [B, nb, T, H, D] (dense). Block 0 and the
    diagonal blocks are views of the cache passed to the kernels through their
    batch and block strides; the gradients of the caches are written the same way
    into one [B, nb, T, H, D] buffer each. With a separate block-0 k0/v0 (a ring
    share), the cache's block 0 is unused and gets a zero gradient."""

    @staticmethod
    def forward(ctx, prob, q, cache_k, cache_v, k0, v0):
        own = k0 is None
        kk0 = cache_k[:, 0] if own else k0
        vv0 = cache_v[:, 0] if own else v0
        out, lse = fwd(prob, q, kk0, vv0, cache_k[:, 1:], cache_v[:, 1:])
        ctx.prob, ctx.own = prob, own
        ctx.save_for_backward(q, cache_k, cache_v, kk0, vv0, out, lse)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, cache_k, cache_v, k0, v0, out, lse = ctx.saved_tensors
        prob = ctx.prob
        dck = torch.empty_like(cache_k)
        dcv = torch.empty_like(cache_v)
        if ctx.own:
            dk0, dv0 = dck[:, 0], dcv[:, 0]
        else:
            dck[:, 0].zero_()
            dcv[:, 0].zero_()
            dk0, dv0 = torch.empty_like(k0), torch.empty_like(v0)
        grads = (torch.empty_like(q), dk0, dv0, dck[:, 1:], dcv[:, 1:])
        dq, dk0, dv0, _, _ = bwd(prob, dout.contiguous(), q, k0, v0, cache_k[:, 1:], cache_v[:, 1:],
                                 out, lse, grads=grads)
        if ctx.own:
            return None, dq, dck, dcv, None, None
        return None, dq, dck, dcv, dk0, dv0


def cached_attention(q: torch.Tensor, cache_k, cache_v, scale: float, cu_seqlens=None,
                     layout: str = "full", cp: int = 1, rank: int = 0,
                     k0: Optional[torch.Tensor] = None, v0: Optional[torch.Tensor] = None):
    """EAGLE-3 mixed attention with autograd, in the forms of the pages'
    cached_*_attention (ring_attention page, `cached_ring_attention`;
    `_CachedRingAttention` stacks the lists into [B, nb, T, H, D]):
      - cache_k / cache_v as lists of [B, T, H, D] (index 0 = the step-0 sequence,
        1.. = TTT steps); the TTT blocks are stacked (one copy);
      - cache_k / cache_v as dense [B, nb, T, H, D] tensors: no copy, the blocks
        are read and their gradients written through strides.
    For a ring share (contiguous / zig-zag), pass the full-sequence block-0 k0/v0
    [B, T_kv, H, D] explicitly; the cache's block 0 is then ignored. Returns out
    [B, T, H, D] in q's dtype."""
    B, T, H, D = q.shape
    if isinstance(cache_k, torch.Tensor):
        if not (isinstance(cache_v, torch.Tensor) and cache_k.shape == cache_v.shape
                and cache_k.dim() == 5 and cache_k.is_contiguous() and cache_v.is_contiguous()):
            raise ValueError("stacked caches must be dense [B, nb, T, H, D] tensors of one shape")
        nb = cache_k.shape[1]
        if tuple(cache_k.shape) != (B, nb, T, H, D):
            raise ValueError(f"cache shape {tuple(cache_k.shape)} does not match q {tuple(q.shape)}")
        Tkv = T if k0 is None else k0.shape[1]
        blk = nb * T * H * D
        prob = Problem(B, T, Tkv, H, D, nb, scale, dtype=q.dtype, layout=layout, cp=cp,
                       rank=rank, cu_seqlens=cu_seqlens, device=q.device,
                       k0_batch_stride=blk if k0 is None else 0, kd_batch_stride=blk,
                       kd_block_stride=T * H * D)
        return _CachedAttentionStacked.apply(
            prob, q.contiguous(), cache_k, cache_v,
            None if k0 is None else k0.contiguous(), None if v0 is None else v0.contiguous())
    k0 = cache_k[0] if k0 is None else k0
    v0 = cache_v[0] if v0 is None else v0
    nb = len(cache_k)
    if nb > 1:
        kd = torch.stack(list(cache_k[1:]), 1).contiguous()
        vd = torch.stack(list(cache_v[1:]), 1).contiguous()
    else:
        kd = vd = torch.empty(B, 0, T, H, D, dtype=q.dtype, device=q.device)
    prob = Problem(B, T, k0.shape[1], H, D, nb, scale, dtype=q.dtype, layout=layout, cp=cp,
                   rank=rank, cu_seqlens=cu_seqlens, device=q.device)
    return _CachedAttention.apply(prob, q.contiguous(), k0.contiguous(), v0.contiguous(), kd, vd)
