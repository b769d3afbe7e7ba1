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
ABI_VERSION = 3

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


def _check_tensor(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _entry(prob: Problem, kind: str):
    whole = prob.layout in ("full", "headshard")
    return getattr(_load(), f"eagle3_{'attn' if whole else 'shard'}_{kind}")


def fwd(prob: Problem, q, k0, v0, kd=None, vd=None, out=None, lse=None):
    """Forward: returns (out [B,T,H,D] in q's dtype, lse [B,H,T] float32)."""
    dev = q.device
    B, T, Tkv, H, D, N = prob.B, prob.T, prob.T_kv, prob.H, prob.D, prob.N
    _check_tensor("q", q, (B, T, H, D), prob.dtype, dev)
    _check_tensor("k0", k0, (B, Tkv, H, D), prob.dtype, dev)
    _check_tensor("v0", v0, (B, Tkv, H, D), prob.dtype, dev)
    if N > 0:
        _check_tensor("kd", kd, (B, N, T, H, D), prob.dtype, dev)
        _check_tensor("vd", vd, (B, N, T, H, D), prob.dtype, dev)
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
                         ("k0", k0, (B, Tkv, H, D)), ("v0", v0, (B, Tkv, H, D)),
                         ("out", out, (B, T, H, D))):
        _check_tensor(name, t, shp, prob.dtype, dev)
    _check_tensor("lse", lse, (B, H, T), torch.float32, dev)
    if N > 0:
        _check_tensor("kd", kd, (B, N, T, H, D), prob.dtype, dev)
        _check_tensor("vd", vd, (B, N, T, H, D), prob.dtype, dev)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k0), torch.empty_like(v0),
                 torch.empty(B, N, T, H, D, dtype=prob.dtype, device=dev),
                 torch.empty(B, N, T, H, D, dtype=prob.dtype, device=dev))
    dq, dk0, dv0, dkd, dvd = grads
    if workspace is None:
        workspace = torch.empty(max(prob.workspace_bytes(), 256), dtype=torch.uint8, device=dev)
    _check(_entry(prob, "bwd")(prob.ref(), _ptr(dout), _ptr(q), _ptr(k0), _ptr(v0),
                               _ptr(kd if N > 0 else None), _ptr(vd if N > 0 else None),
                               _ptr(out), _ptr(lse), _ptr(workspace), _ptr(dq), _ptr(dk0),
                               _ptr(dv0), _ptr(dkd if N > 0 else None),
                               _ptr(dvd if N > 0 else None), _stream()))
    return dq, dk0, dv0, dkd, dvd


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


class _CachedAttention(torch.autograd.Function):
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


def cached_attention(q: torch.Tensor, cache_k: Sequence[torch.Tensor], cache_v: Sequence[torch.Tensor],
                     scale: float, cu_seqlens=None, layout: str = "full", cp: int = 1, rank: int = 0,
                     k0: Optional[torch.Tensor] = None, v0: Optional[torch.Tensor] = None):
    """EAGLE-3 mixed attention with autograd, in the list form of the pages'
    cached_*_attention: cache_k / cache_v are lists of [B, T, H, D] (index 0 = the
    step-0 sequence, 1.. = TTT steps). For a ring share (contiguous / zig-zag),
    pass the full-sequence block-0 k0/v0 [B, T_kv, H, D] explicitly; cache_k[0] is
    then ignored. Returns out [B, T, H, D] in q's dtype."""
    B, T, H, D = q.shape
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
