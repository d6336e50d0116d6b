"""Python binding of libpbsa (ctypes): argument marshalling only.

Every function here checks dtypes, devices and shapes of torch tensors, then calls the C
entry point of the same name with raw device pointers and torch's current HIP stream.  All
arithmetic runs in the library's gfx950 kernels.  If libpbsa.so is missing the first call
raises; there is no fallback.

Token tensors are bf16 torch tensors of shape (tokens, heads, head_dim) whose last
dimension is contiguous; any other token/head strides are passed through (so an
(H, T, d) tensor can be handed over as ``x.permute(1, 0, 2)``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpbsa.so")
_lib = None

PBSA_OK = 0
PBSA_OP_MEMORY_UPDATE = 1
PBSA_OP_ATTN_BWD = 2
PBSA_OP_ATTN_BWD_PERSISTENT = 3
PBSA_OP_ATTN_FWD_FP8 = 4
PBSA_ROUTE_WINDOW = 0
PBSA_ROUTE_UNION = 1
PBSA_KV_BF16 = 0
PBSA_KV_FP8 = 1


class PbsaError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32), ("frame_tokens", ctypes.c_int32),
                ("chunk_frames", ctypes.c_int32), ("window_frames", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("sinks", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("route_mode", ctypes.c_int32), ("kv_format", ctypes.c_int32)]


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("token_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


class CacheC(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("rep", ctypes.c_void_p),
                ("block_id", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("chunk_index", ctypes.c_int64), ("chunk_index_dev", ctypes.c_void_p),
                ("kv_scale", ctypes.c_void_p)]


MAX_PASSES = 8


class ChunkArgs(ctypes.Structure):
    _fields_ = [("passes", ctypes.c_int32), ("q", Tensor * MAX_PASSES),
                ("k", Tensor * MAX_PASSES), ("v", Tensor * MAX_PASSES),
                ("o", Tensor * MAX_PASSES), ("lse", ctypes.c_void_p * MAX_PASSES),
                ("q_rep", ctypes.c_void_p), ("scores", ctypes.c_void_p), ("sel", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("fp8_arithmetic", ctypes.c_int32), ("attn_workspace", ctypes.c_void_p),
                ("attn_workspace_bytes", ctypes.c_size_t)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "pbsa_abi_version": ([], ctypes.c_int),
    "pbsa_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "pbsa_last_error": ([], ctypes.c_char_p),
    "pbsa_check_dims": ([ctypes.POINTER(Dims), _I32], ctypes.c_int),
    "pbsa_cache_slots": ([ctypes.POINTER(Dims)], ctypes.c_int64),
    "pbsa_cache_bytes": ([ctypes.POINTER(Dims)], ctypes.c_size_t),
    "pbsa_check_cache_table": ([ctypes.POINTER(Dims), _P, _P, ctypes.c_int64], ctypes.c_int),
    "pbsa_check_selection": ([ctypes.POINTER(Dims), _P, _P], ctypes.c_int),
    "pbsa_check_selection_2lvl": ([ctypes.POINTER(Dims), _I32, _P, _P, _I32], ctypes.c_int),
    "pbsa_workspace_bytes": ([ctypes.POINTER(Dims), _I32, _I32, _I32], ctypes.c_size_t),
    "pbsa_cache_reset": ([ctypes.POINTER(Dims), ctypes.POINTER(CacheC), _P], ctypes.c_int),
    "pbsa_pool": ([ctypes.POINTER(Dims), Tensor, _I32, _P, _P, _P], ctypes.c_int),
    "pbsa_score_topk": ([ctypes.POINTER(Dims), _P, ctypes.POINTER(CacheC), _P, _P, _P],
                        ctypes.c_int),
    "pbsa_route": ([ctypes.POINTER(Dims), Tensor, ctypes.POINTER(CacheC), _P, _P, _P, _P],
                   ctypes.c_int),
    "pbsa_attn_fwd": ([ctypes.POINTER(Dims), Tensor, ctypes.POINTER(CacheC), Tensor, Tensor, _P,
                       Tensor, _P, _P], ctypes.c_int),
    "pbsa_attn_fwd_fp8": ([ctypes.POINTER(Dims), Tensor, ctypes.POINTER(CacheC), Tensor, Tensor,
                           _P, Tensor, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "pbsa_memory_update": ([ctypes.POINTER(Dims), _P, ctypes.POINTER(CacheC), Tensor, Tensor, _P,
                            _P, ctypes.c_size_t, _P], ctypes.c_int),
    "pbsa_memory_select": ([ctypes.POINTER(Dims), _P, ctypes.POINTER(CacheC), _P, ctypes.c_size_t,
                            _P], ctypes.c_int),
    "pbsa_memory_apply": ([ctypes.POINTER(Dims), ctypes.POINTER(CacheC), Tensor, Tensor, _P, _P,
                           ctypes.c_size_t, _P], ctypes.c_int),
    "pbsa_memory_update_noalloc": ([ctypes.POINTER(Dims), _P, ctypes.POINTER(CacheC), Tensor,
                                    Tensor, _P, _P], ctypes.c_int),
    "pbsa_score_topk_2lvl": ([ctypes.POINTER(Dims), _I32, _I32, ctypes.POINTER(_I32), _P, _P, _P,
                              _I32, _P, _P, _P], ctypes.c_int),
    "pbsa_attn_fwd_2lvl": ([ctypes.POINTER(Dims), _I32, Tensor, Tensor, Tensor, _P, _P, _I32,
                            Tensor, _P, _P], ctypes.c_int),
    "pbsa_attn_bwd": ([ctypes.POINTER(Dims), _I32, Tensor, Tensor, Tensor, Tensor, _P, Tensor,
                       _P, _P, _I32, Tensor, Tensor, Tensor, _P, ctypes.c_size_t, _P],
                      ctypes.c_int),
    "pbsa_attn_bwd_persistent": ([ctypes.POINTER(Dims), Tensor, ctypes.POINTER(CacheC), Tensor,
                                  Tensor, _P, Tensor, _P, Tensor, Tensor, Tensor, Tensor, _P, _P,
                                  _P, ctypes.c_size_t, _P], ctypes.c_int),
    "pbsa_chunk_step": ([ctypes.POINTER(Dims), ctypes.POINTER(ChunkArgs), ctypes.POINTER(CacheC),
                         _P], ctypes.c_int),
    "pbsa_chunk_graph_create": ([ctypes.POINTER(Dims), ctypes.POINTER(ChunkArgs),
                                 ctypes.POINTER(CacheC), ctypes.POINTER(_P)], ctypes.c_int),
    "pbsa_chunk_graph_launch": ([_P, ctypes.POINTER(CacheC), _P], ctypes.c_int),
    "pbsa_chunk_graph_destroy": ([_P], None),
    # measurement probes (pbsa_probe.h)
    "pbsa_probe_mfma": ([ctypes.c_int64, _P, _P], ctypes.c_int),
    "pbsa_probe_mfma_flop": ([ctypes.c_int64], ctypes.c_int64),
    "pbsa_probe_fp8_decode": ([_P, _P, _P, _I32, _P], ctypes.c_int),
    "pbsa_probe_gather": ([ctypes.POINTER(Dims), Tensor, ctypes.POINTER(CacheC), Tensor, Tensor,
                           _P, _P], ctypes.c_int),
}


def lib():
    """Load libpbsa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_pbsa_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(fn, st):
    if st != PBSA_OK:
        raise PbsaError(fn, st, lib().pbsa_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, name, dtype):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _contig(t, name, dtype, shape):
    _dev(t, name, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _tok(t, name, tokens, heads, head_dim):
    _dev(t, name, torch.bfloat16)
    if t.dim() != 3 or tuple(t.shape) != (tokens, heads, head_dim):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                         f"{(tokens, heads, head_dim)} (tokens, heads, head_dim)")
    if t.stride(2) != 1:
        raise ValueError(f"{name}: the head_dim axis must be contiguous")
    return Tensor(t.data_ptr(), t.stride(0), t.stride(1))


@dataclass(frozen=True)
class Shape:
    """Shapes of one attention layer (mirrors pbsa_dims)."""
    heads: int
    head_dim: int
    frame_tokens: int
    chunk_frames: int
    window_frames: int = 1
    capacity: int = 0
    sinks: int = 0
    topk: int = 1
    scale: float | None = None
    block: int = 64
    route_mode: int = 0    # PBSA_ROUTE_WINDOW (0) or PBSA_ROUTE_UNION (1)
    kv_format: int = 0     # PBSA_KV_BF16 (0) or PBSA_KV_FP8 (1)

    @property
    def nb(self) -> int:
        return -(-self.frame_tokens // self.block)

    @property
    def nq(self) -> int:
        return self.chunk_frames * self.nb

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_frames * self.frame_tokens

    @property
    def slots(self) -> int:
        return self.capacity + self.window_frames * self.nb

    def c(self) -> Dims:
        s = self.scale if self.scale is not None else self.head_dim ** -0.5
        return Dims(self.heads, self.head_dim, self.block, self.frame_tokens, self.chunk_frames,
                    self.window_frames, self.capacity, self.sinks, self.topk, s, self.route_mode,
                    self.kv_format)


class Cache:
    """Device buffers of one layer's persistent-mode KV cache (see pbsa_cache in pbsa.h)."""

    def __init__(self, shape: Shape, device="cuda", device_counter: bool = False):
        H, S, d = shape.heads, shape.slots, shape.head_dim
        self.shape = shape
        kv_dtype = torch.uint8 if shape.kv_format == PBSA_KV_FP8 else torch.bfloat16
        self.k = torch.zeros(H, S, shape.block, d, dtype=kv_dtype, device=device)
        self.v = torch.zeros_like(self.k)
        # FP8 cache: K and V scale of every slot
        self.kv_scale = torch.ones(H, S, 2, dtype=torch.float32, device=device) \
            if shape.kv_format == PBSA_KV_FP8 else None
        self.rep = torch.zeros(H, S, d, dtype=torch.float32, device=device)
        self.block_id = torch.full((H, S), -1, dtype=torch.int32, device=device)
        self.len = torch.zeros(H, S, dtype=torch.int32, device=device)
        self.chunk_index = 0
        # device copy of chunk_index (needed by captured chunk steps), or None
        self.chunk_dev = torch.zeros(1, dtype=torch.int64, device=device) if device_counter \
            else None

    def c(self) -> CacheC:
        return CacheC(self.k.data_ptr(), self.v.data_ptr(), self.rep.data_ptr(),
                      self.block_id.data_ptr(), self.len.data_ptr(), self.chunk_index,
                      self.chunk_dev.data_ptr() if self.chunk_dev is not None else None,
                      self.kv_scale.data_ptr() if self.kv_scale is not None else None)

    def nbytes(self) -> int:
        ts = [self.k, self.v, self.rep, self.block_id, self.len]
        if self.kv_scale is not None:
            ts.append(self.kv_scale)
        return sum(t.numel() * t.element_size() for t in ts)


# ------------------------------------------------------------------------------ calls
def pbsa_cache_slots(shape: Shape) -> int:
    return int(lib().pbsa_cache_slots(ctypes.byref(shape.c())))


def pbsa_workspace_bytes(shape: Shape, op: int, arg: int = 0, arg2: int = 0) -> int:
    return int(lib().pbsa_workspace_bytes(ctypes.byref(shape.c()), op, arg, arg2))


def pbsa_cache_reset(shape: Shape, cache: Cache):
    cc = cache.c()
    _check("pbsa_cache_reset", lib().pbsa_cache_reset(ctypes.byref(shape.c()), ctypes.byref(cc),
                                                      _stream()))
    cache.chunk_index = cc.chunk_index


def pbsa_pool(shape: Shape, x, frames: int, block_rep, frame_rep=None):
    H, d, nb = shape.heads, shape.head_dim, shape.nb
    xt = _tok(x, "x", frames * shape.frame_tokens, H, d)
    _contig(block_rep, "block_rep", torch.float32, (H, frames * nb, d))
    if frame_rep is not None:
        _contig(frame_rep, "frame_rep", torch.float32, (H, frames, d))
    _check("pbsa_pool", lib().pbsa_pool(ctypes.byref(shape.c()), xt, frames, _ptr(block_rep),
                                        _ptr(frame_rep), _stream()))


def pbsa_score_topk(shape: Shape, q_rep, cache: Cache, scores, sel):
    H, d = shape.heads, shape.head_dim
    _contig(q_rep, "q_rep", torch.float32, (H, shape.nq, d))
    _contig(scores, "scores", torch.float32, (H, shape.nq, shape.slots))
    _contig(sel, "sel", torch.int32, (H, shape.nq, shape.topk))
    _check("pbsa_score_topk", lib().pbsa_score_topk(ctypes.byref(shape.c()), _ptr(q_rep),
                                                    ctypes.byref(cache.c()), _ptr(scores),
                                                    _ptr(sel), _stream()))


def pbsa_route(shape: Shape, q, cache: Cache, q_rep, scores, sel):
    """pbsa_pool of q and pbsa_score_topk in one launch; q_rep may be None."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    qt = _tok(q, "q", T, H, d)
    if q_rep is not None:
        _contig(q_rep, "q_rep", torch.float32, (H, shape.nq, d))
    _contig(scores, "scores", torch.float32, (H, shape.nq, shape.slots))
    _contig(sel, "sel", torch.int32, (H, shape.nq, shape.topk))
    _check("pbsa_route", lib().pbsa_route(ctypes.byref(shape.c()), qt, ctypes.byref(cache.c()),
                                          _ptr(q_rep), _ptr(scores), _ptr(sel), _stream()))


def pbsa_attn_fwd(shape: Shape, q, cache: Cache, chunk_k, chunk_v, sel, o, lse):
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    qt = _tok(q, "q", T, H, d)
    kt = _tok(chunk_k, "chunk_k", T, H, d)
    vt = _tok(chunk_v, "chunk_v", T, H, d)
    ot = _tok(o, "o", T, H, d)
    _contig(sel, "sel", torch.int32, (H, shape.nq, shape.topk))
    _contig(lse, "lse", torch.float32, (H, T))
    _check("pbsa_attn_fwd", lib().pbsa_attn_fwd(ctypes.byref(shape.c()), qt,
                                                ctypes.byref(cache.c()), kt, vt, _ptr(sel), ot,
                                                _ptr(lse), _stream()))


def pbsa_attn_fwd_fp8(shape: Shape, q, cache: Cache, chunk_k, chunk_v, sel, o, lse, workspace):
    """pbsa_attn_fwd over an FP8 cache in FP8 arithmetic (pbsa.h); workspace: uint8 device
    tensor of at least pbsa_workspace_bytes(shape, PBSA_OP_ATTN_FWD_FP8) bytes."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    qt = _tok(q, "q", T, H, d)
    kt = _tok(chunk_k, "chunk_k", T, H, d)
    vt = _tok(chunk_v, "chunk_v", T, H, d)
    ot = _tok(o, "o", T, H, d)
    _contig(sel, "sel", torch.int32, (H, shape.nq, shape.topk))
    _contig(lse, "lse", torch.float32, (H, T))
    _dev(workspace, "workspace", torch.uint8)
    _check("pbsa_attn_fwd_fp8", lib().pbsa_attn_fwd_fp8(
        ctypes.byref(shape.c()), qt, ctypes.byref(cache.c()), kt, vt, _ptr(sel), ot, _ptr(lse),
        _ptr(workspace), workspace.numel(), _stream()))


def pbsa_probe_gather(shape: Shape, q, cache: Cache, chunk_k, chunk_v, sel):
    """Measurement probe: the gathers of pbsa_attn_fwd without its math (pbsa_probe.h)."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    qt = _tok(q, "q", T, H, d)
    kt = _tok(chunk_k, "chunk_k", T, H, d)
    vt = _tok(chunk_v, "chunk_v", T, H, d)
    _contig(sel, "sel", torch.int32, (H, shape.nq, shape.topk))
    _check("pbsa_probe_gather", lib().pbsa_probe_gather(ctypes.byref(shape.c()), qt,
                                                        ctypes.byref(cache.c()), kt, vt,
                                                        _ptr(sel), _stream()))


def pbsa_probe_mfma(iters: int, out):
    """Measurement probe: independent bf16 MFMA chains on every SIMD; returns the FLOP."""
    _contig(out, "out", torch.float32, (131072,))
    _check("pbsa_probe_mfma", lib().pbsa_probe_mfma(int(iters), _ptr(out), _stream()))
    return int(lib().pbsa_probe_mfma_flop(int(iters)))


def pbsa_memory_update(shape: Shape, scores, cache: Cache, chunk_k, chunk_v, chunk_rep,
                       workspace):
    """chunk_rep=None: the chunk's block means are computed from chunk_k in the update."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    _contig(scores, "scores", torch.float32, (H, shape.nq, shape.slots))
    kt = _tok(chunk_k, "chunk_k", T, H, d)
    vt = _tok(chunk_v, "chunk_v", T, H, d)
    if chunk_rep is not None:
        _contig(chunk_rep, "chunk_rep", torch.float32, (H, shape.nq, d))
    _dev(workspace, "workspace", torch.uint8)
    cc = cache.c()
    _check("pbsa_memory_update", lib().pbsa_memory_update(
        ctypes.byref(shape.c()), _ptr(scores), ctypes.byref(cc), kt, vt, _ptr(chunk_rep),
        _ptr(workspace), workspace.numel(), _stream()))
    cache.chunk_index = cc.chunk_index


def pbsa_memory_update_noalloc(shape: Shape, scores, cache: Cache, chunk_k, chunk_v, chunk_rep):
    """pbsa_memory_update with the library-held workspace (no workspace argument)."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    _contig(scores, "scores", torch.float32, (H, shape.nq, shape.slots))
    kt = _tok(chunk_k, "chunk_k", T, H, d)
    vt = _tok(chunk_v, "chunk_v", T, H, d)
    if chunk_rep is not None:
        _contig(chunk_rep, "chunk_rep", torch.float32, (H, shape.nq, d))
    cc = cache.c()
    _check("pbsa_memory_update_noalloc", lib().pbsa_memory_update_noalloc(
        ctypes.byref(shape.c()), _ptr(scores), ctypes.byref(cc), kt, vt, _ptr(chunk_rep),
        _stream()))
    cache.chunk_index = cc.chunk_index


def pbsa_memory_select(shape: Shape, scores, cache: Cache, workspace):
    """First half of pbsa_memory_update: the selection into the workspace (reads the cache
    only; may run on another stream while the chunk's attention reads the cache)."""
    H = shape.heads
    _contig(scores, "scores", torch.float32, (H, shape.nq, shape.slots))
    _dev(workspace, "workspace", torch.uint8)
    cc = cache.c()
    _check("pbsa_memory_select", lib().pbsa_memory_select(
        ctypes.byref(shape.c()), _ptr(scores), ctypes.byref(cc), _ptr(workspace),
        workspace.numel(), _stream()))


def pbsa_memory_apply(shape: Shape, cache: Cache, chunk_k, chunk_v, chunk_rep, workspace):
    """Second half of pbsa_memory_update: writes the workspace's selection and the chunk into
    the cache and advances cache.chunk_index."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    kt = _tok(chunk_k, "chunk_k", T, H, d)
    vt = _tok(chunk_v, "chunk_v", T, H, d)
    if chunk_rep is not None:
        _contig(chunk_rep, "chunk_rep", torch.float32, (H, shape.nq, d))
    _dev(workspace, "workspace", torch.uint8)
    cc = cache.c()
    _check("pbsa_memory_apply", lib().pbsa_memory_apply(
        ctypes.byref(shape.c()), ctypes.byref(cc), kt, vt, _ptr(chunk_rep), _ptr(workspace),
        workspace.numel(), _stream()))
    cache.chunk_index = cc.chunk_index


def pbsa_score_topk_2lvl(shape: Shape, chunks: int, top_frames: int, k_per_chunk, q_rep,
                         block_rep, frame_rep, sel, nsel):
    H, d = shape.heads, shape.head_dim
    nq = chunks * shape.nq
    _contig(q_rep, "q_rep", torch.float32, (H, nq, d))
    _contig(block_rep, "block_rep", torch.float32, (H, nq, d))
    _contig(frame_rep, "frame_rep", torch.float32, (H, chunks * shape.chunk_frames, d))
    _dev(sel, "sel", torch.int32)
    if sel.dim() != 3 or tuple(sel.shape[:2]) != (H, nq) or not sel.is_contiguous():
        raise ValueError("sel must be a contiguous (heads, Nq, max_sel) int32 tensor")
    _contig(nsel, "nsel", torch.int32, (H, nq))
    ks = (ctypes.c_int32 * chunks)(*[int(k) for k in k_per_chunk])
    _check("pbsa_score_topk_2lvl", lib().pbsa_score_topk_2lvl(
        ctypes.byref(shape.c()), chunks, top_frames, ks, _ptr(q_rep), _ptr(block_rep),
        _ptr(frame_rep), sel.shape[2], _ptr(sel), _ptr(nsel), _stream()))


def pbsa_attn_fwd_2lvl(shape: Shape, chunks: int, q, k, v, sel, nsel, o, lse):
    H, d = shape.heads, shape.head_dim
    T = chunks * shape.chunk_tokens
    nq = chunks * shape.nq
    qt, kt, vt, ot = (_tok(t, nm, T, H, d) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o")))
    _dev(sel, "sel", torch.int32)
    _contig(nsel, "nsel", torch.int32, (H, nq))
    _contig(lse, "lse", torch.float32, (H, T))
    _check("pbsa_attn_fwd_2lvl", lib().pbsa_attn_fwd_2lvl(
        ctypes.byref(shape.c()), chunks, qt, kt, vt, _ptr(sel), _ptr(nsel), sel.shape[2], ot,
        _ptr(lse), _stream()))


def pbsa_attn_bwd(shape: Shape, chunks: int, q, k, v, o, lse, dout, sel, nsel, dq, dk, dv,
                  workspace):
    H, d = shape.heads, shape.head_dim
    T = chunks * shape.chunk_tokens
    nq = chunks * shape.nq
    ts = [_tok(t, nm, T, H, d) for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"),
                                              (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv"))]
    _contig(lse, "lse", torch.float32, (H, T))
    _dev(sel, "sel", torch.int32)
    _contig(nsel, "nsel", torch.int32, (H, nq))
    _dev(workspace, "workspace", torch.uint8)
    _check("pbsa_attn_bwd", lib().pbsa_attn_bwd(
        ctypes.byref(shape.c()), chunks, ts[0], ts[1], ts[2], ts[3], _ptr(lse), ts[4],
        _ptr(sel), _ptr(nsel), sel.shape[2], ts[5], ts[6], ts[7], _ptr(workspace),
        workspace.numel(), _stream()))


def chunk_args(shape: Shape, passes, q_rep, scores, sel, os_, lses, workspace,
               attn_workspace=None) -> ChunkArgs:
    """pbsa_chunk_args for `passes` = [(q, k, v), ...] (the last pass's K/V enter the cache),
    per-pass outputs os_[p], lses[p] and the shared routing / update buffers; with
    attn_workspace (uint8 device tensor) the attentions run in FP8 arithmetic."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    n = len(passes)
    if not 1 <= n <= MAX_PASSES or len(os_) < n or len(lses) < n:
        raise ValueError(f"need 1..{MAX_PASSES} passes with an output each")
    a = ChunkArgs()
    a.passes = n
    for p, (q, k, v) in enumerate(passes):
        a.q[p] = _tok(q, "q", T, H, d)
        a.k[p] = _tok(k, "k", T, H, d)
        a.v[p] = _tok(v, "v", T, H, d)
        a.o[p] = _tok(os_[p], "o", T, H, d)
        _contig(lses[p], "lse", torch.float32, (H, T))
        a.lse[p] = lses[p].data_ptr()
    if q_rep is not None:
        _contig(q_rep, "q_rep", torch.float32, (H, shape.nq, d))
    _contig(scores, "scores", torch.float32, (H, shape.nq, shape.slots))
    _contig(sel, "sel", torch.int32, (H, shape.nq, shape.topk))
    _dev(workspace, "workspace", torch.uint8)
    a.q_rep = q_rep.data_ptr() if q_rep is not None else None
    a.scores, a.sel = scores.data_ptr(), sel.data_ptr()
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    if attn_workspace is not None:
        _dev(attn_workspace, "attn_workspace", torch.uint8)
        a.fp8_arithmetic = 1
        a.attn_workspace = attn_workspace.data_ptr()
        a.attn_workspace_bytes = attn_workspace.numel()
    return a


def pbsa_chunk_step(shape: Shape, args: ChunkArgs, cache: Cache):
    """The chunk step (all passes, then the memory update) as one call."""
    cc = cache.c()
    _check("pbsa_chunk_step", lib().pbsa_chunk_step(ctypes.byref(shape.c()), ctypes.byref(args),
                                                    ctypes.byref(cc), _stream()))
    cache.chunk_index = cc.chunk_index


class ChunkGraph:
    """The chunk step captured once as a HIP graph (pbsa_chunk_graph_*).  The tensors
    behind `args` must stay alive as long as the graph: it keeps references to them."""

    def __init__(self, shape: Shape, args: ChunkArgs, cache: Cache, keep=()):
        if cache.chunk_dev is None:
            raise ValueError("the cache needs a device chunk counter (device_counter=True)")
        self._keep = tuple(keep)
        h = ctypes.c_void_p()
        _check("pbsa_chunk_graph_create", lib().pbsa_chunk_graph_create(
            ctypes.byref(shape.c()), ctypes.byref(args), ctypes.byref(cache.c()),
            ctypes.byref(h)))
        self._h = h

    def launch(self, cache: Cache):
        cc = cache.c()
        _check("pbsa_chunk_graph_launch", lib().pbsa_chunk_graph_launch(self._h, ctypes.byref(cc),
                                                                        _stream()))
        cache.chunk_index = cc.chunk_index

    def close(self):
        if self._h:
            lib().pbsa_chunk_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass


def pbsa_attn_bwd_persistent(shape: Shape, q, cache: Cache, chunk_k, chunk_v, sel, o, lse, dout,
                             dq, dk, dv, dk_cache, dv_cache, workspace):
    """Gradient of pbsa_attn_fwd: dq, the chunk's dk/dv, and every cache slot's dk/dv
    (dk_cache, dv_cache shaped like cache.k)."""
    H, d, T = shape.heads, shape.head_dim, shape.chunk_tokens
    ts = [_tok(t, nm, T, H, d) for t, nm in ((q, "q"), (chunk_k, "chunk_k"), (chunk_v, "chunk_v"),
                                              (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"),
                                              (dv, "dv"))]
    _contig(sel, "sel", torch.int32, (H, shape.nq, shape.topk))
    _contig(lse, "lse", torch.float32, (H, T))
    for t, nm in ((dk_cache, "dk_cache"), (dv_cache, "dv_cache")):
        _contig(t, nm, torch.bfloat16, tuple(cache.k.shape))
    _dev(workspace, "workspace", torch.uint8)
    _check("pbsa_attn_bwd_persistent", lib().pbsa_attn_bwd_persistent(
        ctypes.byref(shape.c()), ts[0], ctypes.byref(cache.c()), ts[1], ts[2], _ptr(sel), ts[3],
        _ptr(lse), ts[4], ts[5], ts[6], ts[7], _ptr(dk_cache), _ptr(dv_cache), _ptr(workspace),
        workspace.numel(), _stream()))


# ---- host-side checks (numpy int32 arrays; no device access)
def _np_i32(a, name, shape):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.int32)
    if tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {a.shape}, expected {tuple(shape)}")
    return a


def pbsa_cache_bytes(shape: Shape) -> int:
    return int(lib().pbsa_cache_bytes(ctypes.byref(shape.c())))


def pbsa_check_cache_table(shape: Shape, block_id, len_, chunk_index: int):
    """Raises PbsaError (status PBSA_ERR_INDEX) if the host table is not a valid cache table."""
    b = _np_i32(block_id, "block_id", (shape.heads, shape.slots))
    n = _np_i32(len_, "len", (shape.heads, shape.slots))
    _check("pbsa_check_cache_table", lib().pbsa_check_cache_table(
        ctypes.byref(shape.c()), b.ctypes.data, n.ctypes.data, int(chunk_index)))


def pbsa_check_selection(shape: Shape, block_id, sel):
    b = _np_i32(block_id, "block_id", (shape.heads, shape.slots))
    sl = _np_i32(sel, "sel", (shape.heads, shape.nq, shape.topk))
    _check("pbsa_check_selection", lib().pbsa_check_selection(ctypes.byref(shape.c()),
                                                              b.ctypes.data, sl.ctypes.data))


def pbsa_check_selection_2lvl(shape: Shape, chunks: int, sel, nsel):
    import numpy as np
    sl = np.ascontiguousarray(sel, dtype=np.int32)
    if sl.ndim != 3 or sl.shape[:2] != (shape.heads, chunks * shape.nq):
        raise ValueError("sel must be (heads, Nq, max_sel)")
    ns = _np_i32(nsel, "nsel", (shape.heads, chunks * shape.nq))
    _check("pbsa_check_selection_2lvl", lib().pbsa_check_selection_2lvl(
        ctypes.byref(shape.c()), chunks, sl.ctypes.data, ns.ctypes.data, sl.shape[2]))


def pbsa_probe_fp8_decode(codes, scales, out):
    """The FP8 attention's decode (pbsa_probe.h): codes uint8 [n], scales fp32 [n / 16],
    out int16 [n] (bf16 bits)."""
    _dev(codes, "codes", torch.uint8)
    _dev(scales, "scales", torch.float32)
    _dev(out, "out", torch.int16)
    n = codes.numel()
    if scales.numel() * 16 != n or out.numel() != n:
        raise ValueError("need n codes, n / 16 scales and n outputs")
    _check("pbsa_probe_fp8_decode", lib().pbsa_probe_fp8_decode(_ptr(codes), _ptr(scales),
                                                                _ptr(out), n, _stream()))
