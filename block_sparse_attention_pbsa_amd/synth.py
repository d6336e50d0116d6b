"""Seeded synthetic inputs and workload shapes for PBSA.

This module holds no step of the method: it only draws random tensors, rounds them to
bf16 and records the shapes of the workloads.  Both the HIP path's tests and the CPU
oracle's tests take their inputs from here.

Workloads (shapes of a Wan2.1-1.3B-like autoregressive video model, one attention layer):
  tiny      1 head, d=64, 256-token frames, 1-frame chunks, 4 history frames, window 2,
            capacity 4 (1 sink), top-4; fp32 N(0,1) rounded to bf16.
  wan_5s    12 heads, d=128, 1560-token frames (24 full 64-token blocks + a 24-token tail),
            3-frame chunks, 21 history frames, window 6, capacity 64, top-32.
  wan_20s   same shapes, 81 history frames, capacity 128, top-48, planted blocks re-drawn
            every 10 frames.
  wan_1min  same shapes, 240 history frames, capacity 256, top-64.
  wan_train the trainable path: a 24-frame clip of 3-frame chunks, two-level selection
            (8 frames by pooled frame representative, then blocks inside them) with a
            per-chunk budget drawn from alpha_i ~ U[0, 1].

Structure: K and V are N(0,1); on planted "salient" blocks they are shifted by 3 along a
per-head unit direction u_h, and every query token by 1 along u_h, so that the planted
blocks score high for every query block.  All draws are float32 and are then rounded
to bf16 (round to nearest even); the float32 arrays returned hold exactly those values.
Random streams are keyed by (seed, tag, index) so any chunk can be drawn on its own.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    head_dim: int
    block: int
    frame_tokens: int
    chunk_frames: int
    history_frames: int
    window_frames: int
    capacity: int
    sinks: int
    topk: int
    planted_per_segment: int = 0
    segment_frames: int = 0        # planted blocks re-drawn every this many frames
    q_align: float = 0.0           # query shift along u_h
    kv_shift: float = 0.0          # K/V shift along u_h on planted blocks
    # each planted segment draws its own direction u_{h,seg} (K/V of its planted blocks
    # and the queries of its frames shift along it), instead of one u_h per head
    direction_per_segment: bool = False
    # trainable two-level path
    clip_chunks: int = 0
    top_frames: int = 0

    @property
    def nb(self) -> int:
        return -(-self.frame_tokens // self.block)

    @property
    def scale(self) -> float:
        return float(self.head_dim) ** -0.5

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_frames * self.frame_tokens

    @property
    def measured_chunk(self) -> int:
        """Index of the chunk generated right after the history (history / chunk frames)."""
        return self.history_frames // self.chunk_frames

    @property
    def plant_frames(self) -> int:
        """Frames over which the planted blocks are laid out: the history, the measured
        chunk and EXTRA_CHUNKS chunks after it (the rollout continues past the measured
        chunk when successive chunks are timed)."""
        return self.history_frames + self.chunk_frames * (1 + EXTRA_CHUNKS)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 64, 256, 1, 4, 2, 4, 1, 4),
    "wan_5s": Workload("wan_5s", 12, 128, 64, 1560, 3, 21, 6, 64, 1, 32,
                       planted_per_segment=8, segment_frames=24, q_align=1.0, kv_shift=3.0),
    "wan_20s": Workload("wan_20s", 12, 128, 64, 1560, 3, 81, 6, 128, 1, 48,
                        planted_per_segment=8, segment_frames=10, q_align=1.0, kv_shift=3.0),
    "wan_1min": Workload("wan_1min", 12, 128, 64, 1560, 3, 240, 6, 256, 1, 64,
                         planted_per_segment=8, segment_frames=10, q_align=1.0,
                         kv_shift=3.0),
    "wan_train": Workload("wan_train", 12, 128, 64, 1560, 3, 21, 6, 64, 1, 32,
                          planted_per_segment=8, segment_frames=24, q_align=1.0,
                          kv_shift=3.0, clip_chunks=8, top_frames=8),
}

# chunks after the measured one that keep the same planted layout
EXTRA_CHUNKS = 128

SEEDS = {"tiny": 1001, "wan_5s": 1002, "wan_20s": 1003, "wan_1min": 1004, "wan_train": 1005}

_TAGS = {"u": 1, "plant": 2, "qkv": 3, "alpha": 4, "dout": 5, "pass": 6}


def rng(seed: int, tag: str, index: int = 0) -> np.random.Generator:
    """Independent PCG64 stream keyed by (seed, tag, index)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag],
                                                                       index])))


def _rne_high_half(x) -> np.ndarray:
    """uint32 words whose high half is x rounded to bf16 (nearest, ties to even) and whose
    low half is zero.  Finite inputs only (the sum cannot carry out of 32 bits for them)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u
    r &= np.uint32(0xFFFF0000)
    return r


def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the raw uint16 bits."""
    return (_rne_high_half(x) >> 16).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """The float32 value of raw bf16 bits."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x) -> np.ndarray:
    """float32 array holding x rounded to bf16."""
    return _rne_high_half(x).view(np.float32)


def directions(wl: Workload, seed: int, segment: int = 0) -> np.ndarray:
    """Per-head unit direction u_h [H, d] (float32); with direction_per_segment, the
    direction of planted segment `segment`."""
    idx = segment if wl.direction_per_segment else 0
    u = rng(seed, "u", idx).standard_normal((wl.heads, wl.head_dim))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    return u.astype(np.float32)


def planted_blocks(wl: Workload, seed: int, frames: int) -> np.ndarray:
    """Sorted global block ids of the planted salient blocks among `frames` frames.

    Each segment of `segment_frames` frames gets `planted_per_segment` distinct blocks,
    drawn uniformly among that segment's blocks, the sink blocks excluded.
    """
    if wl.planted_per_segment == 0 or frames == 0:
        return np.zeros(0, dtype=np.int64)
    out = []
    seg = wl.segment_frames
    for s0 in range(0, frames, seg):
        f1 = min(frames, s0 + seg)
        lo = max(s0 * wl.nb, wl.sinks)
        hi = f1 * wl.nb
        cnt = min(wl.planted_per_segment, hi - lo)
        pick = rng(seed, "plant", s0).choice(hi - lo, size=cnt, replace=False)
        out.extend(int(lo + p) for p in pick)
    return np.array(sorted(out), dtype=np.int64)


def _plant_mask_tokens(wl: Workload, planted: np.ndarray, f0: int, frames: int) -> np.ndarray:
    """Boolean [frames*n] marking tokens of planted blocks inside frames [f0, f0+frames)."""
    n, B, nb = wl.frame_tokens, wl.block, wl.nb
    m = np.zeros(frames * n, dtype=bool)
    for g in planted:
        f, j = divmod(int(g), nb)
        if f0 <= f < f0 + frames:
            a = (f - f0) * n + B * j
            m[a:(f - f0) * n + min(B * (j + 1), n)] = True
    return m


def chunk_qkv(wl: Workload, seed: int, c: int, total_frames: int | None = None):
    """Q, K, V of chunk c as float32 [F*n, H, d] arrays holding bf16 values.

    total_frames: frames over which planted blocks are laid out (default:
    wl.plant_frames).
    """
    return _draw_qkv(wl, seed, c, rng(seed, "qkv", c), total_frames)


def pass_qkv(wl: Workload, seed: int, c: int, p: int, passes: int, total_frames: int | None = None):
    """Q, K, V of denoising pass p (0-based, of `passes`) of chunk c.  The last pass is the
    chunk itself (chunk_qkv: the pass whose K/V enter the cache); earlier passes draw their
    own tokens with the same structure."""
    if p == passes - 1:
        return chunk_qkv(wl, seed, c, total_frames)
    return _draw_qkv(wl, seed, c, rng(seed, "pass", 64 * c + p), total_frames)


def _draw_qkv(wl: Workload, seed: int, c: int, g, total_frames):
    F, n, H, d = wl.chunk_frames, wl.frame_tokens, wl.heads, wl.head_dim
    q, k, v = (g.standard_normal((F * n, H, d), dtype=np.float32) for _ in range(3))
    if wl.planted_per_segment:
        tf = total_frames if total_frames is not None else wl.plant_frames
        pm = _plant_mask_tokens(wl, planted_blocks(wl, seed, tf), c * F, F)
        if not wl.direction_per_segment:
            u = directions(wl, seed)
            k[pm] += wl.kv_shift * u[None, :, :]
            v[pm] += wl.kv_shift * u[None, :, :]
            q += wl.q_align * u[None, :, :]
        else:
            for fl in range(F):
                u = directions(wl, seed, (c * F + fl) // wl.segment_frames)
                sl = slice(fl * n, (fl + 1) * n)
                m = pm[sl]
                k[sl][m] += wl.kv_shift * u[None, :, :]
                v[sl][m] += wl.kv_shift * u[None, :, :]
                q[sl] += wl.q_align * u[None, :, :]
    return round_bf16(q), round_bf16(k), round_bf16(v)


def clip_qkv(wl: Workload, seed: int):
    """Q, K, V of the whole training clip (clip_chunks chunks), float32 [T, H, d]."""
    parts = [chunk_qkv(wl, seed, c, total_frames=wl.clip_chunks * wl.chunk_frames)
             for c in range(wl.clip_chunks)]
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(3))


def clip_alphas(wl: Workload, seed: int) -> np.ndarray:
    """alpha_i ~ U[0, 1] per chunk of the training clip (float64)."""
    return rng(seed, "alpha").uniform(0.0, 1.0, size=wl.clip_chunks)


def clip_dout(wl: Workload, seed: int, tokens: int) -> np.ndarray:
    """Upstream gradient dO, float32 [T, H, d] holding bf16 values."""
    g = rng(seed, "dout")
    return round_bf16(g.standard_normal((tokens, wl.heads, wl.head_dim), dtype=np.float32))


def tiny_tokens(seed: int, shape) -> np.ndarray:
    """Raw float32 N(0,1) draws (not rounded), for checks that want unrounded values."""
    return rng(seed, "qkv", 10_000).standard_normal(shape, dtype=np.float32)
