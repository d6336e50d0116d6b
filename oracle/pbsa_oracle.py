"""Plain, slow, float64 CPU oracle for Persistent Block-Sparse Attention (PBSA).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg import this module.  It shares no code, table or helper with the
HIP library, and it imports nothing from that library's package.

What it follows.  No page prints code, pseudo-code or a worked example for PBSA; the
method is described in prose, and the oracle takes the plainest reading of it:

  [SF]  "Sparse Forcing: Native Trainable Sparse Attention for Real-time Autoregressive
        Diffusion Video Generation" (gist.science explainers, English/Chinese/Portuguese),
        section 2 "Methodology": B "Core Mechanism: Structured Memory Decomposition"
        (persistent memory P_t with sinks + local sliding window L_t), C "Persistent
        Block-Sparse Attention" (dense access to P_t, top-K routing inside L_t from
        compressed block representatives, Top-C update of P_t as the window slides),
        and the Chinese page's 2.2 (blockified compression, coarse scoring, the hybrid
        mask).
  [LF]  "Light Forcing: Accelerating Autoregressive Video Diffusion via Sparse Attention"
        (papernotes.org), "Key designs": chunk-aware growth (the per-chunk sparsity
        s_i = s_base - alpha_i * beta and its FLOPs identity) and hierarchical sparse
        attention (mean pooling at block and frame level, frame top-K united with forced
        frames, block top-K inside the chosen frames, and the block mask).

Readings taken where the pages leave a step open (each is restated at its function):
  * blocks tile each latent frame on its own; the last block of a frame may be short;
  * a representative is the arithmetic mean of its block's tokens (frame rep: mean of
    the frame's tokens, not the mean of block reps);
  * the coarse score is scale * <q_rep, k_rep>;
  * ordering for every top-k is (score descending, id ascending); lists are returned
    ascending;
  * top-K chooses among the window blocks only; P_t is attended whole; the current
    chunk's own blocks are always attended, with no causal mask inside the chunk (a
    variant routes among the non-sink persistent blocks and the window together, the
    sinks alone attended whole);
  * sink blocks are the first S blocks of frame 0, pinned in P_t from the first update;
  * the memory score of a history block is the sum over the chunk's query blocks of its
    coarse score (a column sum).  The pages fix that the blocks the chunk's queries score
    highest are promoted; the pins fix the orientation (an aggregate over the chunk's
    query blocks of each candidate's own column), the sign and strict monotonicity (a
    candidate scored at least as high by every query block, and higher by one, is never
    dropped while the other is kept).  Which strictly monotone aggregate (a sum rather
    than, say, a softmax mass) stays a reading.

Everything floating point is float64.  Inputs given as float32/bf16-valued arrays are
widened to float64 first.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------------------
# Blockified compression.  [SF] 2.C / Chinese 2.2: the latent is tiled into blocks, each
# summarised by one representative vector; [LF] HSA step (1): mean pooling at block and
# frame level.
# --------------------------------------------------------------------------------------


def blocks_per_frame(n: int, B: int) -> int:
    """Number of blocks a frame of n tokens splits into (last block may be short)."""
    return -(-n // B)


def frame_block_ranges(n: int, B: int):
    """Token ranges [a, b) of the blocks of one frame: block j is [B*j, min(B*(j+1), n))."""
    return [(B * j, min(B * (j + 1), n)) for j in range(blocks_per_frame(n, B))]


def block_token_range(g: int, n: int, B: int):
    """Token range [a, b) of global block g = f*nb + j inside a frame-major token array."""
    nb = blocks_per_frame(n, B)
    f, j = divmod(g, nb)
    a, b = frame_block_ranges(n, B)[j]
    return f * n + a, f * n + b


def mean_pool(x, n: int, B: int):
    """Block and frame representatives of a frame-major token array.

    x: [frames * n, d].  Returns (block_rep [frames*nb, d], frame_rep [frames, d]) as the
    plain arithmetic means of the tokens each covers ([LF] HSA (1), mean pooling).
    """
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    if T % n:
        raise ValueError("token count is not a whole number of frames")
    frames = T // n
    nb = blocks_per_frame(n, B)
    block_rep = np.zeros((frames * nb, d))
    frame_rep = np.zeros((frames, d))
    for f in range(frames):
        frame = x[f * n:(f + 1) * n]
        frame_rep[f] = frame.sum(axis=0) / n
        for j, (a, b) in enumerate(frame_block_ranges(n, B)):
            block_rep[f * nb + j] = frame[a:b].sum(axis=0) / (b - a)
    return block_rep, frame_rep


# --------------------------------------------------------------------------------------
# Coarse scoring and routing.  [SF] 2.C: block-level scores from the compressed
# representatives; top-K blocks of the window kept per query block.
# --------------------------------------------------------------------------------------


def coarse_scores(q_rep, k_rep, scale: float):
    """S[r, j] = scale * <q_rep[r], k_rep[j]> (block-level attention logits)."""
    q_rep = np.asarray(q_rep, dtype=np.float64)
    k_rep = np.asarray(k_rep, dtype=np.float64)
    return scale * (q_rep @ k_rep.T)


def top_ids(values, ids, k: int):
    """The first k of `ids` ordered by (value descending, id ascending), returned ascending.

    Ties go to the lower id.  If k >= len(ids) every id is kept.
    """
    values = np.asarray(values, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    if values.shape != ids.shape:
        raise ValueError("values and ids differ in length")
    if k <= 0 or ids.size == 0:
        return []
    # np.lexsort sorts by its last key first: primary = -value, secondary = id.
    order = np.lexsort((ids, -values))
    return sorted(int(g) for g in ids[order[:k]])


# --------------------------------------------------------------------------------------
# Attention.  [SF] 2.C / Chinese 2.2 "fine-grained attention" and "mask mechanism": each
# query attends to every persistent block plus its selected window blocks; with a fixed
# selection that is ordinary softmax attention restricted by a block mask.
# --------------------------------------------------------------------------------------


def masked_attention(q, k, v, mask, scale: float):
    """Dense softmax attention with an explicit boolean mask [Tq, Tk].

    O[t] = sum_s softmax_s(scale * q_t . k_s over allowed s) v_s, LSE[t] = log sum_s exp(.)
    (natural log).  A row with no allowed key is an error.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    if not mask.any(axis=1).all():
        raise ValueError("a query row has no allowed key")
    s = np.where(mask, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s - m), 0.0)
    l = e.sum(axis=1, keepdims=True)
    o = (e / l) @ v
    lse = (m + np.log(l))[:, 0]
    return o, lse


def masked_attention_grad(q, k, v, mask, scale: float, dout):
    """Closed-form gradient of masked_attention's O with respect to q, k and v.

    With P = softmax rows (zero where masked): dV = P^T dO; dP = dO V^T;
    D = rowsum(dO * O); dS = P * (dP - D); dQ = scale dS K; dK = scale dS^T Q.
    The mask (the block selection) is held constant: no gradient flows through routing.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    s = np.where(mask, scale * (q @ k.T), -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s - m), 0.0)
    p = e / e.sum(axis=1, keepdims=True)
    o = p @ v
    dv = p.T @ dout
    dp = dout @ v.T
    D = (dout * o).sum(axis=1, keepdims=True)
    ds = p * (dp - D)
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def block_mask(q_blocks, kv_blocks_per_query_block, n: int, B: int, q_tokens: int,
               kv_tokens: int, q_block_ids=None):
    """Expand per-query-block allowed KV block lists into a token mask [q_tokens, kv_tokens].

    q_blocks: the query blocks, as global ids in the query token array's own tiling.
    kv_blocks_per_query_block[i]: allowed KV global block ids for q_blocks[i].
    """
    mask = np.zeros((q_tokens, kv_tokens), dtype=bool)
    for r, allowed in zip(q_blocks, kv_blocks_per_query_block):
        a, b = block_token_range(r, n, B)
        for g in allowed:
            ka, kb = block_token_range(g, n, B)
            mask[a:b, ka:kb] = True
    return mask


# --------------------------------------------------------------------------------------
# Persistent memory and sliding window bookkeeping.  [SF] 2.B (P_t bounded, sinks always
# kept, L_t = recent blocks) and 2.C "dynamic update" (window slides, leaving blocks are
# scored, the best are promoted, the rest dropped).
# --------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Schedule:
    """Shapes of one persistent-mode rollout (per head)."""
    n: int          # tokens per latent frame
    B: int          # tokens per block
    F: int          # frames per generated chunk
    W: int          # window length in history frames
    C: int          # persistent capacity in blocks (sinks included)
    S: int          # sink blocks: global ids 0..S-1 (frame 0)
    K: int          # top-K window blocks per query block
    scale: float
    # routing variant: False = top-K among the window blocks, every persistent block
    # attended; True = top-K among the non-sink persistent blocks and the window blocks
    # together, only the sinks attended whole
    union: bool = False

    @property
    def nb(self) -> int:
        return blocks_per_frame(self.n, self.B)

    def window_frames(self, c: int):
        """History frames inside the window while chunk c (0-based) is generated."""
        h = c * self.F
        return list(range(max(0, h - self.W), h))

    def window_blocks(self, c: int):
        """L_t: blocks of the window frames, sinks excluded (they live in P_t)."""
        return [f * self.nb + j for f in self.window_frames(c) for j in range(self.nb)
                if f * self.nb + j >= self.S]

    def evicted_blocks(self, c: int):
        """Window blocks that leave the window when chunk c's frames are appended."""
        h = c * self.F
        lo, hi = max(0, h - self.W), max(0, h + self.F - self.W)
        return [f * self.nb + j for f in range(lo, hi) for j in range(self.nb)
                if f * self.nb + j >= self.S]

    def chunk_blocks(self, c: int):
        """Global ids of chunk c's own blocks."""
        return list(range(c * self.F * self.nb, (c + 1) * self.F * self.nb))


def route(scores_window, window_ids, K: int):
    """Per query block, the top-K window blocks by (score desc, id asc), ascending."""
    return [top_ids(row, window_ids, K) for row in np.asarray(scores_window)]


def memory_scores(P, sinks, scores_P, evicted_ids, scores_E):
    """Candidates of the Top-C update and their memory scores.

    Candidates R = (P without sinks) + evicted (in that order); the memory score of a
    candidate is the sum over the chunk's query blocks of its coarse score (a column sum
    of the block-score matrix).  Returns (ids, scores).
    """
    sinks = set(sinks)
    P = list(P)
    scores_P = np.asarray(scores_P, dtype=np.float64)
    scores_E = np.asarray(scores_E, dtype=np.float64)
    if scores_P.shape[-1:] != (len(P),) or scores_E.shape[-1:] != (len(evicted_ids),):
        raise ValueError("score columns do not match the candidate ids")
    cand, msum = [], []
    for i, g in enumerate(P):
        if g not in sinks:
            cand.append(g)
            msum.append(scores_P[:, i].sum())
    for i, g in enumerate(evicted_ids):
        cand.append(g)
        msum.append(scores_E[:, i].sum())
    return cand, msum


def memory_update(P, sinks, scores_P, evicted_ids, scores_E, C: int):
    """Top-C retention of the persistent memory.

    P: current persistent ids (sinks included); scores_P[r, i]: coarse score of P[i] for
    query block r; evicted_ids / scores_E likewise for the blocks leaving the window.
    P' = sinks + the first (C - |sinks|) candidates (see memory_scores) by (memory score
    desc, id asc).  Unkept evicted blocks are dropped.
    """
    sinks = sorted(set(sinks))
    cand, msum = memory_scores(P, sinks, scores_P, evicted_ids, scores_E)
    keep = top_ids(msum, cand, C - len(sinks))
    return sorted(sinks + keep)


# --------------------------------------------------------------------------------------
# FP8 KV cache.  Light Forcing ("Key findings"): FP8 deployment of the sparse attention.
# Reading: each stored block's K and V are kept in the OCP float8 E4M3 format (1 sign bit,
# 4 exponent bits with bias 7, 3 mantissa bits; no infinities; largest finite value 448)
# with one power-of-two scale per block and tensor, the smallest 2^e with amax <= 448 * 2^e
# (amax = the largest |value| of the block's valid tokens; 1 for an all-zero block), and
# round-to-nearest-even.  Attention then runs on the decoded values code * scale, which
# are exact in bf16 (four significant bits times a power of two).
# --------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(code):
    """Value of E4M3 codes (uint8 array): normal (-1)^s 2^(e-7) (1 + m/8), subnormal
    (-1)^s 2^-6 m/8; exponent 15 with mantissa 7 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    sgn = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sgn * val


def e4m3_encode(y):
    """Nearest E4M3 code to each value of y (|y| <= 448), ties to the even mantissa."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(y) > E4M3_MAX) or np.any(~np.isfinite(y)):
        raise ValueError("value outside the E4M3 range")
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y)
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: a multiple of 2^-9, rounded to nearest even (np.rint), 8 -> 2^-6
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        e = np.floor(np.log2(a[nrm])).astype(np.int64)
        # guard the logarithm's rounding: a = f * 2^e with f in [1, 2)
        e = np.where(a[nrm] < 2.0 ** e, e - 1, e)
        e = np.where(a[nrm] >= 2.0 ** (e + 1), e + 1, e)
        f = a[nrm] / 2.0 ** e
        m = np.rint((f - 1.0) * 8.0).astype(np.int64)
        carry = m == 8
        m = np.where(carry, 0, m)
        e = np.where(carry, e + 1, e)
        out[nrm] = ((e + 7) << 3) | m
    return (out | sign).astype(np.uint8)


def e4m3_block_scale(x):
    """Power-of-two scale of a block: the smallest 2^e with max|x| <= 448 * 2^e (1 when the
    block is all zero)."""
    amax = float(np.max(np.abs(np.asarray(x, dtype=np.float64)))) if np.size(x) else 0.0
    if amax == 0.0:
        return 1.0
    e = math.ceil(math.log2(amax / E4M3_MAX))
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return 2.0 ** e


def e4m3_quantize_block(x):
    """(codes, scale) of one block [len, d]."""
    sc = e4m3_block_scale(x)
    return e4m3_encode(np.asarray(x, dtype=np.float64) / sc), sc


# --------------------------------------------------------------------------------------
# FP8 arithmetic.  [LF] "Key findings": the sparse attention deployed in FP8.  Reading: the
# queries, times the softmax scale in exp2 units, are rounded to E4M3 row by row (each row
# with its own power-of-two scale, the rule of a cache block), the chunk's own K/V block by
# block as the cache stores them, and the attention of those values is exact; the
# probabilities are rounded to E4M3 before their product with V, on a grid that an
# implementation's running offset decides, so the reference bounds that rounding instead of
# reproducing it.
# --------------------------------------------------------------------------------------


def e4m3_rows(x):
    """Each row of x [T, d] rounded to E4M3 with its own scale (e4m3_block_scale of the row),
    as decoded values; a row whose scale would fall below 2^-127 (E8M0's smallest, i.e.
    max|x| < 448 * 2^-128) takes 2^-127."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for t in range(x.shape[0]):
        sc = max(e4m3_block_scale(x[t]), 2.0 ** -127)
        out[t] = e4m3_decode(e4m3_encode(x[t] / sc)) * sc
    return out


def fp8_attention(q, K, V, scale: float, head: int = 3):
    """FP8-arithmetic attention of query rows q over keys K, V (already the decoded E4M3
    values): (O, LSE, bound).

    The queries enter as x = c q with c = scale * log2(e), the product and c itself rounded
    to float32 (the scores then come out in exp2 units), and x is rounded to E4M3 row by row
    (e4m3_rows).  O, LSE: the exact attention of those values, softmax in base 2 over
    t = x8 . k (LSE in natural log).
    bound[t, c]: how far rounding the probabilities to E4M3 can move O[t, c] when the
    implementation keeps its row offset so that the row max maps to p >= 2^head (and every
    p <= 448) in its units: a p in E4M3's normal range moves by at most 2^-4 p; one in the
    subnormal range (below 2^-6 in those units, so below 2^(-6-head) pmax in the normalised
    p) by at most min(p, 2^-10 in those units, at most 2^(-10-head) pmax):
        bound = 2^-4 sum_j p_j |V_jc|
                + sum_{p_j < 2^(-6-head) pmax} min(p_j, 2^(-10-head) pmax) |V_jc|
    with p the exact normalised probabilities and pmax their row max.
    """
    c = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    x = (np.asarray(q, dtype=np.float32) * c).astype(np.float64)
    x8 = e4m3_rows(x)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    t = x8 @ K.T
    tm = t.max(axis=1, keepdims=True)
    e = np.exp2(t - tm)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ V
    lse = (np.log(2.0) * (tm + np.log2(l)))[:, 0]
    pmax = p.max(axis=1, keepdims=True)
    aV = np.abs(V)
    sub = np.where(p < 2.0 ** (-6 - head) * pmax, np.minimum(p, 2.0 ** (-10 - head) * pmax), 0.0)
    bound = 2.0 ** -4 * (p @ aV) + sub @ aV
    return o, lse, bound


@dataclass
class PersistentRollout:
    """Oracle state of one head's rollout: P_t plus the tokens of the blocks it can still use.

    Tokens of a block are kept while the block is in the window or in P_t and discarded
    once it is dropped (the pages' "discarded" history); with keep_history=True every
    generated token is also kept, for the dense-mask parity form.  Stored tokens keep the
    caller's dtype and are widened to float64 when used.
    """
    sch: Schedule
    d: int
    keep_history: bool = False
    # stored blocks keep their K and V as E4M3 codes with a power-of-two scale per block
    # (tok_k / tok_v then hold the decoded values; codes and scales in fp8_codes)
    kv_fp8: bool = False
    chunk: int = 0
    P: list = field(default_factory=list)
    tok_k: dict = field(default_factory=dict)   # global block id -> [len, d]
    tok_v: dict = field(default_factory=dict)
    krep: dict = field(default_factory=dict)    # global block id -> [d] float64
    hist_k: list = field(default_factory=list)  # keep_history: per chunk [F*n, d]
    hist_v: list = field(default_factory=list)
    fp8_codes: dict = field(default_factory=dict)  # kv_fp8: block -> (k codes, k scale, v codes, v scale)

    def _reps(self, ids):
        return np.array([self.krep[g] for g in ids]).reshape(len(ids), self.d)

    def select(self, q_chunk):
        """Pool the chunk's queries, score P_t and L_t, route.

        Returns dict(q_rep, P, L, scores_P [Nq, |P|], scores_L [Nq, |L|], cand,
        scores_cand, sel): cand are the blocks the top-K chooses from (L_t; with
        sch.union the non-sink blocks of P_t followed by L_t) and scores_cand their
        columns.
        """
        s = self.sch
        q_rep, _ = mean_pool(q_chunk, s.n, s.B)
        L = s.window_blocks(self.chunk)
        P = list(self.P)
        scores_P = coarse_scores(q_rep, self._reps(P), s.scale) if P else np.zeros((len(q_rep), 0))
        scores_L = coarse_scores(q_rep, self._reps(L), s.scale) if L else np.zeros((len(q_rep), 0))
        if s.union:
            keep = [i for i, g in enumerate(P) if g >= s.S]
            cand = [P[i] for i in keep] + L
            scores_cand = np.concatenate([scores_P[:, keep], scores_L], axis=1)
        else:
            cand, scores_cand = L, scores_L
        sel = route(scores_cand, cand, s.K)
        return dict(q_rep=q_rep, P=P, L=L, scores_P=scores_P, scores_L=scores_L, cand=cand,
                    scores_cand=scores_cand, sel=sel)

    def attended_blocks(self, sel):
        """A_r = P_t + sel[r] + the chunk's own blocks, as global block ids (with sch.union
        only the sinks of P_t are attended whole: A_r = sinks + sel[r] + the chunk)."""
        own = self.sch.chunk_blocks(self.chunk)
        whole = [g for g in self.P if g < self.sch.S] if self.sch.union else self.P
        return [sorted(set(whole) | set(row) | set(own)) for row in sel]

    def attend(self, q_chunk, k_chunk, v_chunk, sel, rows=None):
        """Gathered form: per query block, softmax attention over the tokens of A_r.

        rows: optional iterable of query-token indices (chunk-local) to compute; others
        are left as NaN.  Returns (O [F*n, d], LSE [F*n]).
        """
        s = self.sch
        q = np.asarray(q_chunk)
        base = self.chunk * s.F * s.nb
        own_k, own_v = {}, {}
        for b in range(s.F * s.nb):
            a0, b0 = block_token_range(b, s.n, s.B)
            own_k[base + b], own_v[base + b] = k_chunk[a0:b0], v_chunk[a0:b0]
        Tq = q.shape[0]
        o = np.full((Tq, self.d), np.nan)
        lse = np.full(Tq, np.nan)
        want = None if rows is None else set(int(t) for t in rows)
        for r, allowed in enumerate(self.attended_blocks(sel)):
            a, b = block_token_range(r, s.n, s.B)
            idx = [t for t in range(a, b) if want is None or t in want]
            if not idx:
                continue
            K = np.concatenate([np.asarray(own_k[g] if g in own_k else self.tok_k[g], np.float64)
                                for g in allowed])
            V = np.concatenate([np.asarray(own_v[g] if g in own_v else self.tok_v[g], np.float64)
                                for g in allowed])
            mask = np.ones((len(idx), K.shape[0]), dtype=bool)
            oo, ll = masked_attention(np.asarray(q[idx], np.float64), K, V, mask, s.scale)
            o[idx], lse[idx] = oo, ll
        return o, lse

    def attend_fp8(self, q_chunk, k_chunk, v_chunk, sel, rows=None):
        """attend in FP8 arithmetic over an FP8 cache (kv_fp8): the stored blocks as their
        decoded codes, the chunk's own blocks quantized per block and tensor like a cache
        slot, the queries (times scale * log2 e) per row (fp8_attention).  Returns (O, LSE,
        bound) with rows not asked for left as NaN."""
        if not self.kv_fp8:
            raise ValueError("FP8 arithmetic reads an FP8 cache")
        s = self.sch
        q = np.asarray(q_chunk)
        base = self.chunk * s.F * s.nb
        own_k, own_v = {}, {}
        for b in range(s.F * s.nb):
            a0, b0 = block_token_range(b, s.n, s.B)
            kc, ks = e4m3_quantize_block(k_chunk[a0:b0])
            vc, vs = e4m3_quantize_block(v_chunk[a0:b0])
            own_k[base + b], own_v[base + b] = e4m3_decode(kc) * ks, e4m3_decode(vc) * vs
        Tq = q.shape[0]
        o = np.full((Tq, self.d), np.nan)
        lse = np.full(Tq, np.nan)
        bnd = np.full((Tq, self.d), np.nan)
        want = None if rows is None else set(int(t) for t in rows)
        for r, allowed in enumerate(self.attended_blocks(sel)):
            a, b = block_token_range(r, s.n, s.B)
            idx = [t for t in range(a, b) if want is None or t in want]
            if not idx:
                continue
            K = np.concatenate([own_k[g] if g in own_k else np.asarray(self.tok_k[g], np.float64)
                                for g in allowed])
            V = np.concatenate([own_v[g] if g in own_v else np.asarray(self.tok_v[g], np.float64)
                                for g in allowed])
            o[idx], lse[idx], bnd[idx] = fp8_attention(np.asarray(q[idx], np.float64), K, V,
                                                       s.scale)
        return o, lse, bnd

    def attend_grad(self, q_chunk, k_chunk, v_chunk, sel, dout):
        """Gradient of attend's output O (dout = dL/dO) with the selection held constant
        ([SF] 2.D: training runs the same sparse cache as inference).

        The keys are every block whose tokens are stored (P_t and the window) followed by
        the chunk; each query block's allowed keys are those of attend; masked_attention_grad
        gives the gradients.  Returns (dq [F*n, d], dk_chunk, dv_chunk [F*n, d],
        dk_blocks, dv_blocks) where dk_blocks[g] / dv_blocks[g] are [len(g), d] for every
        stored block g (zero for a block no query attends)."""
        s = self.sch
        stored = sorted(set(self.P) | set(s.window_blocks(self.chunk)))
        Ks = [np.asarray(self.tok_k[g], np.float64) for g in stored] + [np.asarray(k_chunk, np.float64)]
        Vs = [np.asarray(self.tok_v[g], np.float64) for g in stored] + [np.asarray(v_chunk, np.float64)]
        K, V = np.concatenate(Ks), np.concatenate(Vs)
        off, o = {}, 0
        for g, kk in zip(stored, Ks):
            off[g] = (o, o + kk.shape[0])
            o += kk.shape[0]
        base = self.chunk * s.F * s.nb
        for b in range(s.F * s.nb):
            a0, b0 = block_token_range(b, s.n, s.B)
            off[base + b] = (o + a0, o + b0)
        q = np.asarray(q_chunk, np.float64)
        mask = np.zeros((q.shape[0], K.shape[0]), dtype=bool)
        for r, allowed in enumerate(self.attended_blocks(sel)):
            a, b = block_token_range(r, s.n, s.B)
            for g in allowed:
                ka, kb = off[g]
                mask[a:b, ka:kb] = True
        dq, dk, dv = masked_attention_grad(q, K, V, mask, s.scale, dout)
        dk_blocks = {g: dk[off[g][0]:off[g][1]] for g in stored}
        dv_blocks = {g: dv[off[g][0]:off[g][1]] for g in stored}
        return dq, dk[o:], dv[o:], dk_blocks, dv_blocks

    def attend_dense(self, q_chunk, k_chunk, v_chunk, sel):
        """Parity form: dense attention over the whole history + chunk with the block mask
        (needs keep_history=True)."""
        if not self.keep_history:
            raise ValueError("the dense form needs keep_history=True")
        s = self.sch
        K_all = np.concatenate([np.asarray(x, np.float64) for x in self.hist_k + [k_chunk]])
        V_all = np.concatenate([np.asarray(x, np.float64) for x in self.hist_v + [v_chunk]])
        q = np.asarray(q_chunk, np.float64)
        base = self.chunk * s.F * s.nb
        allowed = self.attended_blocks(sel)
        # query block r of the chunk is global block base + r of the full token array
        mask_full = block_mask([base + r for r in range(len(allowed))], allowed, s.n, s.B,
                               K_all.shape[0], K_all.shape[0])
        q0 = self.chunk * s.F * s.n
        mask = mask_full[q0:q0 + q.shape[0]]
        return masked_attention(q, K_all, V_all, mask, s.scale)

    def update_candidates(self, routed):
        """(candidate ids, memory scores) the Top-C update of this chunk ranks."""
        s = self.sch
        E = s.evicted_blocks(self.chunk)
        col = {g: i for i, g in enumerate(routed["L"])}
        scores_E = routed["scores_L"][:, [col[g] for g in E]] if E else \
            np.zeros((routed["scores_L"].shape[0], 0))
        return memory_scores(routed["P"], list(range(s.S)), routed["scores_P"], E, scores_E)

    def update(self, routed, k_chunk, v_chunk, P_override=None):
        """Top-C memory update, then append the chunk (advances the chunk index).

        P_override: a persistent set chosen elsewhere among equally valid ones (when memory
        scores tie within rounding); it must be the sinks plus candidates of this update.
        """
        s = self.sch
        sinks = list(range(s.S))
        cand, msum = self.update_candidates(routed)
        if P_override is None:
            self.P = sorted(sinks + top_ids(msum, cand, s.C - s.S))
        else:
            if not set(P_override) <= set(sinks) | set(cand) or len(P_override) > s.C:
                raise ValueError("override is not sinks plus candidates")
            self.P = sorted(int(g) for g in P_override)
        base = self.chunk * s.F * s.nb
        krep, _ = mean_pool(k_chunk, s.n, s.B)
        for b in range(s.F * s.nb):
            a0, b0 = block_token_range(b, s.n, s.B)
            self.tok_k[base + b] = k_chunk[a0:b0]
            self.tok_v[base + b] = v_chunk[a0:b0]
            self.krep[base + b] = krep[b]
            if self.kv_fp8:
                kc, ks = e4m3_quantize_block(k_chunk[a0:b0])
                vc, vs = e4m3_quantize_block(v_chunk[a0:b0])
                self.fp8_codes[base + b] = (kc, ks, vc, vs)
                self.tok_k[base + b] = e4m3_decode(kc) * ks
                self.tok_v[base + b] = e4m3_decode(vc) * vs
        if self.keep_history:
            self.hist_k.append(k_chunk)
            self.hist_v.append(v_chunk)
        self.chunk += 1
        live = set(self.P) | set(s.window_blocks(self.chunk))
        for g in [g for g in self.tok_k if g not in live]:
            del self.tok_k[g], self.tok_v[g], self.krep[g]
            self.fp8_codes.pop(g, None)


# --------------------------------------------------------------------------------------
# Trainable two-level path.  [LF] HSA: frame-level top-K of pooled frame representatives
# united with forced frames, then block-level top-K among the blocks of those frames; the
# block mask is 1 exactly on the chosen (frame, block) pairs.  [LF] CAG: per-chunk budget.
# --------------------------------------------------------------------------------------


def two_level_frames(q_rep_row, k_frame_rep, i: int, F: int, top_frames: int, scale: float):
    """Frame stage for a query block of chunk i >= 2 (1-based): (history frames, their
    scores, the chosen frame set T).  p(f) = scale <q_rep, k_frame_rep[f]> over history
    frames f < F(i-1); T = the top_frames best (ties to the lower frame) united with the
    forced frames {0, F(i-1)-1} and the chunk's own F frames."""
    hist = list(range(F * (i - 1)))
    p = coarse_scores(q_rep_row[None, :], k_frame_rep[hist], scale)[0]
    T = set(top_ids(p, hist, top_frames))
    T |= {0, F * (i - 1) - 1}
    T |= {F * (i - 1) + t for t in range(F)}
    return hist, p, sorted(T)


def two_level_blocks(q_rep_row, k_block_rep, frames, nb: int, scale: float):
    """Block stage: every block of the given frames and its score scale <q_rep, k_rep>."""
    cand = [f * nb + j for f in sorted(frames) for j in range(nb)]
    o = coarse_scores(q_rep_row[None, :], k_block_rep[cand], scale)[0]
    return cand, o


def two_level_select(q_rep_row, k_block_rep, k_frame_rep, i: int, F: int, nb: int,
                     top_frames: int, k_i: int, scale: float):
    """Selected KV blocks (global ids, ascending) for one query block of chunk i (1-based).

    Chunk 1 attends densely to its own frames.  For i >= 2: the frames of
    two_level_frames, then the first min(k_i, candidates) of their blocks by (score desc,
    id asc).
    """
    if i == 1:
        return list(range(F * nb))
    _, _, T = two_level_frames(q_rep_row, k_frame_rep, i, F, top_frames, scale)
    cand, o = two_level_blocks(q_rep_row, k_block_rep, T, nb, scale)
    return top_ids(o, cand, min(k_i, len(cand)))


def cag_budgets(alphas, k_ref: int, i_ref: int):
    """Per-chunk block budgets k_i for chunks i = 1..len(alphas) ([LF] CAG).

    Each chunk i >= 2 keeps the fraction (1 - s_base + alpha_i * beta) of the N_i blocks it
    can see, where N_i grows linearly with i.  Reading: 1 - s_base and beta are both the
    fraction that makes chunk i_ref keep k_ref blocks at alpha = 0, so
    k_i = floor(k_ref * i * (1 + alpha_i) / i_ref + 1/2), at least 1.  Chunk 1 is dense
    (the identity's sum starts at i = 2) and is reported as 0 here.
    """
    out = []
    for i, a in enumerate(alphas, start=1):
        if i == 1:
            out.append(0)
            continue
        out.append(max(1, int(math.floor(k_ref * i * (1.0 + float(a)) / i_ref + 0.5))))
    return out


def cag_target_sparsity(alphas, s_base: float, beta: float, lq, lk):
    """s_target implied by the CAG FLOPs identity over chunks i = 2..n ([LF] CAG):

    sum_i (1 - s_base + alpha_i beta) lq_i lk_i d = (1 - s_target) sum_i lq_i lk_i d.
    (d cancels.)
    """
    num = sum((1.0 - s_base + a * beta) * q * k for a, q, k in
              zip(alphas[1:], lq[1:], lk[1:]))
    den = sum(q * k for q, k in zip(lq[1:], lk[1:]))
    return 1.0 - num / den
