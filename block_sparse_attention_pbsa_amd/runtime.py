"""Host-side driver of one layer's PBSA rollout: the per-chunk step as a sequence of
library calls on torch's current stream, with every buffer allocated once up front.

Per chunk (Sparse Forcing, gist.science, 2.C):
    route(q, cache) -> q_rep, scores, sel  (pool of q, scores, top-K in one launch);
    attn_fwd(q, cache, k, v, sel) -> o, lse;
    memory_update(scores, cache, k, v) (which pools k into the cache's representatives).
`step(..., overlap=True)` runs the memory update's selection (which only reads the cache
and the scores) on a second stream while the attention reads the cache, and its apply half
after both; on the GPU this hides the selection, but from Python the two extra stream
synchronisations cost about what it saves, so the default is the plain sequence.
With several denoising passes per chunk the persistent memory is shared: only the last
pass (the one whose K/V enter the cache) calls memory_update.
"""
from __future__ import annotations

import torch

from . import ops


class PersistentLayer:
    def __init__(self, shape: ops.Shape, device="cuda", passes: int = 1,
                 device_counter: bool = False, fp8_arithmetic: bool = False):
        self.shape = shape
        H, d, nq, T = shape.heads, shape.head_dim, shape.nq, shape.chunk_tokens
        # device_counter: the cache keeps a device copy of its chunk index (needed by the
        # captured chunk step, step_graph)
        self.cache = ops.Cache(shape, device, device_counter=device_counter)
        self._graphs = {}
        self.q_rep = torch.empty(H, nq, d, dtype=torch.float32, device=device)
        self.scores = torch.empty(H, nq, shape.slots, dtype=torch.float32, device=device)
        self.sel = torch.empty(H, nq, shape.topk, dtype=torch.int32, device=device)
        # one output per denoising pass of a chunk
        self.os = [torch.empty(T, H, d, dtype=torch.bfloat16, device=device)
                   for _ in range(passes)]
        self.lses = [torch.empty(H, T, dtype=torch.float32, device=device) for _ in range(passes)]
        self.o, self.lse = self.os[0], self.lses[0]
        nbytes = ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_MEMORY_UPDATE)
        self.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
        self.side = torch.cuda.Stream(device=device)  # default priority
        # fp8_arithmetic (FP8 cache only): the attention runs pbsa_attn_fwd_fp8, whose
        # workspace holds the chunk's quantized K/V
        self.fp8_arithmetic = fp8_arithmetic
        if fp8_arithmetic:
            nb8 = ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_FWD_FP8)
            if nb8 == 0:
                raise ValueError("FP8 arithmetic needs an FP8 cache (kv_format PBSA_KV_FP8)")
            self.workspace8 = torch.empty(nb8, dtype=torch.uint8, device=device)

    def reset(self):
        ops.pbsa_cache_reset(self.shape, self.cache)

    def route(self, q):
        ops.pbsa_route(self.shape, q, self.cache, self.q_rep, self.scores, self.sel)

    def attend(self, q, k, v, p: int = 0):
        if self.fp8_arithmetic:
            ops.pbsa_attn_fwd_fp8(self.shape, q, self.cache, k, v, self.sel, self.os[p],
                                  self.lses[p], self.workspace8)
            return
        ops.pbsa_attn_fwd(self.shape, q, self.cache, k, v, self.sel, self.os[p], self.lses[p])

    def update(self, k, v):
        s = self.shape
        ops.pbsa_memory_update(s, self.scores, self.cache, k, v, None, self.workspace)

    def step(self, q, k, v, attend=True, overlap=False):
        """One chunk: route, attend (optional), update the memory and append the chunk.
        overlap: the memory selection runs on the side stream beside the attention."""
        self.route(q)
        if not overlap:
            if attend:
                self.attend(q, k, v)
            self.update(k, v)
            return
        if not attend:
            self.update(k, v)
            return
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)            # the scores of this chunk are complete
        with torch.cuda.stream(self.side):
            ops.pbsa_memory_select(self.shape, self.scores, self.cache, self.workspace)
        self.attend(q, k, v)
        main.wait_stream(self.side)            # selection done; attention done (same stream)
        ops.pbsa_memory_apply(self.shape, self.cache, k, v, None, self.workspace)


    def step_passes(self, passes):
        """One chunk with len(passes) denoising passes sharing the memory: each pass
        (q, k, v) is routed and attended (outputs in os[p], lses[p]); then the memory is
        updated with the last pass's scores and its K/V enter the cache."""
        for p, (q, k, v) in enumerate(passes):
            self.route(q)
            self.attend(q, k, v, p)
        q, k, v = passes[-1]
        self.update(k, v)

    def _args(self, passes):
        return ops.chunk_args(self.shape, passes, self.q_rep, self.scores, self.sel, self.os,
                              self.lses, self.workspace,
                              self.workspace8 if self.fp8_arithmetic else None)

    def step_fused(self, passes):
        """step_passes as one library call (pbsa_chunk_step)."""
        ops.pbsa_chunk_step(self.shape, self._args(passes), self.cache)

    def step_graph(self, passes):
        """step_passes replayed from a HIP graph captured for these input tensors (one
        capture per distinct set of input buffers; later chunks reuse it when their inputs
        are written into the same buffers).  The selection of the memory update runs on a
        captured side branch beside the last pass's attention."""
        key = tuple(t.data_ptr() for qkv in passes for t in qkv)
        g = self._graphs.get(key)
        if g is None:
            g = ops.ChunkGraph(self.shape, self._args(passes), self.cache,
                               keep=[t for qkv in passes for t in qkv])
            self._graphs[key] = g
        g.launch(self.cache)

    def close_graphs(self):
        for g in self._graphs.values():
            g.close()
        self._graphs.clear()


class TwoLevelClip:
    """Buffers and calls of the trainable two-level path over one clip."""

    def __init__(self, shape: ops.Shape, chunks: int, top_frames: int, max_sel: int,
                 device="cuda"):
        self.shape, self.chunks, self.top_frames, self.max_sel = shape, chunks, top_frames, max_sel
        H, d = shape.heads, shape.head_dim
        nq = chunks * shape.nq
        T = chunks * shape.chunk_tokens
        self.q_rep = torch.empty(H, nq, d, dtype=torch.float32, device=device)
        self.k_rep = torch.empty(H, nq, d, dtype=torch.float32, device=device)
        self.k_frame = torch.empty(H, chunks * shape.chunk_frames, d, dtype=torch.float32,
                                   device=device)
        self.sel = torch.full((H, nq, max_sel), -1, dtype=torch.int32, device=device)
        self.nsel = torch.zeros(H, nq, dtype=torch.int32, device=device)
        self.o = torch.empty(T, H, d, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(H, T, dtype=torch.float32, device=device)
        self.dq = torch.empty(T, H, d, dtype=torch.bfloat16, device=device)
        self.dk = torch.empty_like(self.dq)
        self.dv = torch.empty_like(self.dq)
        nbytes = ops.pbsa_workspace_bytes(shape, ops.PBSA_OP_ATTN_BWD, chunks, max_sel)
        self.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)

    def select(self, q, k, k_per_chunk):
        s, F = self.shape, self.chunks * self.shape.chunk_frames
        ops.pbsa_pool(s, q, F, self.q_rep)
        ops.pbsa_pool(s, k, F, self.k_rep, self.k_frame)
        ops.pbsa_score_topk_2lvl(s, self.chunks, self.top_frames, k_per_chunk, self.q_rep,
                                 self.k_rep, self.k_frame, self.sel, self.nsel)

    def forward(self, q, k, v):
        ops.pbsa_attn_fwd_2lvl(self.shape, self.chunks, q, k, v, self.sel, self.nsel, self.o,
                               self.lse)

    def backward(self, q, k, v, dout):
        ops.pbsa_attn_bwd(self.shape, self.chunks, q, k, v, self.o, self.lse, dout, self.sel,
                          self.nsel, self.dq, self.dk, self.dv, self.workspace)


def cag_budgets(alphas, k_ref: int, i_ref: int):
    """Per-chunk block budgets of the trainable path (Light Forcing, chunk-aware growth):
    chunk i >= 2 keeps a fraction of the blocks it sees that grows with its noise level
    alpha_i; with the fraction chosen so chunk i_ref keeps k_ref blocks at alpha = 0,
    k_i = floor(k_ref * i * (1 + alpha_i) / i_ref + 1/2) (at least 1).  Chunk 1 is dense
    and gets 0 here (its entry is not read)."""
    import math
    out = [0]
    for i in range(2, len(alphas) + 1):
        out.append(max(1, int(math.floor(k_ref * i * (1.0 + float(alphas[i - 1])) / i_ref + 0.5))))
    return out
