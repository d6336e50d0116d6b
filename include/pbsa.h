/*
 * pbsa.h -- C ABI of libpbsa, Persistent Block-Sparse Attention (PBSA) for MI355X (gfx950).
 *
 * The method: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
 * Autoregressive Diffusion Video Generation" (gist.science explainer), section 2
 * "Methodology": B (the KV cache split into a bounded persistent memory P_t, sinks
 * included, plus a sliding local window L_t), C "Persistent Block-Sparse Attention" (block
 * representatives, coarse block scores, top-K routing inside L_t, dense access to P_t, a
 * Top-C update of P_t as the window slides), E (one kernel family for decoding and
 * training).  The trainable two-level selection follows "Light Forcing: Accelerating
 * Autoregressive Video Diffusion via Sparse Attention" (papernotes.org), "Key designs":
 * hierarchical sparse attention (frame-level then block-level top-K) and chunk-aware growth
 * (per-chunk budgets).
 *
 * Conventions for every call
 *  - Tokens are bf16, passed as raw 16-bit patterns.  Representatives, scores and
 *    log-sum-exp values are fp32.  Block lists are int32 global block ids.
 *  - Frames are tiled into blocks on their own: block j of frame f holds tokens
 *    f*frame_tokens + [block*j, min(block*(j+1), frame_tokens)); the last block of a frame
 *    may be short.  Global block id g = f*nb + j with nb = ceil(frame_tokens / block).
 *  - Pointers are DEVICE pointers unless a comment says "host".  The caller owns every
 *    buffer; the library never allocates, frees or keeps device memory, and keeps no
 *    state between calls except the thread-local error text.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only enqueues work on
 *    it and returns; no call synchronises or reads device memory back.  Buffers must stay
 *    valid until that work has run.
 *  - Arguments are validated before anything is enqueued; on error nothing is enqueued
 *    and a status below is returned, with detail in pbsa_last_error().  A failed launch
 *    returns PBSA_ERR_HIP.  Calls are reentrant.
 *  - Supported: head_dim 64 or 128, block 64, 1 <= frame_tokens, token strides multiples
 *    of 8 elements and token pointers 16-byte aligned.  Size limits (PBSA_ERR_UNSUPPORTED
 *    beyond them): persistent mode: capacity + window blocks <= 4096, capacity - sinks
 *    <= 1024, window blocks <= 1024, topk <= 1024 and, for pbsa_attn_fwd, capacity +
 *    chunk blocks + 2*topk <= 3072; two-level mode: pbsa_attn_fwd_2lvl and pbsa_attn_bwd
 *    max_sel <= 1536;
 *    a head's token rows of q, k, v and dout span at most 2 GiB and 2^24 tokens, and
 *    token strides are at most 2^24 elements.
 */
#ifndef PBSA_H_
#define PBSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PBSA_ABI_VERSION 3

typedef enum pbsa_status {
  PBSA_OK = 0,
  PBSA_ERR_NULL = 1,        /* a required pointer is NULL */
  PBSA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range */
  PBSA_ERR_UNSUPPORTED = 3, /* valid but not built: head_dim other than 64/128, block != 64,
                               or beyond a size limit listed above */
  PBSA_ERR_ALIGN = 4,       /* token pointer or stride not aligned for 16-byte loads */
  PBSA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than pbsa_workspace_bytes */
  PBSA_ERR_STATE = 6,       /* cache bookkeeping out of range (chunk_index) */
  PBSA_ERR_HIP = 7,         /* a HIP call failed; its text is in pbsa_last_error() */
  PBSA_ERR_INDEX = 8        /* a block list or cache table holds an id it may not hold
                               (pbsa_check_*; the first offender is in pbsa_last_error()) */
} pbsa_status;

/* Shapes of one attention layer.  For the two-level (trainable) calls only heads,
 * head_dim, block, frame_tokens, chunk_frames and scale are read. */
typedef struct pbsa_dims {
  int32_t heads;         /* H */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t block;         /* tokens per block: 64 */
  int32_t frame_tokens;  /* tokens per latent frame, n */
  int32_t chunk_frames;  /* frames generated per chunk, F */
  int32_t window_frames; /* history frames in the local window, W (F <= W) */
  int32_t capacity;      /* persistent memory capacity in blocks, C (sinks included) */
  int32_t sinks;         /* sink blocks S: global ids 0..S-1, S <= min(C, nb) */
  int32_t topk;          /* window blocks routed per query block, K >= 1 */
  float scale;           /* softmax scale, usually 1/sqrt(d) */
  int32_t route_mode;    /* persistent mode: PBSA_ROUTE_WINDOW (0) or PBSA_ROUTE_UNION (1) */
  int32_t kv_format;     /* persistent cache K/V: PBSA_KV_BF16 (0) or PBSA_KV_FP8 (1) */
} pbsa_dims;

/* How the persistent cache keeps K and V (Light Forcing, "Key findings": FP8 deployment):
 *   PBSA_KV_BF16: bf16 values.
 *   PBSA_KV_FP8:  OCP float8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 *                 bits; largest value 448), one byte per value, with one power-of-two scale
 *                 per slot and tensor, the smallest 2^e with max|x| <= 448 * 2^e over the
 *                 block's tokens (1 for an all-zero block); codes are the nearest to
 *                 x / 2^e, ties to the even mantissa.  The value a code stands for is
 *                 code * scale.  head_dim 128 only; the chunk's own K/V stay bf16.
 *                 pbsa_attn_bwd_persistent and pbsa_probe_gather do not take this format. */
enum { PBSA_KV_BF16 = 0, PBSA_KV_FP8 = 1 };

/* What the persistent-mode top-K chooses from (Sparse Forcing 2.C, where the query blocks are
 * scored against the persistent memory P and the local window L and the top-k kept):
 *   PBSA_ROUTE_WINDOW: the window blocks; every persistent block is attended.
 *   PBSA_ROUTE_UNION:  the non-sink persistent blocks and the window blocks together; only
 *                      the sinks are attended whole.  Limit: capacity + window blocks
 *                      <= 1024 in this mode.
 * The memory update is the same in both. */
enum { PBSA_ROUTE_WINDOW = 0, PBSA_ROUTE_UNION = 1 };

/* A bf16 token tensor: element (head h, token t, channel c) lives at
 * data[h*head_stride + t*token_stride + c] (strides in elements).  [T][H][d] has
 * token_stride = H*d, head_stride = d; [H][T][d] has token_stride = d, head_stride = T*d. */
typedef struct pbsa_tensor {
  void* data;
  int64_t token_stride;
  int64_t head_stride;
} pbsa_tensor;

/* Persistent-mode KV cache of one layer.  slots = capacity + window_frames*nb per head.
 * Slots [0, capacity) hold P_t (slots [0, sinks) the sinks); slot capacity + (f % W)*nb + j
 * holds window block j of history frame f.  A slot keeps its block's tokens row-major,
 * rows past len zero.  The struct itself is host memory; its pointers are device memory
 * of these sizes:
 *   k, v      bf16 [heads][slots][block][head_dim] (PBSA_KV_FP8: uint8 E4M3 codes)
 *   rep       fp32 [heads][slots][head_dim]   the block's mean key (its representative)
 *   block_id  int32 [heads][slots]            global block id, -1 = empty
 *   len       int32 [heads][slots]            valid tokens of the block
 * chunk_index counts the chunks appended so far; pbsa_memory_update advances it.
 * chunk_index_dev (optional, device int64, 8-byte aligned): a device copy of that count.
 * When it is not NULL the update kernels take the chunk index from it and advance it on
 * the device, so that an update captured once in a graph (pbsa_chunk_graph_create) is
 * right for every later chunk it is replayed for; the calls still advance chunk_index,
 * and the caller keeps the two equal (a graph replay advances only the device copy;
 * pbsa_chunk_graph_launch advances chunk_index as well).  pbsa_cache_reset zeroes both.
 * kv_scale (PBSA_KV_FP8 only, else unused): fp32 [heads][slots][2], the K and V scale of
 * each slot. */
typedef struct pbsa_cache {
  void* k;
  void* v;
  float* rep;
  int32_t* block_id;
  int32_t* len;
  int64_t chunk_index;
  int64_t* chunk_index_dev;
  float* kv_scale;
} pbsa_cache;

/* ---- helpers ---------------------------------------------------------------------- */

int pbsa_abi_version(void);
const char* pbsa_status_str(int status);
/* Text of the last error on this thread ("" if none). */
const char* pbsa_last_error(void);

/* Checks dims alone (range and support).  mode 0: persistent calls; 1: two-level calls. */
pbsa_status pbsa_check_dims(const pbsa_dims* dims, int32_t mode);

/* Slots per head of the persistent cache: capacity + window_frames * nb (0 if invalid). */
int64_t pbsa_cache_slots(const pbsa_dims* dims);

/* Device bytes of one layer's persistent cache (k, v, rep, block_id, len and, for
 * PBSA_KV_FP8, kv_scale; see pbsa_cache), 0 if dims are invalid. */
size_t pbsa_cache_bytes(const pbsa_dims* dims);

/* ---- host-side checks of lists and tables (no device access) ------------------------
 * For callers that build or keep routing lists and cache tables themselves: each check
 * reads HOST copies (taken after the caller's synchronisation) and returns PBSA_OK, or
 * PBSA_ERR_INDEX with the first offending entry described in pbsa_last_error().
 *
 * pbsa_check_cache_table: block_id, len [heads][slots] of a persistent cache that has
 *   appended chunk_index chunks (Sparse Forcing 2.B): the sink blocks 0..S-1 in slots
 *   0..S-1 (once a chunk has been appended); other persistent slots empty or holding
 *   distinct non-sink blocks of frames that have left the window; window slot
 *   capacity + (f % W)*nb + j holding block f*nb + j for every non-sink block of the W
 *   latest history frames (others empty); every length the block's token count.
 * pbsa_check_selection: sel [heads][Nq][topk] against such a table: per query block the
 *   ids before the first -1 strictly ascending, -1 only in the tail, every id a non-sink
 *   block the table holds in a window slot (PBSA_ROUTE_UNION: or in a persistent slot),
 *   and exactly min(topk, candidates) of them.
 * pbsa_check_selection_2lvl: sel [heads][Nq][max_sel], nsel [heads][Nq] of a clip of
 *   `chunks` chunks: 1 <= nsel <= max_sel, the first nsel ids strictly ascending, each a
 *   block of a frame the query block's chunk sees (frames < chunk_frames * i, chunk i
 *   1-based). */
pbsa_status pbsa_check_cache_table(const pbsa_dims* dims, const int32_t* block_id,
                                   const int32_t* len, int64_t chunk_index);
pbsa_status pbsa_check_selection(const pbsa_dims* dims, const int32_t* block_id,
                                 const int32_t* sel);
pbsa_status pbsa_check_selection_2lvl(const pbsa_dims* dims, int32_t chunks, const int32_t* sel,
                                      const int32_t* nsel, int32_t max_sel);

enum {
  PBSA_OP_MEMORY_UPDATE = 1,
  PBSA_OP_ATTN_BWD = 2,
  PBSA_OP_ATTN_BWD_PERSISTENT = 3,
  PBSA_OP_ATTN_FWD_FP8 = 4
};
/* Workspace bytes a call needs.  MEMORY_UPDATE, ATTN_BWD_PERSISTENT and ATTN_FWD_FP8: `arg`,
 * `arg2` unused.  ATTN_BWD: `arg` = clip chunks, `arg2` = max_sel. */
size_t pbsa_workspace_bytes(const pbsa_dims* dims, int32_t op, int32_t arg, int32_t arg2);

/* Empties the cache (block_id = -1, len = 0, chunk_index = 0).  K/V/rep are left as they
 * are; slots are fully written before they are first read. */
pbsa_status pbsa_cache_reset(const pbsa_dims* dims, pbsa_cache* cache, void* stream);

/* ---- step 1: pooling -----------------------------------------------------------------
 * Blockified compression (Sparse Forcing 2.C; Light Forcing, hierarchical sparse
 * attention step 1, mean pooling).  For `frames` frames of x (frames*frame_tokens tokens
 * per head) writes block_rep[h][g][c] = mean of block g's tokens and, if frame_rep is not
 * NULL, frame_rep[h][f][c] = mean of frame f's frame_tokens tokens.
 * block_rep: fp32 [heads][frames*nb][head_dim]; frame_rep: fp32 [heads][frames][head_dim].
 */
pbsa_status pbsa_pool(const pbsa_dims* dims, pbsa_tensor x, int32_t frames, float* block_rep,
                      float* frame_rep, void* stream);

/* ---- step 2: coarse scores and top-K routing (persistent mode) -----------------------
 * Sparse Forcing 2.C: for the chunk's Nq = chunk_frames*nb query blocks, with q_rep fp32
 * [heads][Nq][head_dim] (from pbsa_pool of the chunk's queries):
 *   scores[h][r][s] = scale * <q_rep[h][r], cache.rep[h][s]> for every valid slot s
 *                     (P_t and window), -inf for empty slots; fp32 [heads][Nq][slots].
 *   sel[h][r][0..K) = the K window blocks (sinks excluded; with PBSA_ROUTE_UNION the K
 *                     non-sink blocks of P_t and the window) with the highest score, ties
 *                     to the lower global id, written as global ids in ascending order; -1
 *                     fills the tail when there are fewer than K candidates.
 *                     int32 [heads][Nq][topk].
 */
pbsa_status pbsa_score_topk(const pbsa_dims* dims, const float* q_rep, const pbsa_cache* cache,
                            float* scores, int32_t* sel, void* stream);

/* Steps 1 and 2 of the query side in one launch: pools the chunk's query blocks (as
 * pbsa_pool of q) and scores and routes them (as pbsa_score_topk), with the same results.
 * q: chunk_frames*frame_tokens tokens per head.  q_rep: fp32 [heads][Nq][head_dim], 16-byte
 * aligned, receives the query block means, or NULL when they are not needed.  scores, sel:
 * as pbsa_score_topk.
 */
pbsa_status pbsa_route(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                       float* q_rep, float* scores, int32_t* sel, void* stream);

/* ---- step 3: attention over the selected blocks (persistent mode) --------------------
 * Sparse Forcing 2.C and the Chinese page's 2.2 (fine-grained attention, hybrid mask):
 * every query token t of query block r attends, with softmax scale dims.scale, to the
 * valid tokens of: every occupied persistent slot (PBSA_ROUTE_UNION: the sink slots), the
 * blocks sel[h][r][*], and all chunk_frames*nb blocks of the current chunk
 * (chunk_k/chunk_v, no causal mask inside the chunk).  Writes o (bf16, same shape as q: chunk_frames*frame_tokens tokens per head)
 * and lse[h][t] = natural-log sum of exp(scale * q.k) over the attended keys (fp32
 * [heads][chunk tokens]).  q, chunk_k, chunk_v: chunk_frames*frame_tokens tokens each.
 * sel: int32 [heads][Nq][topk] as pbsa_score_topk writes it: distinct global ids of blocks
 * the cache holds (window blocks; with PBSA_ROUTE_UNION also non-sink persistent blocks) in
 * ascending order, -1 only in the tail.  Other contents give undefined values (an id the
 * cache does not hold contributes nothing in PBSA_ROUTE_UNION mode) but every read stays
 * inside the cache and the chunk.
 */
pbsa_status pbsa_attn_fwd(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                          pbsa_tensor chunk_k, pbsa_tensor chunk_v, const int32_t* sel,
                          pbsa_tensor o, float* lse, void* stream);

/* ---- step 3 in FP8 arithmetic (FP8 cache) --------------------------------------------
 * Light Forcing, "Key findings" (the sparse attention deployed in FP8).  The attention of
 * pbsa_attn_fwd over an FP8 cache (dims.kv_format = PBSA_KV_FP8: the cache's E4M3 codes and
 * power-of-two block scales), computed on FP8 matrix cores instead of after an exact decode
 * to bf16:
 *   - each query row, times c = scale * log2(e) (fp32 product), is quantized to E4M3 with
 *     its own power-of-two scale (the smallest 2^e with max|c q| <= 448 * 2^e), nearest even;
 *   - the chunk's K/V blocks are quantized per block and tensor as pbsa_memory_update
 *     quantizes a cache slot (codes and scales go to the workspace);
 *   - scores are exact products of the decoded values summed in fp32 (in exp2 units); the
 *     probabilities p = 2^(s - m) (a per-row offset m with every p <= 448) are rounded to
 *     E4M3 (nearest even) for the product with V, while the row sum adds the unrounded
 *     values.
 * The offset keeps the row max at p >= 8, so o differs from the exact attention of the
 * quantized q by at most 2^-4 * sum_j p_j |v_j| / sum_j p_j per channel (the rounding of p in
 * E4M3's normal range) plus fp32 and bf16 rounding and the subnormal range's absolute 2^-10
 * per p (p below 2^-9 of the row max); lse is that of the quantized q.
 * Arguments, layouts and errors as pbsa_attn_fwd, plus: kv_format must be PBSA_KV_FP8
 * (PBSA_ERR_UNSUPPORTED otherwise); workspace: device, 16-byte aligned,
 * >= pbsa_workspace_bytes(dims, PBSA_OP_ATTN_FWD_FP8, 0, 0) bytes (overwritten;
 * PBSA_ERR_WORKSPACE if smaller).  Two kernels on `stream`: the chunk's quantization, then
 * the attention. */
pbsa_status pbsa_attn_fwd_fp8(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                              pbsa_tensor chunk_k, pbsa_tensor chunk_v, const int32_t* sel,
                              pbsa_tensor o, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---- step 4: persistent-memory update and window append ------------------------------
 * Sparse Forcing 2.B/2.C (Top-C retention as the window slides, sinks always kept).  With
 * c = cache.chunk_index and h = c*chunk_frames appended frames, appending the chunk pushes
 * frames [max(0,h-W), max(0,h+F-W)) out of the window; their non-sink blocks E join the
 * non-sink persistent blocks as candidates R; each candidate's memory score is the sum over
 * the chunk's query blocks of its coarse score (column sums of `scores` from
 * pbsa_score_topk of this chunk); the new P_t is the sinks plus the C - S best candidates
 * by (memory score desc, id asc).  Kept blocks stay in their slots, promoted blocks are
 * copied (K, V, rep, len) into the freed slots in ascending id order, and the chunk's K/V
 * and chunk_rep (fp32 [heads][Nq][head_dim], pbsa_pool of chunk_k) are written into the
 * window slots of the frames that left.  chunk_rep may be NULL: the block means of chunk_k
 * are then computed from the rows being copied (fp32, equal to pbsa_pool's up to the order
 * of the additions).  On chunk 0 the sink blocks go to slots [0, S).
 * Finally cache->chunk_index is incremented (host).
 * workspace: device, >= pbsa_workspace_bytes(dims, PBSA_OP_MEMORY_UPDATE, 0, 0) bytes.
 */
pbsa_status pbsa_memory_update(const pbsa_dims* dims, const float* scores, pbsa_cache* cache,
                               pbsa_tensor chunk_k, pbsa_tensor chunk_v, const float* chunk_rep,
                               void* workspace, size_t workspace_bytes, void* stream);

/* The two halves of pbsa_memory_update, for callers that overlap the selection with the
 * chunk's attention; select then apply on the same cache state and workspace give exactly
 * the result of pbsa_memory_update.
 * pbsa_memory_select: the candidate scores, the new P_t and the copy list, written to the
 *   workspace only; it reads the cache (block_id, len, chunk_index) and `scores`, and
 *   writes nothing the attention reads, so it may run on another stream while
 *   pbsa_attn_fwd of the same chunk reads the cache (after `scores` are complete).
 * pbsa_memory_apply: writes the new P_t, the promotion copies and the chunk into the cache
 *   from that workspace (it must follow the select and every reader of the cache), then
 *   increments cache->chunk_index (host).  Errors as pbsa_memory_update; the workspace
 *   must hold a select of the same cache state and chunk_index (otherwise the cache's
 *   contents are undefined, though every write stays inside the cache). */
pbsa_status pbsa_memory_select(const pbsa_dims* dims, const float* scores,
                               const pbsa_cache* cache, void* workspace, size_t workspace_bytes,
                               void* stream);
pbsa_status pbsa_memory_apply(const pbsa_dims* dims, pbsa_cache* cache, pbsa_tensor chunk_k,
                              pbsa_tensor chunk_v, const float* chunk_rep, void* workspace,
                              size_t workspace_bytes, void* stream);

/* pbsa_memory_update without a workspace argument, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid
 * allocation).  The workspace is a library-held device array of 1 MiB per GPU (held until
 * the process ends); dims needing more (pbsa_workspace_bytes(dims, PBSA_OP_MEMORY_UPDATE))
 * return PBSA_ERR_UNSUPPORTED.  The call allocates nothing.  Every call on one GPU shares
 * that array: calls that overlap on one GPU (on different streams, or from several
 * threads) race and give undefined results; calls ordered on one stream are safe (each
 * call writes every workspace word it reads).  Otherwise exactly pbsa_memory_update. */
pbsa_status pbsa_memory_update_noalloc(const pbsa_dims* dims, const float* scores,
                                       pbsa_cache* cache, pbsa_tensor chunk_k,
                                       pbsa_tensor chunk_v, const float* chunk_rep,
                                       void* stream);

/* Gradient of pbsa_attn_fwd (persistent mode) with the selection held constant: Sparse
 * Forcing's own trainable layout (English page, 2.D: the model is trained with the same
 * dynamic sparse cache it uses at inference; 3: one kernel family for decoding and
 * training).  Same arguments as pbsa_attn_fwd (the cache state and `sel` it attended),
 * plus its o and lse and the upstream gradient dout (like q).  Writes dq (like q), dk and
 * dv for the chunk's own keys and values (like chunk_k), and dk_cache, dv_cache: bf16
 * [heads][slots][block][head_dim], the gradient of every cache slot's K and V (all block
 * rows written: zero past the slot's length, and for slots no query attended).  No
 * gradient flows through routing, pooling or the memory update.  Deterministic: atomics
 * only build integer lists and hand out work; every floating-point sum runs in a fixed
 * order.  Limit: capacity + topk + chunk blocks <= 1536.
 * workspace: >= pbsa_workspace_bytes(dims, PBSA_OP_ATTN_BWD_PERSISTENT, 0, 0) bytes. */
pbsa_status pbsa_attn_bwd_persistent(const pbsa_dims* dims, pbsa_tensor q,
                                     const pbsa_cache* cache, pbsa_tensor chunk_k,
                                     pbsa_tensor chunk_v, const int32_t* sel, pbsa_tensor o,
                                     const float* lse, pbsa_tensor dout, pbsa_tensor dq,
                                     pbsa_tensor dk, pbsa_tensor dv, void* dk_cache,
                                     void* dv_cache, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* ---- the chunk step: T denoising passes sharing the memory --------------------------
 * Sparse Forcing 2.B (P_t and the window persist while a chunk is denoised; the Chinese
 * page's 2.1: the memory is shared between diffusion steps) with the update of 2.C.  For
 * p = 0 .. passes-1: pbsa_route(q[p]) then pbsa_attn_fwd(q[p], k[p], v[p]) -> o[p], lse[p];
 * then pbsa_memory_update with the last pass's scores and k/v (chunk_rep = NULL): the last
 * pass is the one whose K/V enter the cache.  Every buffer is as in those calls (q_rep may
 * be NULL); scores and sel are shared by the passes and end up holding the last pass's.
 * workspace: >= pbsa_workspace_bytes(dims, PBSA_OP_MEMORY_UPDATE, 0, 0) bytes.
 * fp8_arithmetic != 0 (FP8 cache only, else PBSA_ERR_UNSUPPORTED): the attentions are
 * pbsa_attn_fwd_fp8, with attn_workspace (16-byte aligned, >= pbsa_workspace_bytes(dims,
 * PBSA_OP_ATTN_FWD_FP8, 0, 0) bytes; it must not overlap `workspace`, which the captured
 * update's selection uses at the same time); otherwise attn_workspace is not read. */
#define PBSA_MAX_PASSES 8
typedef struct pbsa_chunk_args {
  int32_t passes;
  pbsa_tensor q[PBSA_MAX_PASSES];
  pbsa_tensor k[PBSA_MAX_PASSES];
  pbsa_tensor v[PBSA_MAX_PASSES];
  pbsa_tensor o[PBSA_MAX_PASSES];
  float* lse[PBSA_MAX_PASSES];
  float* q_rep;
  float* scores;
  int32_t* sel;
  void* workspace;
  size_t workspace_bytes;
  int32_t fp8_arithmetic;
  void* attn_workspace;
  size_t attn_workspace_bytes;
} pbsa_chunk_args;

/* The chunk step as one call: the launches above in order on `stream`; advances
 * cache->chunk_index. */
pbsa_status pbsa_chunk_step(const pbsa_dims* dims, const pbsa_chunk_args* args,
                            pbsa_cache* cache, void* stream);

/* The same step captured once as a HIP graph (host object, created by the library and
 * released by pbsa_chunk_graph_destroy; it owns two streams and two events, no device
 * memory).  The update's selection runs on a second branch beside the last pass's
 * attention.  The cache must carry chunk_index_dev: the captured update reads the chunk
 * index there, so one graph serves every later chunk whose inputs are written into the
 * captured buffers (args' pointers are baked in; the buffers must outlive the graph).
 * pbsa_chunk_graph_launch replays it on `stream` for the cache it was captured on
 * (PBSA_ERR_STATE otherwise) and advances cache->chunk_index. */
typedef struct pbsa_chunk_graph pbsa_chunk_graph;
pbsa_status pbsa_chunk_graph_create(const pbsa_dims* dims, const pbsa_chunk_args* args,
                                    const pbsa_cache* cache, pbsa_chunk_graph** out);
pbsa_status pbsa_chunk_graph_launch(pbsa_chunk_graph* graph, pbsa_cache* cache, void* stream);
void pbsa_chunk_graph_destroy(pbsa_chunk_graph* graph);

/* ---- trainable path: two-level selection ---------------------------------------------
 * Light Forcing, hierarchical sparse attention (steps 2 and 3) with the chunk-aware
 * budget.  A clip of `chunks` chunks (chunk_frames frames each) is processed as one
 * forward.  For query block r of chunk i (1-based):
 *   i = 1:  all blocks of chunk 1's own frames (dense).
 *   i >= 2: frame scores scale*<q_rep, frame_rep[f]> over history frames f < F(i-1); the
 *           top_frames best (ties to the lower frame) united with frame 0, frame F(i-1)-1
 *           and the chunk's own frames; among all blocks of those frames, the
 *           min(k_per_chunk[i-1], candidates) best by scale*<q_rep, block_rep[g]>, ties to
 *           the lower id.
 * Writes sel[h][r][0..nsel) ascending global ids (int32 [heads][Nq][max_sel], the tail
 * left untouched) and nsel[h][r] (int32 [heads][Nq]), Nq = chunks*chunk_frames*nb.
 * q_rep, block_rep: fp32 [heads][Nq][head_dim]; frame_rep fp32 [heads][chunks*F][head_dim].
 * k_per_chunk: HOST int32 [chunks] (entry 0 unused), chunks <= 256.  max_sel must be at
 * least chunk_frames*nb and every k_per_chunk entry.  Scores are fp32 products summed in
 * fp32 (on the matrix cores, 32 query blocks at a time, when a chunk's scores fit in LDS;
 * else as per-row dot products), so selections are exact up to the order of the fp32
 * additions (near-ties).
 */
pbsa_status pbsa_score_topk_2lvl(const pbsa_dims* dims, int32_t chunks, int32_t top_frames,
                                 const int32_t* k_per_chunk, const float* q_rep,
                                 const float* block_rep, const float* frame_rep,
                                 int32_t max_sel, int32_t* sel, int32_t* nsel, void* stream);

/* Attention of the clip's queries over their selected blocks (sel/nsel from
 * pbsa_score_topk_2lvl): o (bf16, like q) and lse (fp32 [heads][clip tokens]).
 * q, k, v: chunks*chunk_frames*frame_tokens tokens per head.  max_sel <= 1536.
 * sel/nsel are meant to pass pbsa_check_selection_2lvl (what pbsa_score_topk_2lvl writes
 * does); for other lists the values are undefined (the forward attends every listed id,
 * the backward's dK/dV leave out blocks the query block's chunk cannot see), but ids
 * outside the clip are skipped and no read leaves q, k, v and the lists. */
pbsa_status pbsa_attn_fwd_2lvl(const pbsa_dims* dims, int32_t chunks, pbsa_tensor q,
                               pbsa_tensor k, pbsa_tensor v, const int32_t* sel,
                               const int32_t* nsel, int32_t max_sel, pbsa_tensor o, float* lse,
                               void* stream);

/* Gradient of pbsa_attn_fwd_2lvl's output with the selection held constant (no gradient
 * through routing or pooling): given o, lse from the forward and the upstream gradient
 * dout, writes dq, dk, dv (bf16, same shapes as q, k, v).  Deterministic: atomics only build
 * integer lists and hand out work; every floating-point sum runs in a fixed order.
 * workspace: device, >= pbsa_workspace_bytes(dims, PBSA_OP_ATTN_BWD, chunks, max_sel). */
pbsa_status pbsa_attn_bwd(const pbsa_dims* dims, int32_t chunks, pbsa_tensor q, pbsa_tensor k,
                          pbsa_tensor v, pbsa_tensor o, const float* lse, pbsa_tensor dout,
                          const int32_t* sel, const int32_t* nsel, int32_t max_sel,
                          pbsa_tensor dq, pbsa_tensor dk, pbsa_tensor dv, void* workspace,
                          size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PBSA_H_ */
