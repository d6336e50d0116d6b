// C ABI of libpbsa: argument validation, then launches on the caller's stream.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/pbsa.h"
#include "../../include/pbsa_probe.h"
#include "launch.h"
#include "step_internal.h"

namespace pbsa {
namespace api {

thread_local std::string g_err;

pbsa_status fail(pbsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

pbsa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) {
    g_err.clear();
    return PBSA_OK;
  }
  return fail(PBSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxSlots = 4096;
constexpr int kMaxChunks = 256;

pbsa_status check_dims(const pbsa_dims* d, int mode) {
  if (!d) return fail(PBSA_ERR_NULL, "dims is NULL");
  if (d->heads < 1) return fail(PBSA_ERR_SHAPE, "heads must be >= 1 (got %d)", d->heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(d->head_dim > 0 ? PBSA_ERR_UNSUPPORTED : PBSA_ERR_SHAPE,
                "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->block != 64)
    return fail(d->block > 0 ? PBSA_ERR_UNSUPPORTED : PBSA_ERR_SHAPE,
                "block must be 64 (got %d)", d->block);
  if (d->frame_tokens < 1) return fail(PBSA_ERR_SHAPE, "frame_tokens must be >= 1");
  if (d->chunk_frames < 1) return fail(PBSA_ERR_SHAPE, "chunk_frames must be >= 1");
  if (!(d->scale > 0.f) || !std::isfinite(d->scale))
    return fail(PBSA_ERR_SHAPE, "scale must be a positive finite number");
  if (mode == 0) {
    const int nb = pbsa::nb_of(*d);
    if (d->window_frames < d->chunk_frames)
      return fail(PBSA_ERR_SHAPE, "window_frames (%d) must be >= chunk_frames (%d)",
                  d->window_frames, d->chunk_frames);
    if (d->sinks < 0 || d->sinks > d->capacity || d->sinks > nb)
      return fail(PBSA_ERR_SHAPE, "need 0 <= sinks <= min(capacity, blocks per frame)");
    if (d->capacity < 0) return fail(PBSA_ERR_SHAPE, "capacity must be >= 0");
    if (d->route_mode != PBSA_ROUTE_WINDOW && d->route_mode != PBSA_ROUTE_UNION)
      return fail(PBSA_ERR_SHAPE, "route_mode must be PBSA_ROUTE_WINDOW or PBSA_ROUTE_UNION");
    if (d->kv_format != PBSA_KV_BF16 && d->kv_format != PBSA_KV_FP8)
      return fail(PBSA_ERR_SHAPE, "kv_format must be PBSA_KV_BF16 or PBSA_KV_FP8");
    if (d->kv_format == PBSA_KV_FP8 && d->head_dim != 128)
      return fail(PBSA_ERR_UNSUPPORTED, "the FP8 cache is built for head_dim 128");
    if (d->kv_format == PBSA_KV_FP8 &&
        int64_t{d->capacity} + d->topk + int64_t{d->chunk_frames} * pbsa::nb_of(*d) >
            pbsa::kAttnListCap / 2)
      return fail(PBSA_ERR_UNSUPPORTED, "FP8 cache: capacity + topk + chunk blocks must be <= %d",
                  pbsa::kAttnListCap / 2);
    if (d->topk < 1) return fail(PBSA_ERR_SHAPE, "topk must be >= 1");
    if (d->topk > 1024) return fail(PBSA_ERR_UNSUPPORTED, "topk must be <= 1024");
    const int64_t slots = pbsa::slots_of(*d);
    if (slots > kMaxSlots)
      return fail(PBSA_ERR_UNSUPPORTED, "capacity + window blocks = %lld exceeds %lld",
                  static_cast<long long>(slots), static_cast<long long>(kMaxSlots));
    if (d->capacity - d->sinks > 1024)
      return fail(PBSA_ERR_UNSUPPORTED, "capacity - sinks must be <= 1024");
    if (static_cast<int64_t>(d->window_frames) * nb > 1024)
      return fail(PBSA_ERR_UNSUPPORTED, "window blocks must be <= 1024");
    if (d->route_mode == PBSA_ROUTE_UNION && slots > 1024)
      return fail(PBSA_ERR_UNSUPPORTED,
                  "PBSA_ROUTE_UNION needs capacity + window blocks <= 1024 (got %lld)",
                  static_cast<long long>(slots));
    // LDS of the memory-update selection: block tables, candidate list and partial sums,
    // free list (the limits above keep it under 80 KB)
    const int64_t ncand = static_cast<int64_t>(d->capacity - d->sinks) + int64_t{d->chunk_frames} * nb;
    if ((2 * slots + 5 * ncand + d->capacity) * 4 > 150 * 1024)
      return fail(PBSA_ERR_UNSUPPORTED, "capacity/window too large for the memory update");
  } else if (mode != 1) {
    return fail(PBSA_ERR_SHAPE, "mode must be 0 (persistent) or 1 (two-level)");
  }
  return PBSA_OK;
}

pbsa_status check_tok(const pbsa_tensor& t, const char* name, int head_dim) {
  if (!t.data) return fail(PBSA_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(t.data) % 16)
    return fail(PBSA_ERR_ALIGN, "%s must be 16-byte aligned", name);
  if (t.token_stride % 8 || t.head_stride % 8)
    return fail(PBSA_ERR_ALIGN, "%s strides must be multiples of 8 elements", name);
  if (t.token_stride < head_dim || t.head_stride < 0)
    return fail(PBSA_ERR_SHAPE, "%s strides out of range", name);
  return PBSA_OK;
}

// The attention kernels address a head's token rows with 32-bit byte offsets (a 64-row
// block with 32-bit offsets from its first row, hence the stride limit) and name a token
// block by its first token in 24 bits.
pbsa_status check_span(const pbsa_tensor& t, const char* name, int64_t tokens, int head_dim) {
  const int64_t bytes = (tokens - 1) * t.token_stride * 2 + int64_t{head_dim} * 2;
  if (tokens > 0 && bytes > (int64_t{1} << 31))
    return fail(PBSA_ERR_UNSUPPORTED, "%s spans more than 2 GiB per head", name);
  if (tokens > (int64_t{1} << 24))
    return fail(PBSA_ERR_UNSUPPORTED, "%s has more than 2^24 tokens", name);
  if (t.token_stride > (int64_t{1} << 24))
    return fail(PBSA_ERR_UNSUPPORTED, "%s token stride exceeds 2^24 elements", name);
  return PBSA_OK;
}

pbsa_status check_cache(const pbsa_cache* c, const pbsa_dims* d) {
  if (!c) return fail(PBSA_ERR_NULL, "cache is NULL");
  if (d && d->kv_format == PBSA_KV_FP8) {
    if (!c->kv_scale) return fail(PBSA_ERR_NULL, "an FP8 cache needs kv_scale");
    if (reinterpret_cast<uintptr_t>(c->kv_scale) % 8)
      return fail(PBSA_ERR_ALIGN, "kv_scale must be 8-byte aligned");
  }
  if (!c->k || !c->v || !c->rep || !c->block_id || !c->len)
    return fail(PBSA_ERR_NULL, "a cache buffer is NULL");
  if (reinterpret_cast<uintptr_t>(c->k) % 16 || reinterpret_cast<uintptr_t>(c->v) % 16 ||
      reinterpret_cast<uintptr_t>(c->rep) % 16)
    return fail(PBSA_ERR_ALIGN, "cache k, v and rep must be 16-byte aligned");
  if (c->chunk_index < 0) return fail(PBSA_ERR_STATE, "chunk_index is negative");
  if (reinterpret_cast<uintptr_t>(c->chunk_index_dev) % 8)
    return fail(PBSA_ERR_ALIGN, "chunk_index_dev must be 8-byte aligned");
  return PBSA_OK;
}

hipStream_t stream_of(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace api
}  // namespace pbsa

using namespace pbsa::api;

extern "C" {

int pbsa_abi_version(void) { return PBSA_ABI_VERSION; }

const char* pbsa_status_str(int status) {
  switch (status) {
    case PBSA_OK: return "ok";
    case PBSA_ERR_NULL: return "null pointer";
    case PBSA_ERR_SHAPE: return "bad shape";
    case PBSA_ERR_UNSUPPORTED: return "unsupported";
    case PBSA_ERR_ALIGN: return "misaligned";
    case PBSA_ERR_WORKSPACE: return "workspace too small";
    case PBSA_ERR_STATE: return "bad cache state";
    case PBSA_ERR_HIP: return "hip error";
    case PBSA_ERR_INDEX: return "bad index";
    default: return "unknown status";
  }
}

const char* pbsa_last_error(void) { return g_err.c_str(); }

pbsa_status pbsa_check_dims(const pbsa_dims* dims, int32_t mode) {
  PBSA_TRY(check_dims(dims, mode));
  g_err.clear();
  return PBSA_OK;
}

int64_t pbsa_cache_slots(const pbsa_dims* dims) {
  if (check_dims(dims, 0) != PBSA_OK) return 0;
  return pbsa::slots_of(*dims);
}

size_t pbsa_cache_bytes(const pbsa_dims* dims) {
  if (check_dims(dims, 0) != PBSA_OK) return 0;
  const bool fp8 = dims->kv_format == PBSA_KV_FP8;
  const size_t per_slot = 2 * static_cast<size_t>(dims->block) * dims->head_dim * (fp8 ? 1 : 2) +
                          static_cast<size_t>(dims->head_dim) * 4 + 2 * 4 + (fp8 ? 2 * 4 : 0);
  return static_cast<size_t>(dims->heads) * static_cast<size_t>(pbsa::slots_of(*dims)) * per_slot;
}

pbsa_status pbsa_check_cache_table(const pbsa_dims* dims, const int32_t* block_id,
                                   const int32_t* len, int64_t chunk_index) {
  PBSA_TRY(check_dims(dims, 0));
  if (!block_id || !len) return fail(PBSA_ERR_NULL, "block_id and len are required");
  if (chunk_index < 0) return fail(PBSA_ERR_STATE, "chunk_index is negative");
  const int nb = pbsa::nb_of(*dims), C = dims->capacity, S = dims->sinks, W = dims->window_frames;
  const int64_t slots = pbsa::slots_of(*dims);
  const int64_t hist = chunk_index * dims->chunk_frames;  // history frames
  const int64_t win0 = std::max<int64_t>(0, hist - W);    // first window frame
  auto blen = [&](int64_t g) { return pbsa::block_len(static_cast<int>(g % nb), dims->frame_tokens); };
  std::vector<char> seen;
  for (int h = 0; h < dims->heads; ++h) {
    const int32_t* b = block_id + static_cast<int64_t>(h) * slots;
    const int32_t* l = len + static_cast<int64_t>(h) * slots;
    seen.assign(static_cast<size_t>(std::max<int64_t>(1, win0 * nb)), 0);
    for (int s = 0; s < C; ++s) {
      const int32_t g = b[s];
      if (s < S && chunk_index > 0) {
        if (g != s || l[s] != blen(s))
          return fail(PBSA_ERR_INDEX, "head %d slot %d: sink %d missing (holds %d, len %d)", h, s,
                      s, g, l[s]);
        continue;
      }
      if (g < 0) {
        if (l[s] != 0) return fail(PBSA_ERR_INDEX, "head %d slot %d: empty with len %d", h, s, l[s]);
        continue;
      }
      if (g < S || g >= win0 * nb)
        return fail(PBSA_ERR_INDEX, "head %d persistent slot %d holds block %d (not a non-sink "
                    "block that has left the window)", h, s, g);
      if (seen[g]) return fail(PBSA_ERR_INDEX, "head %d: block %d held twice", h, g);
      seen[g] = 1;
      if (l[s] != blen(g))
        return fail(PBSA_ERR_INDEX, "head %d slot %d: block %d has len %d", h, s, g, l[s]);
    }
    for (int64_t s = C; s < slots; ++s) {
      const int64_t rel = s - C, fr = rel / nb, j = rel % nb;
      // the latest history frame that maps to this ring slot
      int64_t f = -1;
      if (hist > 0) {
        const int64_t last = hist - 1;
        f = last - ((last - fr) % W + W) % W;
      }
      const int64_t g = f * nb + j;
      const bool want = f >= win0 && f >= 0 && g >= S;
      if (want ? (b[s] != g || l[s] != blen(g)) : (b[s] != -1 || l[s] != 0))
        return fail(PBSA_ERR_INDEX, "head %d window slot %lld holds block %d (len %d), expected %lld",
                    h, static_cast<long long>(s), b[s], l[s], static_cast<long long>(want ? g : -1));
    }
  }
  g_err.clear();
  return PBSA_OK;
}

pbsa_status pbsa_check_selection(const pbsa_dims* dims, const int32_t* block_id,
                                 const int32_t* sel) {
  PBSA_TRY(check_dims(dims, 0));
  if (!block_id || !sel) return fail(PBSA_ERR_NULL, "block_id and sel are required");
  const int nb = pbsa::nb_of(*dims), C = dims->capacity, S = dims->sinks, K = dims->topk;
  const int nq = dims->chunk_frames * nb;
  const int64_t slots = pbsa::slots_of(*dims);
  const bool uni = dims->route_mode == PBSA_ROUTE_UNION;
  for (int h = 0; h < dims->heads; ++h) {
    const int32_t* b = block_id + static_cast<int64_t>(h) * slots;
    int ncand = 0;
    for (int64_t s = uni ? 0 : C; s < slots; ++s) ncand += b[s] >= S;
    const int want = std::min(K, ncand);
    for (int r = 0; r < nq; ++r) {
      const int32_t* row = sel + (static_cast<int64_t>(h) * nq + r) * K;
      int n = 0;
      while (n < K && row[n] >= 0) ++n;
      for (int j = n; j < K; ++j)
        if (row[j] != -1)
          return fail(PBSA_ERR_INDEX, "head %d query block %d: entry %d after the -1 tail", h, r, j);
      if (n != want)
        return fail(PBSA_ERR_INDEX, "head %d query block %d: %d ids, expected %d", h, r, n, want);
      for (int j = 0; j < n; ++j) {
        const int32_t g = row[j];
        if (j > 0 && g <= row[j - 1])
          return fail(PBSA_ERR_INDEX, "head %d query block %d: ids not strictly ascending at %d",
                      h, r, j);
        const int64_t ws = C + static_cast<int64_t>((g / nb) % dims->window_frames) * nb + g % nb;
        bool held = g >= S && b[ws] == g;
        for (int s = S; uni && !held && s < C; ++s) held = b[s] == g;
        if (!held)
          return fail(PBSA_ERR_INDEX, "head %d query block %d: block %d is not a candidate the "
                      "cache holds", h, r, g);
      }
    }
  }
  g_err.clear();
  return PBSA_OK;
}

pbsa_status pbsa_check_selection_2lvl(const pbsa_dims* dims, int32_t chunks, const int32_t* sel,
                                      const int32_t* nsel, int32_t max_sel) {
  PBSA_TRY(check_dims(dims, 1));
  if (!sel || !nsel) return fail(PBSA_ERR_NULL, "sel and nsel are required");
  if (chunks < 1 || max_sel < 1) return fail(PBSA_ERR_SHAPE, "chunks and max_sel must be >= 1");
  const int nb = pbsa::nb_of(*dims), F = dims->chunk_frames;
  const int64_t nq = static_cast<int64_t>(chunks) * F * nb;
  for (int h = 0; h < dims->heads; ++h)
    for (int64_t r = 0; r < nq; ++r) {
      const int64_t hr = static_cast<int64_t>(h) * nq + r;
      const int n = nsel[hr];
      if (n < 1 || n > max_sel)
        return fail(PBSA_ERR_INDEX, "head %d query block %lld: nsel %d outside [1, %d]", h,
                    static_cast<long long>(r), n, max_sel);
      const int64_t i = r / (static_cast<int64_t>(F) * nb) + 1;  // chunk, 1-based
      const int32_t* row = sel + hr * max_sel;
      for (int j = 0; j < n; ++j) {
        const int32_t g = row[j];
        if (g < 0 || g >= nq || g / nb >= F * i)
          return fail(PBSA_ERR_INDEX, "head %d query block %lld: block %d is not visible to it",
                      h, static_cast<long long>(r), g);
        if (j > 0 && g <= row[j - 1])
          return fail(PBSA_ERR_INDEX, "head %d query block %lld: ids not strictly ascending at %d",
                      h, static_cast<long long>(r), j);
      }
    }
  g_err.clear();
  return PBSA_OK;
}

size_t pbsa_workspace_bytes(const pbsa_dims* dims, int32_t op, int32_t arg, int32_t arg2) {
  if (op == PBSA_OP_MEMORY_UPDATE) {
    if (check_dims(dims, 0) != PBSA_OK) return 0;
    return pbsa::memory_update_workspace(*dims);
  }
  if (op == PBSA_OP_ATTN_BWD_PERSISTENT) {
    if (check_dims(dims, 0) != PBSA_OK) return 0;
    return pbsa::attn_bwd_persistent_workspace(*dims);
  }
  if (op == PBSA_OP_ATTN_FWD_FP8) {
    if (check_dims(dims, 0) != PBSA_OK || dims->kv_format != PBSA_KV_FP8) return 0;
    return pbsa::attn_fwd_f8_workspace(*dims);
  }
  if (op == PBSA_OP_ATTN_BWD) {
    if (check_dims(dims, 1) != PBSA_OK || arg < 1 || arg2 < 1) return 0;
    return pbsa::attn_bwd_workspace(*dims, arg, arg2);
  }
  return 0;
}

pbsa_status pbsa_cache_reset(const pbsa_dims* dims, pbsa_cache* cache, void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  cache->chunk_index = 0;
  return hip_status(pbsa::launch_cache_reset(*dims, *cache, stream_of(stream)), "cache_reset");
}

pbsa_status pbsa_pool(const pbsa_dims* dims, pbsa_tensor x, int32_t frames, float* block_rep,
                      float* frame_rep, void* stream) {
  PBSA_TRY(check_dims(dims, 1));
  PBSA_TRY(check_tok(x, "x", dims->head_dim));
  if (frames < 0) return fail(PBSA_ERR_SHAPE, "frames must be >= 0");
  if (!block_rep) return fail(PBSA_ERR_NULL, "block_rep is NULL");
  if (reinterpret_cast<uintptr_t>(block_rep) % 16)
    return fail(PBSA_ERR_ALIGN, "block_rep must be 16-byte aligned");
  return hip_status(pbsa::launch_pool(*dims, pbsa::tok_in(x), frames, block_rep, frame_rep,
                                      stream_of(stream)),
                    "pool");
}

pbsa_status pbsa_score_topk(const pbsa_dims* dims, const float* q_rep, const pbsa_cache* cache,
                            float* scores, int32_t* sel, void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  if (!q_rep || !scores || !sel) return fail(PBSA_ERR_NULL, "q_rep, scores and sel are required");
  if (reinterpret_cast<uintptr_t>(q_rep) % 16)
    return fail(PBSA_ERR_ALIGN, "q_rep must be 16-byte aligned");
  return hip_status(pbsa::launch_score_topk(*dims, q_rep, *cache, scores, sel, stream_of(stream)),
                    "score_topk");
}

pbsa_status pbsa_route(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                       float* q_rep, float* scores, int32_t* sel, void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  PBSA_TRY(check_tok(q, "q", dims->head_dim));
  if (!scores || !sel) return fail(PBSA_ERR_NULL, "scores and sel are required");
  if (reinterpret_cast<uintptr_t>(q_rep) % 16)
    return fail(PBSA_ERR_ALIGN, "q_rep must be 16-byte aligned");
  return hip_status(pbsa::launch_route(*dims, pbsa::tok_in(q), q_rep, *cache, scores, sel,
                                       stream_of(stream)),
                    "route");
}

pbsa_status pbsa_attn_fwd(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                          pbsa_tensor chunk_k, pbsa_tensor chunk_v, const int32_t* sel,
                          pbsa_tensor o, float* lse, void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  PBSA_TRY(check_tok(q, "q", dims->head_dim));
  PBSA_TRY(check_tok(chunk_k, "chunk_k", dims->head_dim));
  PBSA_TRY(check_tok(chunk_v, "chunk_v", dims->head_dim));
  PBSA_TRY(check_tok(o, "o", dims->head_dim));
  const int64_t ctok = int64_t{dims->chunk_frames} * dims->frame_tokens;
  const int64_t list = int64_t{dims->capacity} + int64_t{dims->chunk_frames} * pbsa::nb_of(*dims) +
                       2 * int64_t{dims->topk};
  if (list > pbsa::kAttnListCap)
    return fail(PBSA_ERR_UNSUPPORTED, "capacity + chunk blocks + 2*topk = %lld exceeds %d",
                static_cast<long long>(list), pbsa::kAttnListCap);
  PBSA_TRY(check_span(chunk_k, "chunk_k", ctok, dims->head_dim));
  PBSA_TRY(check_span(chunk_v, "chunk_v", ctok, dims->head_dim));
  if (!sel || !lse) return fail(PBSA_ERR_NULL, "sel and lse are required");
  if (dims->kv_format == PBSA_KV_FP8)
    return hip_status(pbsa::launch_attn_fwd_fp8(*dims, pbsa::tok_in(q), *cache,
                                                pbsa::tok_in(chunk_k), pbsa::tok_in(chunk_v),
                                                sel, pbsa::tok_out(o), lse, stream_of(stream)),
                      "attn_fwd (fp8 cache)");
  return hip_status(pbsa::launch_attn_fwd_persistent(*dims, pbsa::tok_in(q), *cache,
                                                     pbsa::tok_in(chunk_k),
                                                     pbsa::tok_in(chunk_v), sel,
                                                     pbsa::tok_out(o), lse, stream_of(stream)),
                    "attn_fwd");
}

pbsa_status pbsa_attn_fwd_fp8(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                              pbsa_tensor chunk_k, pbsa_tensor chunk_v, const int32_t* sel,
                              pbsa_tensor o, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  if (dims->kv_format != PBSA_KV_FP8)
    return fail(PBSA_ERR_UNSUPPORTED, "attn_fwd_fp8 takes an FP8 cache (kv_format PBSA_KV_FP8)");
  PBSA_TRY(check_cache(cache, dims));
  PBSA_TRY(check_tok(q, "q", dims->head_dim));
  PBSA_TRY(check_tok(chunk_k, "chunk_k", dims->head_dim));
  PBSA_TRY(check_tok(chunk_v, "chunk_v", dims->head_dim));
  PBSA_TRY(check_tok(o, "o", dims->head_dim));
  const int64_t ctok = int64_t{dims->chunk_frames} * dims->frame_tokens;
  const int64_t list = int64_t{dims->capacity} + int64_t{dims->chunk_frames} * pbsa::nb_of(*dims) +
                       2 * int64_t{dims->topk};
  if (list > pbsa::kAttnListCap)
    return fail(PBSA_ERR_UNSUPPORTED, "capacity + chunk blocks + 2*topk = %lld exceeds %d",
                static_cast<long long>(list), pbsa::kAttnListCap);
  PBSA_TRY(check_span(q, "q", ctok, dims->head_dim));
  PBSA_TRY(check_span(chunk_k, "chunk_k", ctok, dims->head_dim));
  PBSA_TRY(check_span(chunk_v, "chunk_v", ctok, dims->head_dim));
  if (!sel || !lse) return fail(PBSA_ERR_NULL, "sel and lse are required");
  const size_t need = pbsa::attn_fwd_f8_workspace(*dims);
  if (!workspace || workspace_bytes < need)
    return fail(PBSA_ERR_WORKSPACE, "attn_fwd_fp8 needs %zu workspace bytes (got %zu)", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (reinterpret_cast<uintptr_t>(workspace) % 16)
    return fail(PBSA_ERR_ALIGN, "workspace must be 16-byte aligned");
  return hip_status(pbsa::launch_attn_fwd_f8(*dims, pbsa::tok_in(q), *cache,
                                             pbsa::tok_in(chunk_k), pbsa::tok_in(chunk_v), sel,
                                             pbsa::tok_out(o), lse, workspace,
                                             stream_of(stream)),
                    "attn_fwd_fp8");
}

}  // extern "C"

namespace pbsa {
namespace api {

pbsa_status check_memory_ws(const pbsa_dims* dims, const pbsa_cache* cache, void* workspace,
                            size_t workspace_bytes, const char* name) {
  const size_t need = pbsa::memory_update_workspace(*dims);
  if (!workspace || workspace_bytes < need)
    return fail(PBSA_ERR_WORKSPACE, "%s needs %zu workspace bytes (got %zu)", name, need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (cache->chunk_index > (int64_t{1} << 40) / (dims->chunk_frames * pbsa::nb_of(*dims)))
    return fail(PBSA_ERR_STATE, "chunk_index out of range");
  return PBSA_OK;
}

pbsa_status check_chunk_args(const pbsa_dims* dims, const pbsa_chunk_args* a,
                             const pbsa_cache* cache) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  if (!a) return fail(PBSA_ERR_NULL, "args is NULL");
  if (a->passes < 1 || a->passes > PBSA_MAX_PASSES)
    return fail(PBSA_ERR_SHAPE, "passes must be in [1, %d]", PBSA_MAX_PASSES);
  const int64_t ctok = int64_t{dims->chunk_frames} * dims->frame_tokens;
  const int64_t list = int64_t{dims->capacity} + int64_t{dims->chunk_frames} * pbsa::nb_of(*dims) +
                       2 * int64_t{dims->topk};
  if (list > pbsa::kAttnListCap)
    return fail(PBSA_ERR_UNSUPPORTED, "capacity + chunk blocks + 2*topk = %lld exceeds %d",
                static_cast<long long>(list), pbsa::kAttnListCap);
  for (int p = 0; p < a->passes; ++p) {
    PBSA_TRY(check_tok(a->q[p], "q", dims->head_dim));
    PBSA_TRY(check_tok(a->k[p], "k", dims->head_dim));
    PBSA_TRY(check_tok(a->v[p], "v", dims->head_dim));
    PBSA_TRY(check_tok(a->o[p], "o", dims->head_dim));
    PBSA_TRY(check_span(a->k[p], "k", ctok, dims->head_dim));
    PBSA_TRY(check_span(a->v[p], "v", ctok, dims->head_dim));
    if (!a->lse[p]) return fail(PBSA_ERR_NULL, "lse of pass %d is NULL", p);
  }
  if (!a->scores || !a->sel) return fail(PBSA_ERR_NULL, "scores and sel are required");
  if (reinterpret_cast<uintptr_t>(a->q_rep) % 16)
    return fail(PBSA_ERR_ALIGN, "q_rep must be 16-byte aligned");
  if (a->fp8_arithmetic) {
    if (dims->kv_format != PBSA_KV_FP8)
      return fail(PBSA_ERR_UNSUPPORTED, "fp8_arithmetic needs an FP8 cache (kv_format PBSA_KV_FP8)");
    for (int p = 0; p < a->passes; ++p) PBSA_TRY(check_span(a->q[p], "q", ctok, dims->head_dim));
    const size_t need = pbsa::attn_fwd_f8_workspace(*dims);
    if (!a->attn_workspace || a->attn_workspace_bytes < need)
      return fail(PBSA_ERR_WORKSPACE, "chunk_step with fp8_arithmetic needs %zu attn_workspace "
                  "bytes (got %zu)", need,
                  a->attn_workspace ? a->attn_workspace_bytes : static_cast<size_t>(0));
    if (reinterpret_cast<uintptr_t>(a->attn_workspace) % 16)
      return fail(PBSA_ERR_ALIGN, "attn_workspace must be 16-byte aligned");
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(a->workspace),
                    w1 = w0 + a->workspace_bytes;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(a->attn_workspace), x1 = x0 + need;
    if (x0 < w1 && w0 < x1)
      return fail(PBSA_ERR_WORKSPACE, "attn_workspace overlaps workspace");
  }
  return check_memory_ws(dims, cache, a->workspace, a->workspace_bytes, "chunk_step");
}

}  // namespace api
}  // namespace pbsa

extern "C" {

pbsa_status pbsa_memory_select(const pbsa_dims* dims, const float* scores,
                               const pbsa_cache* cache, void* workspace, size_t workspace_bytes,
                               void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  if (!scores) return fail(PBSA_ERR_NULL, "scores is required");
  PBSA_TRY(check_memory_ws(dims, cache, workspace, workspace_bytes, "memory_select"));
  return hip_status(pbsa::launch_memory_select(*dims, scores, *cache, workspace, true,
                                               stream_of(stream)),
                    "memory_select");
}

pbsa_status pbsa_memory_apply(const pbsa_dims* dims, pbsa_cache* cache, pbsa_tensor chunk_k,
                              pbsa_tensor chunk_v, const float* chunk_rep, void* workspace,
                              size_t workspace_bytes, void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  PBSA_TRY(check_tok(chunk_k, "chunk_k", dims->head_dim));
  PBSA_TRY(check_tok(chunk_v, "chunk_v", dims->head_dim));
  PBSA_TRY(check_memory_ws(dims, cache, workspace, workspace_bytes, "memory_apply"));
  pbsa_status st = hip_status(
      pbsa::launch_memory_apply(*dims, *cache, pbsa::tok_in(chunk_k), pbsa::tok_in(chunk_v),
                                chunk_rep, workspace, stream_of(stream)),
      "memory_apply");
  if (st == PBSA_OK) cache->chunk_index += 1;
  return st;
}

pbsa_status pbsa_memory_update(const pbsa_dims* dims, const float* scores, pbsa_cache* cache,
                               pbsa_tensor chunk_k, pbsa_tensor chunk_v, const float* chunk_rep,
                               void* workspace, size_t workspace_bytes, void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  PBSA_TRY(check_tok(chunk_k, "chunk_k", dims->head_dim));
  PBSA_TRY(check_tok(chunk_v, "chunk_v", dims->head_dim));
  if (!scores) return fail(PBSA_ERR_NULL, "scores is required");
  PBSA_TRY(check_memory_ws(dims, cache, workspace, workspace_bytes, "memory_update"));
  pbsa_status st = hip_status(
      pbsa::launch_memory_update(*dims, scores, *cache, pbsa::tok_in(chunk_k),
                                 pbsa::tok_in(chunk_v), chunk_rep, workspace, stream_of(stream)),
      "memory_update");
  if (st == PBSA_OK) cache->chunk_index += 1;
  return st;
}

pbsa_status pbsa_memory_update_noalloc(const pbsa_dims* dims, const float* scores,
                                       pbsa_cache* cache, pbsa_tensor chunk_k,
                                       pbsa_tensor chunk_v, const float* chunk_rep,
                                       void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  PBSA_TRY(check_tok(chunk_k, "chunk_k", dims->head_dim));
  PBSA_TRY(check_tok(chunk_v, "chunk_v", dims->head_dim));
  if (!scores) return fail(PBSA_ERR_NULL, "scores is required");
  const size_t need = pbsa::memory_update_workspace(*dims);
  if (need > pbsa::kMemoryScratchBytes)
    return fail(PBSA_ERR_UNSUPPORTED,
                "memory_update_noalloc: these dims need %zu scratch bytes, the library holds %zu "
                "(use pbsa_memory_update with a workspace)",
                need, pbsa::kMemoryScratchBytes);
  void* ws = nullptr;
  pbsa_status st = hip_status(pbsa::memory_scratch(&ws), "memory_update_noalloc scratch");
  if (st != PBSA_OK) return st;
  PBSA_TRY(check_memory_ws(dims, cache, ws, need, "memory_update_noalloc"));
  st = hip_status(pbsa::launch_memory_update(*dims, scores, *cache, pbsa::tok_in(chunk_k),
                                             pbsa::tok_in(chunk_v), chunk_rep, ws,
                                             stream_of(stream)),
                  "memory_update_noalloc");
  if (st == PBSA_OK) cache->chunk_index += 1;
  return st;
}

pbsa_status pbsa_score_topk_2lvl(const pbsa_dims* dims, int32_t chunks, int32_t top_frames,
                                 const int32_t* k_per_chunk, const float* q_rep,
                                 const float* block_rep, const float* frame_rep,
                                 int32_t max_sel, int32_t* sel, int32_t* nsel, void* stream) {
  PBSA_TRY(check_dims(dims, 1));
  if (chunks < 1 || chunks > kMaxChunks)
    return fail(PBSA_ERR_SHAPE, "chunks must be in [1, %d]", kMaxChunks);
  if (top_frames < 0) return fail(PBSA_ERR_SHAPE, "top_frames must be >= 0");
  if (!k_per_chunk || !q_rep || !block_rep || !frame_rep || !sel || !nsel)
    return fail(PBSA_ERR_NULL, "a two-level selection buffer is NULL");
  const int nb = pbsa::nb_of(*dims);
  if (max_sel < dims->chunk_frames * nb)
    return fail(PBSA_ERR_SHAPE, "max_sel must be >= chunk_frames * blocks per frame");
  for (int i = 1; i < chunks; ++i)
    if (k_per_chunk[i] < 1 || k_per_chunk[i] > max_sel)
      return fail(PBSA_ERR_SHAPE, "k_per_chunk[%d] = %d outside [1, max_sel]", i, k_per_chunk[i]);
  {
    const int64_t frames_total = static_cast<int64_t>(chunks) * dims->chunk_frames;
    const int64_t fr_max = std::min<int64_t>(int64_t{top_frames} + 2 + dims->chunk_frames, frames_total);
    if (fr_max * nb > 1024 || frames_total > 256)
      return fail(PBSA_ERR_UNSUPPORTED,
                  "two-level selection supports <= 256 clip frames and <= 1024 candidate blocks");
  }
  return hip_status(pbsa::launch_score_topk_2lvl(*dims, chunks, top_frames, k_per_chunk, q_rep,
                                                 block_rep, frame_rep, max_sel, sel, nsel,
                                                 stream_of(stream)),
                    "score_topk_2lvl");
}

pbsa_status pbsa_attn_fwd_2lvl(const pbsa_dims* dims, int32_t chunks, pbsa_tensor q,
                               pbsa_tensor k, pbsa_tensor v, const int32_t* sel,
                               const int32_t* nsel, int32_t max_sel, pbsa_tensor o, float* lse,
                               void* stream) {
  PBSA_TRY(check_dims(dims, 1));
  if (chunks < 1) return fail(PBSA_ERR_SHAPE, "chunks must be >= 1");
  PBSA_TRY(check_tok(q, "q", dims->head_dim));
  PBSA_TRY(check_tok(k, "k", dims->head_dim));
  PBSA_TRY(check_tok(v, "v", dims->head_dim));
  PBSA_TRY(check_tok(o, "o", dims->head_dim));
  if (!sel || !nsel || !lse) return fail(PBSA_ERR_NULL, "sel, nsel and lse are required");
  if (max_sel < 1) return fail(PBSA_ERR_SHAPE, "max_sel must be >= 1");
  if (2 * int64_t{max_sel} > pbsa::kAttnListCap)
    return fail(PBSA_ERR_UNSUPPORTED, "max_sel must be <= %d", pbsa::kAttnListCap / 2);
  const int64_t ctok = int64_t{chunks} * dims->chunk_frames * dims->frame_tokens;
  PBSA_TRY(check_span(k, "k", ctok, dims->head_dim));
  PBSA_TRY(check_span(v, "v", ctok, dims->head_dim));
  return hip_status(pbsa::launch_attn_fwd_2lvl(*dims, chunks, pbsa::tok_in(q), pbsa::tok_in(k),
                                               pbsa::tok_in(v), sel, nsel, max_sel,
                                               pbsa::tok_out(o), lse, stream_of(stream)),
                    "attn_fwd_2lvl");
}

pbsa_status pbsa_attn_bwd(const pbsa_dims* dims, int32_t chunks, pbsa_tensor q, pbsa_tensor k,
                          pbsa_tensor v, pbsa_tensor o, const float* lse, pbsa_tensor dout,
                          const int32_t* sel, const int32_t* nsel, int32_t max_sel,
                          pbsa_tensor dq, pbsa_tensor dk, pbsa_tensor dv, void* workspace,
                          size_t workspace_bytes, void* stream) {
  PBSA_TRY(check_dims(dims, 1));
  if (chunks < 1) return fail(PBSA_ERR_SHAPE, "chunks must be >= 1");
  PBSA_TRY(check_tok(q, "q", dims->head_dim));
  PBSA_TRY(check_tok(k, "k", dims->head_dim));
  PBSA_TRY(check_tok(v, "v", dims->head_dim));
  PBSA_TRY(check_tok(o, "o", dims->head_dim));
  PBSA_TRY(check_tok(dout, "dout", dims->head_dim));
  PBSA_TRY(check_tok(dq, "dq", dims->head_dim));
  PBSA_TRY(check_tok(dk, "dk", dims->head_dim));
  PBSA_TRY(check_tok(dv, "dv", dims->head_dim));
  const int64_t ttok = int64_t{chunks} * dims->chunk_frames * dims->frame_tokens;
  PBSA_TRY(check_span(q, "q", ttok, dims->head_dim));
  PBSA_TRY(check_span(k, "k", ttok, dims->head_dim));
  PBSA_TRY(check_span(v, "v", ttok, dims->head_dim));
  PBSA_TRY(check_span(dout, "dout", ttok, dims->head_dim));
  if (!lse || !sel || !nsel) return fail(PBSA_ERR_NULL, "lse, sel and nsel are required");
  if (max_sel < 1) return fail(PBSA_ERR_SHAPE, "max_sel must be >= 1");
  if (max_sel > pbsa::kAttnListCap / 2)
    return fail(PBSA_ERR_UNSUPPORTED, "max_sel must be <= %d", pbsa::kAttnListCap / 2);
  const size_t need = pbsa::attn_bwd_workspace(*dims, chunks, max_sel);
  if (!workspace || workspace_bytes < need)
    return fail(PBSA_ERR_WORKSPACE, "attn_bwd needs %zu workspace bytes (got %zu)", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  return hip_status(pbsa::launch_attn_bwd(*dims, chunks, pbsa::tok_in(q), pbsa::tok_in(k),
                                          pbsa::tok_in(v), pbsa::tok_in(o), lse,
                                          pbsa::tok_in(dout), sel, nsel, max_sel,
                                          pbsa::tok_out(dq), pbsa::tok_out(dk),
                                          pbsa::tok_out(dv), workspace, stream_of(stream)),
                    "attn_bwd");
}

pbsa_status pbsa_attn_bwd_persistent(const pbsa_dims* dims, pbsa_tensor q,
                                     const pbsa_cache* cache, pbsa_tensor chunk_k,
                                     pbsa_tensor chunk_v, const int32_t* sel, pbsa_tensor o,
                                     const float* lse, pbsa_tensor dout, pbsa_tensor dq,
                                     pbsa_tensor dk, pbsa_tensor dv, void* dk_cache,
                                     void* dv_cache, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  if (dims->kv_format != PBSA_KV_BF16)
    return fail(PBSA_ERR_UNSUPPORTED, "attn_bwd_persistent takes a bf16 cache");
  const char* names[] = {"q", "chunk_k", "chunk_v", "o", "dout", "dq", "dk", "dv"};
  const pbsa_tensor* ts[] = {&q, &chunk_k, &chunk_v, &o, &dout, &dq, &dk, &dv};
  const int64_t ctok = int64_t{dims->chunk_frames} * dims->frame_tokens;
  for (int i = 0; i < 8; ++i) {
    PBSA_TRY(check_tok(*ts[i], names[i], dims->head_dim));
    if (i < 5) PBSA_TRY(check_span(*ts[i], names[i], ctok, dims->head_dim));
  }
  if (!sel || !lse || !dk_cache || !dv_cache)
    return fail(PBSA_ERR_NULL, "sel, lse, dk_cache and dv_cache are required");
  if (reinterpret_cast<uintptr_t>(dk_cache) % 16 || reinterpret_cast<uintptr_t>(dv_cache) % 16)
    return fail(PBSA_ERR_ALIGN, "dk_cache and dv_cache must be 16-byte aligned");
  const int64_t list = int64_t{dims->capacity} + dims->topk +
                       int64_t{dims->chunk_frames} * pbsa::nb_of(*dims);
  if (list > pbsa::kAttnListCap / 2)
    return fail(PBSA_ERR_UNSUPPORTED, "capacity + topk + chunk blocks = %lld exceeds %d",
                static_cast<long long>(list), pbsa::kAttnListCap / 2);
  const size_t need = pbsa::attn_bwd_persistent_workspace(*dims);
  if (!workspace || workspace_bytes < need)
    return fail(PBSA_ERR_WORKSPACE, "attn_bwd_persistent needs %zu workspace bytes (got %zu)",
                need, workspace ? workspace_bytes : static_cast<size_t>(0));
  return hip_status(pbsa::launch_attn_bwd_persistent(
                        *dims, pbsa::tok_in(q), *cache, pbsa::tok_in(chunk_k),
                        pbsa::tok_in(chunk_v), sel, pbsa::tok_in(o), lse, pbsa::tok_in(dout),
                        pbsa::tok_out(dq), pbsa::tok_out(dk), pbsa::tok_out(dv),
                        static_cast<uint16_t*>(dk_cache), static_cast<uint16_t*>(dv_cache),
                        workspace, stream_of(stream)),
                    "attn_bwd_persistent");
}

// ---- measurement probes (pbsa_probe.h)

pbsa_status pbsa_probe_fp8_decode(const uint8_t* codes, const float* scales, uint16_t* out,
                                  int32_t n, void* stream) {
  if (!codes || !scales || !out) return fail(PBSA_ERR_NULL, "codes, scales and out are required");
  if (n < 0 || n % 16) return fail(PBSA_ERR_SHAPE, "n must be a non-negative multiple of 16");
  if (reinterpret_cast<uintptr_t>(codes) % 16 || reinterpret_cast<uintptr_t>(out) % 16)
    return fail(PBSA_ERR_ALIGN, "codes and out must be 16-byte aligned");
  return hip_status(pbsa::launch_probe_fp8_decode(codes, scales, out, n, stream_of(stream)),
                    "probe_fp8_decode");
}

int64_t pbsa_probe_mfma_flop(int64_t iters) {
  return iters < 1 ? 0 : iters * 512 * 4 * 4 * (2 * 32 * 32 * 16);
}

pbsa_status pbsa_probe_mfma(int64_t iters, float* out, void* stream) {
  if (!out) return fail(PBSA_ERR_NULL, "out is NULL");
  if (iters < 1) return fail(PBSA_ERR_SHAPE, "iters must be >= 1");
  return hip_status(pbsa::launch_probe_mfma(iters, out, stream_of(stream)), "probe_mfma");
}

pbsa_status pbsa_probe_gather(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                              pbsa_tensor chunk_k, pbsa_tensor chunk_v, const int32_t* sel,
                              void* stream) {
  PBSA_TRY(check_dims(dims, 0));
  PBSA_TRY(check_cache(cache, dims));
  if (dims->kv_format != PBSA_KV_BF16)
    return fail(PBSA_ERR_UNSUPPORTED, "probe_gather takes a bf16 cache");
  PBSA_TRY(check_tok(q, "q", dims->head_dim));
  PBSA_TRY(check_tok(chunk_k, "chunk_k", dims->head_dim));
  PBSA_TRY(check_tok(chunk_v, "chunk_v", dims->head_dim));
  if (!sel) return fail(PBSA_ERR_NULL, "sel is required");
  const int64_t ctok = int64_t{dims->chunk_frames} * dims->frame_tokens;
  const int64_t list = int64_t{dims->capacity} + int64_t{dims->chunk_frames} * pbsa::nb_of(*dims) +
                       2 * int64_t{dims->topk};
  if (list > pbsa::kAttnListCap)
    return fail(PBSA_ERR_UNSUPPORTED, "capacity + chunk blocks + 2*topk = %lld exceeds %d",
                static_cast<long long>(list), pbsa::kAttnListCap);
  PBSA_TRY(check_span(chunk_k, "chunk_k", ctok, dims->head_dim));
  PBSA_TRY(check_span(chunk_v, "chunk_v", ctok, dims->head_dim));
  return hip_status(pbsa::launch_attn_fwd_persistent(*dims, pbsa::tok_in(q), *cache,
                                                     pbsa::tok_in(chunk_k),
                                                     pbsa::tok_in(chunk_v), sel,
                                                     pbsa::TokOut{nullptr, 0, 0}, nullptr,
                                                     stream_of(stream), true),
                    "probe_gather");
}

}  // extern "C"
