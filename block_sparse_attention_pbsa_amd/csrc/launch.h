// Internal launchers: argument checking happens in api.cpp, these only enqueue kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pbsa.h"
#include "common.h"

namespace pbsa {

inline TokIn tok_in(const pbsa_tensor& t) {
  return TokIn{static_cast<const uint16_t*>(t.data), t.token_stride, t.head_stride};
}
inline TokOut tok_out(const pbsa_tensor& t) {
  return TokOut{static_cast<uint16_t*>(t.data), t.token_stride, t.head_stride};
}

inline int nb_of(const pbsa_dims& d) { return (d.frame_tokens + d.block - 1) / d.block; }
inline int64_t slots_of(const pbsa_dims& d) {
  return static_cast<int64_t>(d.capacity) + static_cast<int64_t>(d.window_frames) * nb_of(d);
}

hipError_t launch_pool(const pbsa_dims& d, TokIn x, int frames, float* block_rep,
                       float* frame_rep, hipStream_t s);

hipError_t launch_cache_reset(const pbsa_dims& d, const pbsa_cache& c, hipStream_t s);

hipError_t launch_score_topk(const pbsa_dims& d, const float* q_rep, const pbsa_cache& c,
                             float* scores, int32_t* sel, hipStream_t s);

hipError_t launch_route(const pbsa_dims& d, TokIn q, float* q_rep, const pbsa_cache& c,
                        float* scores, int32_t* sel, hipStream_t s);

hipError_t launch_score_topk_2lvl(const pbsa_dims& d, int chunks, int top_frames,
                                  const int32_t* k_per_chunk, const float* q_rep,
                                  const float* block_rep, const float* frame_rep, int max_sel,
                                  int32_t* sel, int32_t* nsel, hipStream_t s);

hipError_t launch_attn_fwd_persistent(const pbsa_dims& d, TokIn q, const pbsa_cache& c,
                                      TokIn ck, TokIn cv, const int32_t* sel, TokOut o,
                                      float* lse, hipStream_t s, bool gather_only = false);

hipError_t launch_attn_fwd_fp8(const pbsa_dims& d, TokIn q, const pbsa_cache& c, TokIn ck,
                               TokIn cv, const int32_t* sel, TokOut o, float* lse,
                               hipStream_t s);

size_t attn_fwd_f8_workspace(const pbsa_dims& d);
hipError_t launch_attn_fwd_f8(const pbsa_dims& d, TokIn q, const pbsa_cache& c, TokIn ck,
                              TokIn cv, const int32_t* sel, TokOut o, float* lse,
                              void* workspace, hipStream_t s);

hipError_t launch_probe_mfma(int64_t iters, float* out, hipStream_t s);
hipError_t launch_probe_fp8_decode(const uint8_t* codes, const float* scales, uint16_t* out,
                                   int n, hipStream_t s);

hipError_t launch_attn_fwd_2lvl(const pbsa_dims& d, int chunks, TokIn q, TokIn k, TokIn v,
                                const int32_t* sel, const int32_t* nsel, int max_sel, TokOut o,
                                float* lse, hipStream_t s);

size_t attn_bwd_workspace(const pbsa_dims& d, int chunks, int max_sel);
size_t attn_bwd_persistent_workspace(const pbsa_dims& d);
hipError_t launch_attn_bwd_persistent(const pbsa_dims& d, TokIn q, const pbsa_cache& c,
                                      TokIn ck, TokIn cv, const int32_t* sel, TokIn o,
                                      const float* lse, TokIn dout, TokOut dq, TokOut dk,
                                      TokOut dv, uint16_t* dk_cache, uint16_t* dv_cache,
                                      void* ws, hipStream_t s);
hipError_t launch_attn_bwd(const pbsa_dims& d, int chunks, TokIn q, TokIn k, TokIn v, TokIn o,
                           const float* lse, TokIn dout, const int32_t* sel,
                           const int32_t* nsel, int max_sel, TokOut dq, TokOut dk, TokOut dv,
                           void* ws, hipStream_t s);

size_t memory_update_workspace(const pbsa_dims& d);
hipError_t launch_memory_select(const pbsa_dims& d, const float* scores, const pbsa_cache& c,
                                void* ws, bool beside, hipStream_t s);
hipError_t launch_memory_apply(const pbsa_dims& d, const pbsa_cache& c, TokIn ck, TokIn cv,
                               const float* chunk_rep, void* ws, hipStream_t s);
hipError_t launch_memory_update(const pbsa_dims& d, const float* scores, const pbsa_cache& c,
                                TokIn ck, TokIn cv, const float* chunk_rep, void* ws,
                                hipStream_t s);

// Size of the library-held workspace of pbsa_memory_update_noalloc, and its device address
// on the current device (looked up on first use per device).
constexpr size_t kMemoryScratchBytes = size_t{1} << 20;
hipError_t memory_scratch(void** ptr);

}  // namespace pbsa
