// Argument checks and error text shared by the C entry points (api.cpp, step.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/pbsa.h"

#define PBSA_TRY(x)                   \
  do {                                \
    pbsa_status st__ = (x);           \
    if (st__ != PBSA_OK) return st__; \
  } while (0)

namespace pbsa {
namespace api {

// Sets the thread's error text and returns st.
pbsa_status fail(pbsa_status st, const char* fmt, ...);
// PBSA_OK (and clears the error text) for hipSuccess, else PBSA_ERR_HIP with HIP's text.
pbsa_status hip_status(hipError_t e, const char* where);
pbsa_status check_dims(const pbsa_dims* d, int mode);
pbsa_status check_tok(const pbsa_tensor& t, const char* name, int head_dim);
pbsa_status check_span(const pbsa_tensor& t, const char* name, int64_t tokens, int head_dim);
pbsa_status check_cache(const pbsa_cache* c, const pbsa_dims* d);
pbsa_status check_memory_ws(const pbsa_dims* dims, const pbsa_cache* cache, void* workspace,
                            size_t workspace_bytes, const char* name);
// Everything pbsa_chunk_step reads: dims, cache, every pass's tensors, the routing and
// update buffers.
pbsa_status check_chunk_args(const pbsa_dims* dims, const pbsa_chunk_args* a,
                             const pbsa_cache* cache);

}  // namespace api

hipError_t enqueue_chunk_step(const pbsa_dims& d, const pbsa_chunk_args& a, const pbsa_cache& c,
                              hipStream_t s, hipStream_t side, hipEvent_t fork, hipEvent_t join);

}  // namespace pbsa
