/* pbsa_probe.h — measurement probes of libpbsa (not part of the method).
 *
 * They give the measured ceilings that the method's kernels are compared with: the MFMA
 * rate this GPU sustains on the instruction the attention uses, and the gather of the
 * persistent attention without its math.  Same conventions as pbsa.h: device pointers,
 * asynchronous on `stream`, arguments checked before anything is enqueued, status codes
 * and pbsa_last_error() as there.
 */
#ifndef PBSA_PROBE_H_
#define PBSA_PROBE_H_

#include <stdint.h>

#include "pbsa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Independent chains of v_mfma_f32_32x32x16_bf16 on every SIMD: 512 workgroups of 256
 * threads (two waves per SIMD on a 256-CU MI355X), each wave `iters` x 4 MFMAs.
 * pbsa_probe_mfma_flop(iters) is the work done (2*32*32*16 FLOP per MFMA).  out: device
 * fp32, at least 131072 entries (one per thread, written so the work is not elided).
 * iters >= 1. */
pbsa_status pbsa_probe_mfma(int64_t iters, float* out, void* stream);
int64_t pbsa_probe_mfma_flop(int64_t iters);

/* The gathers of pbsa_attn_fwd (same arguments, same lists, waits and barriers) with the
 * math and the output left out: every persistent block, chunk block and routed window
 * block a workgroup of two query blocks attends is moved from HBM/L2 into LDS once per
 * step.  Nothing is written. */
pbsa_status pbsa_probe_gather(const pbsa_dims* dims, pbsa_tensor q, const pbsa_cache* cache,
                              pbsa_tensor chunk_k, pbsa_tensor chunk_v, const int32_t* sel,
                              void* stream);

/* The FP8 cache's decode as the attention runs it: out[16 i + j] = bf16 bits of
 * E4M3(codes[16 i + j]) * scales[i] for n codes (n a multiple of 16; codes 16-byte
 * aligned).  For checking the decode against the format's definition. */
pbsa_status pbsa_probe_fp8_decode(const uint8_t* codes, const float* scales, uint16_t* out,
                                  int32_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PBSA_PROBE_H_ */
