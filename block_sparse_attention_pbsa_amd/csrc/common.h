// Device-side helpers shared by the gfx950 kernels of libpbsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbsa {

constexpr int kBlock = 64;  // tokens per block (the only block size built)

// Block-list entries the attention forward keeps per workgroup (persistent mode:
// capacity + chunk blocks + 2 * topk; two-level mode: 2 * max_sel).
constexpr int kAttnListCap = 3072;

// A bf16 token tensor (see pbsa_tensor): base, token stride and head stride in elements.
struct TokIn {
  const uint16_t* p;
  int64_t ts;  // token stride (elements)
  int64_t hs;  // head stride (elements)
};
struct TokOut {
  uint16_t* p;
  int64_t ts;
  int64_t hs;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (round to nearest even) with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand layout (wave64): lane l supplies row/col
// (l % 32) and the 8 contraction elements [8*(l/32), 8*(l/32)+8).  Result: lane l holds
// column (l % 32) and rows 8*(i/4) + 4*(l/32) + (i%4) for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Sort key for "score descending, id ascending": order-preserving float bits in the high
// word, ~id in the low word.  NaN scores order as -inf.  Key 0 sorts below every key.
__device__ __forceinline__ uint64_t rank_key(float score, int id) {
  if (score != score) score = -INFINITY;
  const uint32_t b = __float_as_uint(score);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(id));
}
__device__ __forceinline__ int rank_key_id(uint64_t k) {
  return static_cast<int>(~static_cast<uint32_t>(k & 0xffffffffu));
}

// Ceil division.
__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Token range of block j inside a frame of n tokens.
__host__ __device__ __forceinline__ int block_len(int j, int n) {
  int a = kBlock * j;
  int b = a + kBlock < n ? a + kBlock : n;
  return b - a;
}

}  // namespace pbsa
