// Measurement probe: the MFMA rate of v_mfma_f32_32x32x16_bf16 with independent
// accumulators on every SIMD (the instruction the attention kernels use).
#include "attn_common.h"
#include "launch.h"

namespace pbsa {

namespace {
constexpr int kProbeBlocks = 512, kProbeThreads = 256;
}

__global__ void __launch_bounds__(256) mfma_probe_kernel(int64_t iters, float* out) {
  const int t = blockIdx.x * kProbeThreads + threadIdx.x;
  // operands vary per lane (data-dependent power, as with real tiles)
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = 0x3c003c00u ^ ((t * 2654435761u + i * 40503u) & 0x007f007fu);
    b[i] = 0x3b803b80u ^ ((t * 2246822519u + i * 9973u) & 0x007f007fu);
  }
  f32x16 acc[4] = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[t] = s;
}

hipError_t launch_probe_mfma(int64_t iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, s, iters,
                     out);
  return hipGetLastError();
}

// Decodes codes[16 i .. 16 i + 16) with scale scales[i] through the FP8 attention's decode
// (decode_e4m3x16) into out (bf16 bits); one thread per 16 codes.
__global__ void fp8_decode_probe_kernel(const uint8_t* codes, const float* scales, uint16_t* out,
                                        int n16) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 raw = *reinterpret_cast<const u32x4*>(codes + 16 * static_cast<int64_t>(i));
  u32x4 lo, hi;
  decode_e4m3x16(raw, scales[i], lo, hi);
  *reinterpret_cast<u32x4*>(out + 16 * static_cast<int64_t>(i)) = lo;
  *reinterpret_cast<u32x4*>(out + 16 * static_cast<int64_t>(i) + 8) = hi;
}

hipError_t launch_probe_fp8_decode(const uint8_t* codes, const float* scales, uint16_t* out,
                                   int n, hipStream_t s) {
  const int n16 = n / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(fp8_decode_probe_kernel, dim3((n16 + 255) / 256), dim3(256), 0, s, codes,
                     scales, out, n16);
  return hipGetLastError();
}

}  // namespace pbsa
