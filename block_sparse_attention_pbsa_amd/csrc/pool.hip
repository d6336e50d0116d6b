// Blockified compression: block and frame mean representatives of bf16 tokens.
//
// Sparse Forcing (gist.science) 2.C: every block of the latent gets one compressed
// representative; Light Forcing (papernotes.org), hierarchical sparse attention step 1:
// the compression is mean pooling at block and at frame level.
//
// HBM-bound: each token row is read once with 16-byte loads, a wave per block; a small
// second pass turns block means into frame means.  Accumulation is fp32.
#include "common.h"
#include "launch.h"

namespace pbsa {

// 1-D grid of ceil(frames*nb / 4) * H workgroups, head fastest (neighbouring workgroups
// read the same token rows' other heads, so the rows in flight are read whole), 256
// threads: wave w pools global block 4*(blockIdx.x / H) + w of head blockIdx.x % H.
// Lane l owns channels [8*(l % CH), +8) of rows l / CH, l / CH + RPI, ... (CH = D / 8
// chunks per row, RPI = 64 / CH rows per pass).
template <int D>
__global__ void __launch_bounds__(256) pool_blocks_kernel(TokIn x, int n, int nb, int nblocks,
                                                           float* __restrict__ block_rep) {
  constexpr int CH = D / 8;
  constexpr int RPI = 64 / CH;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int H = static_cast<int>(gridDim.x) / ((nblocks + 3) / 4);
  const int g = (static_cast<int>(blockIdx.x) / H) * 4 + w;
  const int h = static_cast<int>(blockIdx.x) % H;
  if (g >= nblocks) return;
  const int f = g / nb, j = g - f * nb;
  const int len = block_len(j, n);
  const int64_t t0 = static_cast<int64_t>(f) * n + static_cast<int64_t>(kBlock) * j;
  const uint16_t* base = x.p + h * x.hs + t0 * x.ts + 8 * (l % CH);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // all of the block's rows are requested before any is summed (64 / RPI loads in flight)
  u32x4 v[kBlock / RPI];
#pragma unroll
  for (int i = 0; i < kBlock / RPI; ++i) {
    const int row = l / CH + RPI * i;
    v[i] = row < len ? *reinterpret_cast<const u32x4*>(base + row * x.ts) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < kBlock / RPI; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(v[i][e] << 16);
      acc[2 * e + 1] += __uint_as_float(v[i][e] & 0xffff0000u);
    }
  // Combine the RPI row groups (lanes l, l + CH, l + 2CH, ...).
#pragma unroll
  for (int o = CH; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }
  if (l < CH) {
    const float inv = 1.f / static_cast<float>(len);
    float* out = block_rep + (static_cast<int64_t>(h) * nblocks + g) * D + 8 * l;
    reinterpret_cast<f32x4*>(out)[0] = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    reinterpret_cast<f32x4*>(out)[1] = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
}

// grid (frames, H), D threads: frame mean = sum_j (block mean_j * len_j) / n, i.e. the mean
// of the frame's tokens (not the mean of its block means: the tail block weighs less).
template <int D>
__global__ void pool_frames_kernel(const float* __restrict__ block_rep, int n, int nb,
                                   int frames, float* __restrict__ frame_rep) {
  const int f = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  const int nblocks = frames * nb;
  const float* s = block_rep + (static_cast<int64_t>(h) * nblocks + f * nb) * D + c;
  float acc = 0.f;
  int j = 0;
  // eight block means loaded before they are added (the order of the additions is kept)
  for (; j + 8 <= nb; j += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s[(j + u) * D];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u] * static_cast<float>(block_len(j + u, n));
  }
  for (; j < nb; ++j) acc += s[j * D] * static_cast<float>(block_len(j, n));
  frame_rep[(static_cast<int64_t>(h) * frames + f) * D + c] = acc / static_cast<float>(n);
}

hipError_t launch_pool(const pbsa_dims& d, TokIn x, int frames, float* block_rep,
                       float* frame_rep, hipStream_t s) {
  const int nb = nb_of(d);
  const int nblocks = frames * nb;
  if (nblocks == 0) return hipSuccess;
  dim3 grid(cdiv(nblocks, 4) * d.heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(pool_blocks_kernel<128>, grid, dim3(256), 0, s, x, d.frame_tokens, nb,
                       nblocks, block_rep);
  else
    hipLaunchKernelGGL(pool_blocks_kernel<64>, grid, dim3(256), 0, s, x, d.frame_tokens, nb,
                       nblocks, block_rep);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !frame_rep) return e;
  dim3 g2(frames, d.heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(pool_frames_kernel<128>, g2, dim3(128), 0, s, block_rep, d.frame_tokens,
                       nb, frames, frame_rep);
  else
    hipLaunchKernelGGL(pool_frames_kernel<64>, g2, dim3(64), 0, s, block_rep, d.frame_tokens,
                       nb, frames, frame_rep);
  return hipGetLastError();
}

}  // namespace pbsa
