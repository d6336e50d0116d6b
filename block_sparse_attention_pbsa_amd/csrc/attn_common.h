// Pieces shared by the attention kernels (forward, dQ pass, dK/dV pass).
#pragma once

#include "common.h"
#include "launch.h"

namespace pbsa {

constexpr float kLog2e = 1.4426950408889634f;

// Row-major LDS tile [64][D + 8] and channel-major tile [D][64 + 4]; the padding staggers
// rows across LDS banks for the 16-byte row reads and the 8-byte column reads.
template <int D>
struct Lds {
  static constexpr int RS = D + 8;       // row-major row pitch (elements)
  static constexpr int CS = kBlock + 4;  // channel-major row pitch (elements)
  static constexpr int ROWS = kBlock * RS;
  static constexpr int COLS = D * CS;
};

// A 64-row x D-channel bf16 tile staged through registers by a 128-thread workgroup.
// Thread t owns channels [8*(t % CH), +8) of rows 4*KG*p + 4*(t / CH) + i (i < 4): each
// load instruction reads whole 256-byte rows, and each thread holds 4 consecutive rows of
// one channel chunk, which it can write row-major or transposed.
template <int D>
struct Tile {
  static constexpr int CH = D / 8;
  static constexpr int KG = 128 / CH;
  static constexpr int NP = kBlock / (4 * KG);
  u32x4 r[NP][4];

  __device__ __forceinline__ void load(const uint16_t* p, int64_t stride, int len, int t) {
    const int cc = t % CH, kg = t / CH;
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * KG * q + 4 * kg + i;
        r[q][i] = row < len ? *reinterpret_cast<const u32x4*>(p + row * stride + 8 * cc)
                            : u32x4{0, 0, 0, 0};
      }
  }

  __device__ __forceinline__ void store_rows(uint16_t* lds, int t) const {
    const int cc = t % CH, kg = t / CH;
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * KG * q + 4 * kg + i;
        *reinterpret_cast<u32x4*>(lds + row * Lds<D>::RS + 8 * cc) = r[q][i];
      }
  }

  __device__ __forceinline__ void store_cols(uint16_t* lds, int t) const {
    const int cc = t % CH, kg = t / CH;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int row0 = 4 * KG * q + 4 * kg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint32_t a, b;
        if (e & 1) {
          a = (r[q][0][w] >> 16) | (r[q][1][w] & 0xffff0000u);
          b = (r[q][2][w] >> 16) | (r[q][3][w] & 0xffff0000u);
        } else {
          a = (r[q][0][w] & 0xffffu) | (r[q][1][w] << 16);
          b = (r[q][2][w] & 0xffffu) | (r[q][3][w] << 16);
        }
        *reinterpret_cast<u32x2*>(lds + (8 * cc + e) * Lds<D>::CS + row0) = u32x2{a, b};
      }
    }
  }
};

// MFMA operand reads from LDS for a wave whose lane l has half h2 = l / 32, c32 = l % 32.
// Row-major tile, rows 32*tile + c32, contraction over channels (k-step s: channels
// 16s + 8*h2 + [0, 8)).
template <int D>
__device__ __forceinline__ u32x4 rd_rows(const uint16_t* lds, int tile, int s, int c32, int h2) {
  return *reinterpret_cast<const u32x4*>(lds + (32 * tile + c32) * Lds<D>::RS + 16 * s + 8 * h2);
}
// Channel-major tile, channel rows 32*dt + c32, contraction over 16 rows of step t4 in the
// order produced by a 32x32 accumulator: rows 16*t4 + 4*h2 + [0,4) then 16*t4 + 8 + 4*h2 +
// [0,4).
template <int D>
__device__ __forceinline__ u32x4 rd_cols(const uint16_t* lds, int dt, int t4, int c32, int h2) {
  const uint16_t* p = lds + (32 * dt + c32) * Lds<D>::CS + 16 * t4 + 4 * h2;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
// B/A operand from two 32-row accumulator tiles: k-step t4 (16 rows) packed to bf16 in the
// order rd_cols expects.
__device__ __forceinline__ u32x4 pack_step(const f32x16* acc, int t4) {
  const int kt = t4 >> 1, rb = 8 * (t4 & 1);
  u32x4 pb;
#pragma unroll
  for (int e = 0; e < 4; ++e) pb[e] = pack_bf16x2(acc[kt][rb + 2 * e], acc[kt][rb + 2 * e + 1]);
  return pb;
}
// Row index (0..31 within a 32-row accumulator tile) of accumulator register r in half h2.
__device__ __forceinline__ int acc_row(int r, int h2) { return 8 * (r >> 2) + 4 * h2 + (r & 3); }

// Register-resident operand: D channels of row `row` (< len) in k-step chunks.
template <int D>
__device__ __forceinline__ void load_row_operand(u32x4* dst, const uint16_t* p, int64_t stride,
                                                 int row, int len, int h2) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    dst[s] = row < len ? *reinterpret_cast<const u32x4*>(p + row * stride + 16 * s + 8 * h2)
                       : u32x4{0, 0, 0, 0};
}

// Block addressing inside a frame-major token tensor.
__device__ __forceinline__ int64_t block_token0(int g, int nb, int n) {
  const int f = g / nb, j = g - f * nb;
  return static_cast<int64_t>(f) * n + kBlock * j;
}

}  // namespace pbsa
