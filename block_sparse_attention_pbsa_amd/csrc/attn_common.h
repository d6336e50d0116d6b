// Pieces shared by the attention kernels (forward, dQ pass, dK/dV pass).
#pragma once

#include "common.h"
#include "launch.h"

namespace pbsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// LDS tile layouts.  Row-major tiles keep 16-byte chunks of a row; for head_dim 128 a row is
// exactly 256 bytes and chunk c of row r sits at chunk position c ^ swz(r), with
// swz(r) = 4*(r % 4) + (r / 4) % 4.  That permutation keeps both access patterns free of
// bank conflicts: 16 consecutive rows reading the same logical chunk (K operand) hit 16
// different positions, and 4 consecutive rows reading an aligned group of 4 chunks (the
// transposing V read) land in 4 different groups.  For head_dim 64 rows are padded by 16
// bytes instead.
template <int D>
struct Lds {
  static constexpr bool SWZ = (D == 128);
  static constexpr int RS = SWZ ? D : D + 8;  // row-major row pitch (elements)
  static constexpr int ROWS = kBlock * RS;
  // element offset of (row, channel chunk c) in a row-major tile
  __host__ __device__ static constexpr int chunk(int row, int c) {
    return row * RS + 8 * (SWZ ? (c ^ (((row & 3) << 2) | ((row >> 2) & 3))) : c);
  }
};

// An R-row x D-channel bf16 tile (R = 64 or 32) staged through registers by NT threads.
// Thread t owns channels [8*(t % CH), +8) of RG consecutive rows RG*KG*q + RG*(t / CH) + i
// (i < RG): each load instruction reads whole 2*D-byte rows, and each thread holds RG
// consecutive rows of one channel chunk.
template <int D, int NT = 128, int R = kBlock>
struct Tile {
  static constexpr int CH = D / 8;                       // 16-byte chunks per row
  static constexpr int CPT = R * CH / NT;                // chunks per thread
  static constexpr int RG = CPT < 4 ? CPT : 4;           // consecutive rows per group
  static constexpr int NP = CPT / RG;                    // row groups per thread
  static constexpr int KG = NT / CH;                     // row groups per pass
  static_assert(CPT >= 1 && RG * KG * NP == R, "unsupported tile split");
  u32x4 r[NP][RG];

  // Rows [0, len) from p (row stride stride_b bytes; p wave-uniform) through a buffer
  // resource whose extent is len rows: rows past len read as zero with no branch, and each
  // row group takes one 32-bit lane offset plus scalar row offsets (callers keep 64 rows
  // of offsets under 2^32).
  __device__ __forceinline__ void load(const uint16_t* p, uint32_t stride_b, int len, int t) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p), 0, static_cast<uint32_t>(len) * stride_b, 0x00020000);
    const int cc = t % CH, kg = t / CH;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const uint32_t voff = (RG * KG * q + RG * kg) * stride_b + 16u * cc;
#pragma unroll
      for (int i = 0; i < RG; ++i)
        r[q][i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i * stride_b, 0));
    }
  }

  __device__ __forceinline__ void store_rows(uint16_t* lds, int t) const {
    const int cc = t % CH, kg = t / CH;
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int row = RG * KG * q + RG * kg + i;
        *reinterpret_cast<u32x4*>(lds + Lds<D>::chunk(row, cc)) = r[q][i];
      }
  }
};

// MFMA operand reads from LDS for a wave whose lane l has half h2 = l / 32, c32 = l % 32.
// Row-major tile, rows 32*tile + c32, contraction over channels (k-step s: channels
// 16s + 8*h2 + [0, 8)).
template <int D>
__device__ __forceinline__ u32x4 rd_rows(const uint16_t* lds, int tile, int s, int c32, int h2) {
  return *reinterpret_cast<const u32x4*>(lds + Lds<D>::chunk(32 * tile + c32, 2 * s + h2));
}
// Channel-major view of a ROW-major tile through gfx950's transposing LDS read
// (ds_read_b64_tr_b16).  Within each 16-lane group the instruction returns to lane i the
// element (4e + i/4, i%4) of the 16 x 4 matrix formed by the lanes' 64-bit reads, e = 0..3.
// Lane j = 4e + m of a group therefore addresses row K0 + e, channels D0 + 4m .. +3, and
// lane i receives rows K0..K0+3 of channel D0 + i.  The operand a wave gets: lane l holds
// channel 32*dt + l % 32, contraction rows 16*t4 + 4*(l / 32) + [0,4) then the same + 8,
// the row order of a 32x32 accumulator.
typedef short s16x4_ __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_ lds_s16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
template <int D>
__device__ __forceinline__ u32x4 rd_rows_tr(const uint16_t* lds, int dt, int t4, int l) {
  const int g = l >> 4, i = l & 15;
  const int d0 = 32 * dt + 16 * (g & 1);
  const int k0 = 16 * t4 + 4 * (g >> 1);
  const int ch = d0 + 4 * (i & 3);  // this lane's 4 channels
  const int row = k0 + (i >> 2);
  const int off_lo = Lds<D>::chunk(row, ch >> 3) + (ch & 4);
  const int off_hi = Lds<D>::chunk(row + 8, ch >> 3) + (ch & 4);
  lds_u16* p = (lds_u16*)(lds);  // generic -> LDS address space
  const s16x4_ lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + off_lo));
  const s16x4_ hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + off_hi));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// B/A operand from two 32-row accumulator tiles: k-step t4 (16 rows) packed to bf16 in the
// order rd_rows_tr produces.
__device__ __forceinline__ u32x4 pack_step(const f32x16* acc, int t4) {
  const int kt = t4 >> 1, rb = 8 * (t4 & 1);
  u32x4 pb;
#pragma unroll
  for (int e = 0; e < 4; ++e) pb[e] = pack_bf16x2(acc[kt][rb + 2 * e], acc[kt][rb + 2 * e + 1]);
  return pb;
}
// Row index (0..31 within a 32-row accumulator tile) of accumulator register r in half h2.
__device__ __forceinline__ int acc_row(int r, int h2) { return 8 * (r >> 2) + 4 * h2 + (r & 3); }

// The transposing read of rd_rows_tr split into this lane's two element offsets for k-step
// 0 (lo: rows 0..3 of its group, hi: rows 8..11) and the read itself; k-step t4 adds 16 t4
// rows to both (swz(r) depends on r % 16 only).
template <int D>
__device__ __forceinline__ void tr_offsets(int dt, int l, int& lo, int& hi) {
  const int g = l >> 4, i = l & 15;
  const int ch = 32 * dt + 16 * (g & 1) + 4 * (i & 3);
  const int row = 4 * (g >> 1) + (i >> 2);
  lo = Lds<D>::chunk(row, ch >> 3) + (ch & 4);
  hi = Lds<D>::chunk(row + 8, ch >> 3) + (ch & 4);
}
__device__ __forceinline__ u32x4 rd_tr(const uint16_t* lds, int lo, int hi) {
  lds_u16* p = (lds_u16*)(lds);
  const s16x4_ a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + lo));
  const s16x4_ b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + hi));
  const u32x2 x = __builtin_bit_cast(u32x2, a), y = __builtin_bit_cast(u32x2, b);
  return u32x4{x[0], x[1], y[0], y[1]};
}

// Sixteen OCP E4M3 codes (bytes of raw, lowest first) times a power-of-two scale, as
// sixteen bf16 values (exact: four significant bits times a power of two) in two 8-value
// chunks, with gfx950's scaled conversion (two codes per instruction).
__device__ __forceinline__ void decode_e4m3x16(u32x4 raw, float scale, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i], scale, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i], scale, true);
    const uint32_t wa = __builtin_bit_cast(uint32_t, a), wb = __builtin_bit_cast(uint32_t, b);
    if (i < 2) {
      lo[2 * i] = wa;
      lo[2 * i + 1] = wb;
    } else {
      hi[2 * (i - 2)] = wa;
      hi[2 * (i - 2) + 1] = wb;
    }
  }
}

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
