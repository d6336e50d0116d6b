// Attention over the FP8 cache with FP8 arithmetic on the matrix cores (fine stage of PBSA,
// FP8 deployment).
//
// Light Forcing (papernotes.org, "Key findings") deploys the sparse attention in FP8.  The
// cache holds OCP E4M3 codes with one power-of-two scale per block and tensor (as the memory
// update writes them); this path also computes in FP8:
//   * Q is quantized per row as c q (c = scale * log2 e, so the scores come out in exp2
//     units): the smallest power of two 2^e with max|c q| <= 448 * 2^e, then each value's
//     nearest E4M3 code (ties to even);
//   * the chunk's own K/V blocks (bf16) are quantized per block and tensor exactly as the
//     memory update quantizes a cache slot, by chunk_e4m3_kernel, into the call's workspace;
//   * S^T = K Q^T runs on gfx950's scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4): the
//     power-of-two scales ride in the instruction as E8M0 exponents, so every product is the
//     exact product of the decoded values and the sums are fp32;
//   * each score tile's first MFMA starts from -m (the row offset) instead of zero, so
//     P = exp2(accumulator) is rounded to E4M3 (nearest even, gfx950's v_cvt_pk_fp8_f32) for
//     O^T += V^T P^T on the same MFMA, while the row sum adds the unrounded fp32 values.  The
//     offset m is raised lazily, as in the bf16 kernel, but so that no p exceeds 448 (E4M3's
//     largest value): a lane whose 32 exponentials of a block sum to more than 448 raises m to
//     its row max minus 3 (the max then maps to p = 8) and redoes the block.  A block whose
//     sum stays at or below 448 has every p <= 448; with the max at 8 the sum of a block's 32
//     values stays below 448 until the row max grows (a larger head room, 2^5, re-raised on
//     most blocks of keys that score alike and cost a quarter of the kernel's time).
//
// gfx950 design: the bf16 kernel's workgroup (two query blocks A, B of one head, four waves of
// 32 query rows; shared blocks gathered once for both) and pipeline (K two steps ahead, V one
// step ahead, a mid barrier between the S phase and the PV phase), with a whole 64-key block
// (8 KB of codes per tensor) where the bf16 kernel takes a 32-key half tile: a shared step takes
// two shared blocks X, Y; a private step A's next block (X) and B's (Y).  Per wave and 64 keys
// the MFMA work is half the bf16 kernel's (2 + 2 scaled FP8 MFMAs of 64 cycles per 32-key tile
// pair against 8 + 8 bf16 MFMAs of 32), the LDS traffic too; the softmax's VALU work is the
// same.  Tiles are row-major [64 keys][128 B] in LDS with the 16-byte chunk c of row r at
// position c ^ swz8(r) (below), filled straight from HBM/L2 by buffer_load ... lds (the
// permutation is in each lane's source address):
//   S^T: A = K (lane l: key l % 32, channels 64 m + 32 (l / 32) + [0, 32), two 16-byte reads),
//        B = Q (registers, the same channels of the lane's query row);
//   O^T: A = V^T (lane l: channel l % 32 of a 32-channel tile, 32 keys from four 8-bit
//        transposing reads ds_read_b64_tr_b8, each giving 8 keys of the lane's channel),
//        B = P^T packed from the S^T accumulators: byte 16 t + i of lane l holds accumulator i
//        of key tile t, i.e. key 32 t + 8 (i / 4) + 4 (l / 32) + i % 4; the V reads take the
//        same keys in the same byte order, so the contraction pairs them.
#include "attn_lists.h"
#include "fp8.h"

namespace pbsa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef __attribute__((address_space(4))) const float cfloat;

constexpr int kD8 = 128;                  // head_dim of the FP8 path
constexpr int kTile8 = kBlock * kD8;      // bytes of one block's codes
constexpr int kPieces8 = kTile8 / 1024;   // gather instructions per block
constexpr int kHP8 = kPieces8 / 2;        // ... per wave (two waves share a block)
constexpr float kRaiseSum8 = 448.f;       // largest E4M3 value
constexpr float kHead8 = 3.f;             // after a raise the row max maps to p = 2^3

template <int N>
struct B8 {
  static constexpr int value = N;
};

// Chunk position of a row's 16-byte chunks: c ^ swz8(r) with swz8(r) = the bits of
// u = (r / 2) % 8 with bits 0 and 1 exchanged.  Of 16 consecutive rows, the 8 even ones and
// the 8 odd ones each take 8 different positions (a K operand read, 16 rows of one chunk per
// pass, is free of bank conflicts), and the rows a transposing V read takes in one pass
// ({0, 1, 2, 3, 8, 9, 10, 11} + 4 g) have positions in different aligned pairs (its two
// chunks' 8-byte halves then fill 32 different bank pairs).
__device__ __forceinline__ int swz8(int row) {
  const int u = (row >> 1) & 7;
  return (u & 4) | ((u & 1) << 1) | ((u >> 1) & 1);
}

// E8M0 exponent field of a power-of-two float.
__device__ __forceinline__ int e8m0_of(float pow2) {
  return static_cast<int>((__float_as_uint(pow2) >> 23) & 0xffu);
}

// 32x32x64 E4M3 MFMA with E8M0 scales: byte SA of sa for the A rows, byte 0 of sb for the B
// columns; fp32 accumulate.
template <int SA>
__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SA, sa, 0, sb);
}

struct F8Args {
  FwdArgs f;          // ck / cv: the cache's E4M3 codes, kv_scale their scales
  const uint8_t* wk;  // the chunk's K codes [H][nq][64][128] (workspace)
  const uint8_t* wv;  // ... V codes
  const float* wsc;   // ... their scales [H][nq][2]
};

// grid (nq, H), 256 threads: block b of the chunk (rows [0, len)) -> codes, rows past the
// length code 0, and the power-of-two scale of each tensor -- the memory update's
// quantization of a slot.
__global__ void __launch_bounds__(256) chunk_e4m3_kernel(TokIn xk, TokIn xv, int nb, int n,
                                                         int nq, uint8_t* wk, uint8_t* wv,
                                                         float* wsc) {
  constexpr int CH = kD8 / 8;               // 8-value chunks per row
  constexpr int PER = kBlock * CH / 256;    // chunks per thread
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int l = t & 63, w = t >> 6;
  const int fl = b / nb, j = b - fl * nb;
  const int len = block_len(j, n);
  const int64_t tok0 = static_cast<int64_t>(fl) * n + static_cast<int64_t>(kBlock) * j;
  u32x4 kv[PER], vv[PER];
  float kmax = 0.f, vmax = 0.f;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int q = t + 256 * p;
    const int row = q / CH, cc = q % CH;
    kv[p] = u32x4{0, 0, 0, 0};
    vv[p] = u32x4{0, 0, 0, 0};
    if (row < len) {
      kv[p] = *reinterpret_cast<const u32x4*>(xk.p + h * xk.hs + (tok0 + row) * xk.ts + 8 * cc);
      vv[p] = *reinterpret_cast<const u32x4*>(xv.p + h * xv.hs + (tok0 + row) * xv.ts + 8 * cc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kmax = fmaxf(kmax, fmaxf(fabsf(__uint_as_float(kv[p][e] << 16)),
                               fabsf(__uint_as_float(kv[p][e] & 0xffff0000u))));
      vmax = fmaxf(vmax, fmaxf(fabsf(__uint_as_float(vv[p][e] << 16)),
                               fabsf(__uint_as_float(vv[p][e] & 0xffff0000u))));
    }
  }
  __shared__ float wmax[2][4];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmax = fmaxf(kmax, __shfl_xor(kmax, o, 64));
    vmax = fmaxf(vmax, __shfl_xor(vmax, o, 64));
  }
  if (l == 0) {
    wmax[0][w] = kmax;
    wmax[1][w] = vmax;
  }
  __syncthreads();
  kmax = fmaxf(fmaxf(wmax[0][0], wmax[0][1]), fmaxf(wmax[0][2], wmax[0][3]));
  vmax = fmaxf(fmaxf(wmax[1][0], wmax[1][1]), fmaxf(wmax[1][2], wmax[1][3]));
  const int ek = e4m3_scale_exp(kmax), ev = e4m3_scale_exp(vmax);
  const float ik = ldexpf(1.f, -ek), iv = ldexpf(1.f, -ev);  // exact reciprocals
  const int64_t blk = static_cast<int64_t>(h) * nq + b;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int q = t + 256 * p;
    const int row = q / CH, cc = q % CH;
    u32x2 kc = {0, 0}, vc = {0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k2 = e4m3_code(__uint_as_float(kv[p][e] << 16) * ik) |
                          (e4m3_code(__uint_as_float(kv[p][e] & 0xffff0000u) * ik) << 8);
      const uint32_t v2 = e4m3_code(__uint_as_float(vv[p][e] << 16) * iv) |
                          (e4m3_code(__uint_as_float(vv[p][e] & 0xffff0000u) * iv) << 8);
      kc[e >> 1] |= k2 << (16 * (e & 1));
      vc[e >> 1] |= v2 << (16 * (e & 1));
    }
    const int64_t o = blk * kTile8 + static_cast<int64_t>(row) * kD8 + 8 * cc;
    *reinterpret_cast<u32x2*>(wk + o) = kc;
    *reinterpret_cast<u32x2*>(wv + o) = vc;
  }
  if (t == 0) {
    wsc[2 * blk] = ldexpf(1.f, ek);
    wsc[2 * blk + 1] = ldexpf(1.f, ev);
  }
}

// Online-softmax state of one wave (32 query rows; this lane's row = column l % 32).  The
// queries are quantized as c q (c = scale * log2 e), so the S MFMAs give scores in exp2 units;
// each score tile's first MFMA starts from `neg` (-m in every entry), so the accumulators
// already hold c s - m and a probability is one exp2.
struct RowState8 {
  i32x8 q[2];     // codes of c q, MFMA m: channels 64 m + 32 h2 + [0, 32)
  int sq;         // E8M0 scale of this lane's query row
  f32x16 acc[4];  // O^T: channels 32 dt + acc_row(r, h2)
  f32x16 neg;     // -m_off in every entry
  float m_off;    // exp2 offset (starts at 0; the first block always sets it)
  float l_run;    // this lane's share of the row sum
  bool first;     // (wave-uniform) no block processed yet

  // Softmax of one block (two 32-key tiles of c s - m) in 8 stages (4 scores each), so that
  // the stages can ride under MFMAs: the exponentials, their sum, and their E4M3 codes
  // packed in the operand's byte order (byte 16 t + i = tile t, score i).
  struct Soft {
    float ps, alpha, delta;
    i32x8 pb;
    bool up;
  };
  __device__ __forceinline__ static void stage(int k, const f32x16 (&s)[2], Soft& so) {
    const int t = k >> 2, i0 = 4 * (k & 3);
    const float p0 = __builtin_amdgcn_exp2f(s[t][i0]);
    const float p1 = __builtin_amdgcn_exp2f(s[t][i0 + 1]);
    const float p2 = __builtin_amdgcn_exp2f(s[t][i0 + 2]);
    const float p3 = __builtin_amdgcn_exp2f(s[t][i0 + 3]);
    const float s4 = (p0 + p1) + (p2 + p3);
    so.ps = k == 0 ? s4 : so.ps + s4;
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
    wd = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, wd, true);
    so.pb[k] = wd;
  }
  // After the 8 stages: a lane whose sum exceeds 448 (or the first block of the rows) sends
  // the wave down the rare branch: the row max (in-lane and from the other lane half), the
  // offset raised by d to the row max minus 3 (set outright on the first block), the scores
  // shifted by -d and the block redone.  The caller shifts a tile computed before the raise
  // (the second block of a shared step) by so.delta.
  __device__ __forceinline__ void finish(f32x16 (&s)[2], Soft& so) {
    asm volatile("" ::"v"(so.pb), "v"(so.ps));
    so.up = first || __any(so.ps > kRaiseSum8);
    so.alpha = 1.f;
    so.delta = 0.f;
    if (so.up) {
      __builtin_amdgcn_sched_barrier(0);
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      float d = first ? mx - kHead8 : fmaxf(0.f, mx - kHead8);
      if (!(mx > -INFINITY)) d = 0.f;  // no valid key of the row in this block
      // (before the first block nothing has been accumulated: the factor is 0, not 2^-d)
      so.alpha = first ? 0.f : __builtin_amdgcn_exp2f(-d);
      so.delta = d;
      m_off += d;
      l_run *= so.alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        neg[r] -= d;
        s[0][r] -= d;
        s[1][r] -= d;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) stage(k, s, so);
      first = false;
    }
    l_run += so.ps;
  }
  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
  }
  // Keys at or past len (a frame's tail block, an empty entry) get -inf.  Key
  // 32 t + acc_row(r, h2) = (32 t + 8 (r / 4) + r % 4) + 4 h2 is compared as a constant
  // against len - 4 h2, so that no per-key index stays in registers.
  __device__ __forceinline__ static void mask(f32x16 (&s)[2], int len, int h2) {
    if (len < kBlock) {
      __builtin_amdgcn_sched_barrier(0);
      const int lim = len - 4 * h2;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + 8 * (r >> 2) + (r & 3) >= lim) s[t][r] = -INFINITY;
    }
  }
};

// MFMA j (tile t = j / 2, m = j % 2) of a block's S^T: its K operand (two 16-byte reads).
__device__ __forceinline__ i32x8 kread8(const uint8_t* kt, const int (&koff)[2][2], int j) {
  const int t = j >> 1, m = j & 1;
  const i32x4 a = *reinterpret_cast<const i32x4*>(kt + 4096 * t + koff[m][0]);
  const i32x4 b = *reinterpret_cast<const i32x4*>(kt + 4096 * t + koff[m][1]);
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// PV MFMA dt of a block: the V^T operand (four transposing reads, 8 keys each).
__device__ __forceinline__ i32x8 vread8(const uint8_t* vt, const int (&voff)[4], int dt) {
  const uint8_t* p = vt + voff[dt];
  const i32x2 r0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  const i32x2 r1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 2048));
  const i32x2 r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 4096));
  const i32x2 r3 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p + 6144));
  return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Wait until at most N of this wave's vector-memory instructions are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait8() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}
// Barrier that waits for this wave's LDS instructions but not for its gathers.
__device__ __forceinline__ void lds_barrier8() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void fence8() { __builtin_amdgcn_sched_barrier(0); }

// 1 KB of codes straight into LDS: piece i of a run of four sharing one LDS base and one
// scalar global base (the immediate 1024 i is added to both addresses; voff is lowered by it).
__device__ __forceinline__ void dma8(int i, __amdgpu_buffer_rsrc_t rs, uint32_t voff, uint8_t* lds) {
  switch (i) {
    case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0); break;
    case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 1024, 0); break;
    case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 2048, 0); break;
    default: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 3072, 0); break;
  }
}
// Buffer resource 3 KB below p (lane offsets, lowered by up to 3 KB, stay non-negative).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_base8(const uint8_t* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p - 3072), (short)0, 0x7fffffff,
                                           0x00020000);
}


}  // namespace

// 1-D grid of 8 * ceil(H * pairs / 8) workgroups of 256 threads (head_dim 128).
__global__ void __launch_bounds__(256, 2) attn_fwd_f8_kernel(F8Args g) {
  const FwdArgs& a = g.f;
  // K and V blocks (X and Y) of even and odd steps
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[2][kTile8];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[2][kTile8];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[2][kTile8];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[2][kTile8];
  __shared__ uint32_t lists[kAttnListCap + 1];
  __shared__ int wave_cnt[4];
  __shared__ int part_cnt[4][3];
  __shared__ int n_list;

  // XCD-aware numbering, as in the bf16 kernel
  const int per = gridDim.x / 8;
  const int L = static_cast<int>(blockIdx.x % 8) * per + static_cast<int>(blockIdx.x / 8);
  if (L >= a.H * a.pairs) return;
  const int h = L / a.pairs, pr = L - h * a.pairs;
  const int t = threadIdx.x, l = t & 63, h2 = l >> 5, c32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int mine = w >> 1;  // 0: query block A, 1: query block B
  const int rA = 2 * pr, rB = 2 * pr + 1;
  const int r = mine ? rB : rA;
  const int qlen = r < a.nq ? block_len(r % a.nb, a.n) : 0;
  const int qrow = 32 * (w & 1) + c32;
  const int64_t t0 = r < a.nq ? block_token0(r, a.nb, a.n) : 0;
  const float c = a.scale * kLog2e;

  // Q codes: this lane's 64 channels of its row times c (fp32), the row max over both lane
  // halves, the power-of-two scale and the nearest codes (rows past the block: zero codes)
  RowState8 st;
  {
    const uint16_t* qp = a.q + h * a.qhs + (t0 + qrow) * a.qts;
    u32x4 raw[8];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // chunk i: channels 64 (i / 4) + 32 h2 + 8 (i % 4) + [0, 8)
      raw[i] = qrow < qlen ? *reinterpret_cast<const u32x4*>(qp + 64 * (i >> 2) + 32 * h2 + 8 * (i & 3))
                           : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(raw[i][e] << 16) * c),
                                 fabsf(__uint_as_float(raw[i][e] & 0xffff0000u) * c)));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int eq = e4m3_scale_exp(amax);
    if (eq < -127) eq = -127;  // E8M0's smallest scale (the codes only get smaller)
    const float iq = ldexpf(1.f, -eq);
    // (v_cvt_pk_fp8_f32 rounds to the nearest E4M3 value, ties to even)
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(
            (__uint_as_float(raw[i][e] << 16) * c) * iq,
            (__uint_as_float(raw[i][e] & 0xffff0000u) * c) * iq, 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(
            (__uint_as_float(raw[i][e + 1] << 16) * c) * iq,
            (__uint_as_float(raw[i][e + 1] & 0xffff0000u) * c) * iq, wd, true);
        st.q[i >> 2][2 * (i & 3) + (e >> 1)] = wd;
      }
    st.sq = 127 + eq;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) st.acc[i] = f32x16{};
  st.neg = f32x16{};
  st.m_off = 0.f;
  st.l_run = 0.f;
  st.first = true;

  const FwdLists fl = build_lists<true, true>(
      a, h, rA, rB, lists, wave_cnt, part_cnt, n_list, reinterpret_cast<int32_t*>(&kb0[0][0]),
      reinterpret_cast<int32_t*>(&kb1[0][0]), reinterpret_cast<int32_t*>(&vb1[0][0]));
  const int cntA = fl.cntA, cntB = fl.cntB, nPq = fl.nPq, nshared = fl.nshared;
  const int offA = fl.offA, offB = fl.offB;
  // a shared step takes two shared blocks (X, Y); a private step A's next block (X) and B's
  // (Y).  Both phases have an even number of steps (empty steps pad them) so that the LDS
  // buffers alternate in a fixed order.
  const int nsh = (nshared + 1) >> 1, nsh2 = nsh + (nsh & 1);
  const int npv = cntA > cntB ? cntA : cntB, npv2 = npv + (npv & 1);
  const int nsteps = nsh2 + npv2;

  const int64_t hs = static_cast<int64_t>(h) * a.slots;
  const int64_t hq = static_cast<int64_t>(h) * a.nq;
  const uint8_t* ck_h = reinterpret_cast<const uint8_t*>(a.ck) + hs * kTile8;
  const uint8_t* cv_h = reinterpret_cast<const uint8_t*>(a.cv) + hs * kTile8;
  const uint8_t* wk_h = g.wk + hq * kTile8;
  const uint8_t* wv_h = g.wv + hq * kTile8;
  // Entries of step s for X and Y (0 = nothing), read one step before they are decoded.
  // The two reads are unconditional (an entry that does not exist reads the word past the
  // lists, which holds 0): reads of `lists` under branches lose the compiler's knowledge
  // that they cannot touch a tile being gathered, and it then waits for every gather first.
  auto fetch = [&](int s, uint32_t& ex, uint32_t& ey) {
    int ix, iy;
    bool vx, vy;
    if (s < nsh2) {
      const int i = 2 * s;
      ix = i < nPq ? i : offB - 1 - (i - nPq);
      iy = i + 1 < nPq ? i + 1 : offB - 2 - (i - nPq);
      vx = i < nshared;
      vy = i + 1 < nshared;
    } else {
      const int k = s - nsh2;
      ix = offA + k;
      iy = offB + k;
      vx = k < cntA && s < nsteps;
      vy = k < cntB && s < nsteps;
    }
    ex = lists[vx ? ix : kAttnListCap];
    ey = lists[vy ? iy : kAttnListCap];
  };
  // Step info: the raw entries of X and Y (0 = nothing) and their E8M0 scales packed in one
  // word (bytes: K of X, K of Y, V of X, V of Y; 1 for an empty entry), which the MFMAs take
  // by byte select.  Block addresses are formed when a gather is issued.
  struct StepInfo {
    uint32_t ex, ey;
    int sc;
  };
  // (scales are read through the constant address space: wave-uniform loads from it are
  // scalar loads, which the gathers' vmcnt waits do not count)
  const cfloat* wsc_h = (const cfloat*)(g.wsc + hq * 2);
  const cfloat* ksc_h = (const cfloat*)(a.kv_scale + hs * 2);
  auto scales_of = [&](uint32_t e) {  // (K scale) | (V scale) << 16
    int r = 127 | (127 << 16);
    if ((e >> 24) & 0x7f) {
      const uint32_t id = e & 0xffffffu;
      const cfloat* sc = ((e >> 31) ? wsc_h : ksc_h) + 2 * id;
      r = e8m0_of(sc[0]) | (e8m0_of(sc[1]) << 16);
    }
    return r;
  };
  auto decode = [&](uint32_t ex_, uint32_t ey_, StepInfo& si) {
    si.ex = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(ex_)));
    si.ey = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(ey_)));
    si.sc = scales_of(si.ex) | (scales_of(si.ey) << 8);
  };
  auto len_of = [](uint32_t e) { return static_cast<int>((e >> 24) & 0x7f); };
  // This wave's block of a step (X for waves 0, 1, Y for waves 2, 3): the K (or V) codes of
  // its entry; an empty entry gathers the chunk's first block (finite codes; masked).
  const int tw = w >> 1;
  auto block_of = [&](const StepInfo& si, bool v) {
    const uint32_t e = tw ? si.ey : si.ex;
    const uint32_t id = e & 0xffffffu;
    const uint8_t* base = (e >> 31) || len_of(e) == 0 ? (v ? wv_h : wk_h) : (v ? cv_h : ck_h);
    return base + (len_of(e) == 0 ? 0 : static_cast<int64_t>(id) * kTile8);
  };

  // Gathers: each wave moves kHP8 = 4 of the 8 K pieces and 4 of the 8 V pieces of its block
  // (waves 0, 1: X; 2, 3: Y).  Piece P is rows 8 P .. 8 P + 7; lane l writes LDS byte 16 l of
  // it, i.e. row 8 P + l / 8, position l % 8, which holds logical chunk
  // (l % 8) ^ swz8(8 P + l / 8); swz8 depends on the row mod 16, so on P's parity.
  const int p0 = (w & 1) * kHP8;
  const uint32_t d_even = (l >> 3) * 128u + 16u * static_cast<uint32_t>((l & 7) ^ swz8(l >> 3));
  const uint32_t d_odd = (l >> 3) * 128u + 16u * static_cast<uint32_t>((l & 7) ^ swz8(8 + (l >> 3)));
  const uint32_t vo_even = 1024u * p0 + d_even + 3072u, vo_odd = 1024u * p0 + d_odd + 3072u;
  auto gather = [&](uint8_t (*buf)[kTile8], const uint8_t* src, int i) {
    dma8(i, dma_base8(src), i & 1 ? vo_odd : vo_even, buf[tw] + 1024 * p0);
  };
  auto wait_keep_next = [&]() { vm_wait8<2 * kHP8>(); };

  // LDS read offsets of this lane.  K (S^T's A operand): key c32, chunks 4 m + 2 h2 + j.
  int koff[2][2];
  {
    const int sw = swz8(c32);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 2; ++j) koff[m][j] = c32 * 128 + 16 * ((4 * m + 2 * h2 + j) ^ sw);
  }
  // V (O^T's A operand): within 16-lane group G lane i = 2 e + m8 addresses row
  // 16 r + rho (read r) with rho = 8 (e / 4) + 4 (G / 2) + e % 4, channels
  // 32 dt + 16 (G % 2) + 8 m8 + [0, 8); the read returns to lane i the 8 rows of channel
  // 32 dt + 16 (G % 2) + i.
  int voff[4];
  {
    const int G = l >> 4, i = l & 15, e8 = i >> 1, m8 = i & 1;
    const int rho = 8 * (e8 >> 2) + 4 * (G >> 1) + (e8 & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      voff[dt] = rho * 128 + 16 * ((2 * dt + (G & 1)) ^ swz8(rho)) + 8 * m8;
  }

  // S^T of one block into s (two tiles); its MFMAs carry `extra` (gathers, softmax stages).
  auto s_mma = [&](auto sel, const uint8_t* kt, int sk, f32x16 (&s)[2], auto&& extra) {
    i32x8 kop[4];
    kop[0] = kread8(kt, koff, 0);
    kop[1] = kread8(kt, koff, 1);
    s[0] = st.neg;
    s[1] = st.neg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[j >> 1] = mfma8<decltype(sel)::value>(kop[j], st.q[j & 1], s[j >> 1], sk, st.sq);
      if (j + 2 < 4) kop[j + 2] = kread8(kt, koff, j + 2);
      extra(j);
      fence8();
    }
    // (the scores are taken here: otherwise the compiler sinks these MFMAs past the next
    // branch, away from the work they were meant to run beside)
    asm volatile("" ::"v"(s[0]), "v"(s[1]));
  };
  // O^T += V^T P^T of one block; its MFMAs carry `extra`.
  auto pv_mma = [&](auto sel, const uint8_t* vt, int sv, const i32x8& pb, auto&& extra) {
    i32x8 vop[4];
    vop[0] = vread8(vt, voff, 0);
    vop[1] = vread8(vt, voff, 1);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      st.acc[dt] = mfma8<decltype(sel)::value>(vop[dt], pb, st.acc[dt], sv, 127);
      if (dt + 2 < 4) vop[dt + 2] = vread8(vt, voff, dt + 2);
      extra(dt);
      fence8();
    }
    asm volatile("" ::"v"(st.acc[0]), "v"(st.acc[1]), "v"(st.acc[2]), "v"(st.acc[3]));
  };

  // prologue: K(0), V(0), K(1)
  StepInfo s0, s1, s2;
  uint32_t ex = 0, ey = 0;
  fetch(0, ex, ey);
  decode(ex, ey, s0);
  fetch(1, ex, ey);
  decode(ex, ey, s1);
  fetch(2, ex, ey);
  vm_wait8<0>();  // Q and the list inputs have landed: the loop's waits count gathers only
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kHP8; ++i) gather(kb0, block_of(s0, false), i);
#pragma unroll
  for (int i = 0; i < kHP8; ++i) gather(vb0, block_of(s0, true), i);
#pragma unroll
  for (int i = 0; i < kHP8; ++i) gather(kb1, block_of(s1, false), i);

  // Step s (kc/vc: its K and V buffers, vn: V buffer of step s+1): top barrier (K(s)
  // published) -> S phase with V(s+1)'s gathers -> mid barrier (V(s) published, K(s) free)
  // -> PV phase with K(s+2)'s gathers into kc.
  auto step = [&](uint8_t (*kc)[kTile8], uint8_t (*vc)[kTile8], uint8_t (*vn)[kTile8], int s,
                  bool shared) {
    wait_keep_next();
    lds_barrier8();
    decode(ex, ey, s2);
    fetch(s + 3, ex, ey);
    const uint8_t* n1 = block_of(s1, true);
    const uint8_t* n2 = block_of(s2, false);
    auto dma_v = [&](int i) {
      fence8();
      gather(vn, n1, i);
    };
    auto dma_k = [&](int i) {
      fence8();
      gather(kc, n2, i);
    };
    f32x16 sx[2], sy[2];
    RowState8::Soft so, sv2;
    if (shared) {
      // S phase: S of X (with two V gathers), S of Y (two V gathers) carrying X's softmax
      __builtin_amdgcn_s_setprio(1);
      s_mma(B8<0>{}, kc[0], s0.sc, sx, [&](int j) {
        if (j < 2) dma_v(j);
      });
      RowState8::mask(sx, len_of(s0.ex), h2);
      s_mma(B8<1>{}, kc[1], s0.sc, sy, [&](int j) {
        st.stage(2 * j, sx, so);
        st.stage(2 * j + 1, sx, so);
        if (j < 2) dma_v(2 + j);
      });
      __builtin_amdgcn_s_setprio(0);
      st.finish(sx, so);
      wait_keep_next();
      lds_barrier8();
      // PV phase: PV of X carrying Y's softmax (and the K gathers), then PV of Y.  Y's scores
      // were computed against the offset before X's raise (if any): shift them by its d.
      if (so.up) {
        st.rescale(so.alpha);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sy[0][r] -= so.delta;
          sy[1][r] -= so.delta;
        }
      }
      RowState8::mask(sy, len_of(s0.ey), h2);
      __builtin_amdgcn_s_setprio(1);
      pv_mma(B8<2>{}, vc[0], s0.sc, so.pb, [&](int j) {
        st.stage(2 * j, sy, sv2);
        st.stage(2 * j + 1, sy, sv2);
        dma_k(j);
      });
      __builtin_amdgcn_s_setprio(0);
      st.finish(sy, sv2);
      if (sv2.up) st.rescale(sv2.alpha);
      __builtin_amdgcn_s_setprio(1);
      pv_mma(B8<3>{}, vc[1], s0.sc, sv2.pb, [&](int) {});
      __builtin_amdgcn_s_setprio(0);
    } else {
      const int len = mine ? len_of(s0.ey) : len_of(s0.ex);
      __builtin_amdgcn_s_setprio(1);
      // (this wave's block: X for A's waves, Y for B's; its scales moved to bytes 0 and 2)
      const int scm = mine ? (s0.sc >> 8) : s0.sc;
      s_mma(B8<0>{}, kc[mine], scm, sx, [&](int j) { dma_v(j); });
      __builtin_amdgcn_s_setprio(0);
      RowState8::mask(sx, len, h2);
#pragma unroll
      for (int k = 0; k < 8; ++k) st.stage(k, sx, so);
      st.finish(sx, so);
      wait_keep_next();
      lds_barrier8();
      if (so.up) st.rescale(so.alpha);
      __builtin_amdgcn_s_setprio(1);
      pv_mma(B8<2>{}, vc[mine], scm, so.pb, [&](int j) { dma_k(j); });
      __builtin_amdgcn_s_setprio(0);
    }
    s0 = s1;
    s1 = s2;
  };
  int s = 0;
  for (; s < nsh2; s += 2) {
    step(kb0, vb0, vb1, s, true);
    step(kb1, vb1, vb0, s + 1, true);
  }
  for (; s < nsteps; s += 2) {
    step(kb0, vb0, vb1, s, false);
    step(kb1, vb1, vb0, s + 1, false);
  }
  vm_wait8<0>();  // no gather may still be writing this workgroup's LDS when it exits

  const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
  if (qrow < qlen) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.o + h * a.ohs + (t0 + qrow) * a.ots;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = 32 * dt + 8 * j + 4 * h2;
        u32x2 pk = {pack_bf16x2(st.acc[dt][4 * j] * inv, st.acc[dt][4 * j + 1] * inv),
                    pack_bf16x2(st.acc[dt][4 * j + 2] * inv, st.acc[dt][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + ch) = pk;
      }
    if (h2 == 0) a.lse[h * a.lse_hs + t0 + qrow] = st.m_off * kLn2 + logf(l_tot);
  }
}

size_t attn_fwd_f8_workspace(const pbsa_dims& d) {
  const int64_t blocks = int64_t{d.heads} * d.chunk_frames * nb_of(d);
  return static_cast<size_t>(blocks * (2 * kTile8 + 2 * sizeof(float)));
}

hipError_t launch_attn_fwd_f8(const pbsa_dims& d, TokIn q, const pbsa_cache& c, TokIn ck,
                              TokIn cv, const int32_t* sel, TokOut o, float* lse,
                              void* workspace, hipStream_t s) {
  F8Args g{};
  FwdArgs& a = g.f;
  const int nb = nb_of(d);
  a.q = q.p; a.qts = q.ts; a.qhs = q.hs;
  a.o = o.p; a.ots = o.ts; a.ohs = o.hs;
  a.lse = lse;
  a.lse_hs = static_cast<int64_t>(d.chunk_frames) * d.frame_tokens;
  a.ck = static_cast<const uint16_t*>(c.k);  // E4M3 codes, addressed in bytes
  a.cv = static_cast<const uint16_t*>(c.v);
  a.kv_scale = c.kv_scale;
  a.bid = c.block_id;
  a.blen = c.len;
  a.slots = static_cast<int>(slots_of(d));
  a.C = d.capacity;
  a.W = d.window_frames;
  a.xk = ck.p; a.xv = cv.p; a.xts = ck.ts; a.xhs = ck.hs;
  a.sel = sel;
  a.nsel = nullptr;
  a.sel_stride = d.topk;
  a.nq = d.chunk_frames * nb;
  a.n = d.frame_tokens;
  a.nb = nb;
  a.H = d.heads;
  a.pairs = cdiv(a.nq, 2);
  a.scale = d.scale;
  a.route_union = d.route_mode == PBSA_ROUTE_UNION;
  a.S = d.sinks;
  const int64_t blocks = int64_t{d.heads} * a.nq;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  g.wk = ws;
  g.wv = ws + blocks * kTile8;
  g.wsc = reinterpret_cast<const float*>(ws + 2 * blocks * kTile8);
  hipLaunchKernelGGL(chunk_e4m3_kernel, dim3(a.nq, d.heads), dim3(256), 0, s, ck, cv, nb,
                     d.frame_tokens, a.nq, ws, ws + blocks * kTile8,
                     reinterpret_cast<float*>(ws + 2 * blocks * kTile8));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.H * a.pairs;
  hipLaunchKernelGGL(attn_fwd_f8_kernel, dim3(8 * cdiv(G, 8)), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace pbsa
