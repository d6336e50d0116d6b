// Attention over selected KV blocks with an online softmax (fine stage of PBSA).
//
// Sparse Forcing (gist.science) 2.C and the Chinese page's 2.2: each query attends to all
// persistent blocks and to its query block's top-K window blocks (plus, here, the current
// chunk); with the selection fixed this is softmax attention restricted by a block mask,
// computed block by block with a running max and sum (flash-style).  The trainable
// two-level mode attends to a per-query-block list over the whole clip instead (there the
// shared blocks below are only those both query blocks selected).
//
// gfx950 design.  One workgroup = two 64-token query blocks of one head (A and B), four
// waves of 32 query rows.  The KV blocks every query block of the head attends (the
// persistent memory, the chunk itself, and the window blocks that A and B both routed to)
// are gathered once for both; then each query block's remaining routed window blocks.
// Each step gathers two half blocks (both halves of a shared block, or one half of A's and
// the same half of B's next private block).  Workgroups are numbered so that the eight XCDs each take a
// contiguous run of heads, keeping a head's KV in one XCD's L2.  Per KV block (64 keys,
// possibly fewer in a frame's tail block):
//   * the block is gathered from HBM/L2 with 16-byte loads into row-major LDS tiles; the
//     V operand is read channel-major with gfx950's transposing LDS read;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (Q lives in registers as the B operand), so
//     each lane holds 32 scores of ONE query row: the row max/sum are in-lane plus one
//     exchange with lane l^32;
//   * O^T += V^T P^T on the same MFMA, P converted to bf16 straight from the S^T
//     accumulators (the contraction order over keys is permuted identically in both
//     operands, which leaves the sum unchanged);
//   * gathers run two steps ahead for K and one step ahead for V: a step is split by a
//     mid barrier into its S phase (reads K) and its PV phase (reads V), so K's buffer is
//     free halfway through the step and V's at its end; the gather instructions are issued
//     a few at a time between MFMAs (issued in one burst they stall the wave).
// Softmax runs in base 2 with scale*log2(e) folded in (v_exp_f32), P is packed to bf16 with
// v_cvt_pk_bf16_f32, and the running max is raised lazily (checked on the row sums after
// the exponentials, not by a max before them); accumulators are fp32.
//
// FP8 cache (Light Forcing, papernotes.org, "Key findings": the sparse attention deployed
// with FP8).  The cache holds OCP E4M3 codes with one power-of-two scale per block and
// tensor; the chunk's own K/V stay bf16.  The FP8 instance keeps this pipeline: a cache
// slot's half tile is loaded as codes into registers (as many load instructions as the bf16
// gathers, so the waits stay exact), decoded with gfx950's scaled FP8 -> bf16 conversion
// (exact: the scale is a power of two) and stored into the same LDS layout before the
// barrier that publishes the tile -- K two steps ahead (loaded under a PV phase, stored at
// the end of the next S phase), V one step ahead (loaded under the S phase, stored at the
// end of the PV phase).  Chunk blocks still go straight into LDS.
#include "attn_lists.h"

namespace pbsa {


namespace {

// LDS layout of one 32-row half tile (bytes), chosen so that every LDS read is a per-lane
// base plus an immediate and touches contiguous bytes, and every gather instruction fills
// 1 KB of LDS:
//   K: [row / 16][16-byte channel chunk][row % 16]: the K operand of k-step s (16 rows of
//      one chunk per 16 lanes) is 256 contiguous bytes at base + 512 s;
//   V: [32-channel segment][row][64 bytes]: a transposing read (8 rows x 32 channels) is
//      512 contiguous bytes at base + 2048 dt + 1024 t4 (+ 512 for rows 8..15).
// A gather instruction moves 16 rows x 64 bytes (four chunks of K, one segment of V).
template <int D>
struct HalfTile {
  static constexpr int BYTES = 32 * D * 2;
  static constexpr int PIECES = BYTES / 1024;  // gather instructions per half tile
  static constexpr int KRG = 16 * D * 2;       // K: bytes per 16-row group
};

// Full scheduling fence (the compiler may not move instructions across it).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// Issue priority of a wave while it runs its MFMA groups: ahead of the other wave on its SIMD
// (whose softmax, LDS reads and gathers then fill in behind it), which keeps the matrix pipe
// fed (about 2% on the persistent-mode chunk).
__device__ __forceinline__ void prio_mfma() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_rest() { __builtin_amdgcn_s_setprio(0); }

// Wait until at most N of this wave's vector-memory instructions (here: gathers into LDS)
// are outstanding; they complete in issue order.  A barrier after it makes the landed
// tiles visible to the other waves.  The compiler does not add this wait by itself (a
// barrier's release only covers LDS instructions), so every barrier that publishes
// gathered tiles needs one.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);  // vmcnt(N), expcnt and lgkmcnt not waited
}

// Workgroup barrier that waits for this wave's LDS instructions (lgkmcnt(0)) but not for
// its gathers into LDS.  __syncthreads() (and any workgroup fence) would also wait for
// every outstanding gather; here the gathers are waited for explicitly (vm_wait) and only
// as far as each barrier needs.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from global memory straight into LDS (lane l writes lds + 16 l; the LDS
// address must be wave-uniform), as piece i (0..3) of a run of 1 KB LDS pieces: the
// instruction's immediate offset 1024 i is added to both the global and the LDS address,
// so a run shares one LDS base (M0), one buffer resource and one scalar offset (soff, the
// half tile's position), and each piece costs one vector add for its lane offsets, which
// must already be lowered by 1024 i.
__device__ __forceinline__ void lds_dma16_piece(int i, __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                                uint32_t soff, char* lds) {
  switch (i) {
    case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, soff, 0, 0); break;
    case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, soff, 1024, 0); break;
    case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, soff, 2048, 0); break;
    default: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, soff, 3072, 0); break;
  }
}
// Buffer resource whose base is 3 KB below p: per-piece lane offsets (up to 3 KB lower for
// piece 3) then stay non-negative.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_base(const char* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p - 3072), (short)0, 0x7fffffff,
                                           0x00020000);
}

// A half tile to gather: wave-uniform position (bytes from its tensor's head base), row
// stride (bytes) and valid rows.
struct HalfRef {
  uint32_t off;  // byte offset of the half tile from its tensor's head base
  uint32_t tok;  // 1: a block of the chunk's K/V; 0: a cache slot
  uint32_t stride;
  int len;      // 0 = nothing to gather
  bool f8;      // E4M3 codes of an FP8 cache slot (loaded into registers and decoded)
  float ks, vs; // their K and V scales
};

// Online-softmax state of one wave (32 query rows, this lane's row = column c32).
template <int D>
struct RowState {
  static constexpr int NS = D / 16, ND = D / 32;
  u32x4 qreg[NS];
  f32x16 acc[ND];
  // exp2 offset (the running max times c = scale * log2 e); before the first key it is a
  // huge negative number, so that every exponential overflows and the first tile always
  // sets it from its own row max
  float m_off;
  float l_run;  // this lane's share of the row sum (its 16 keys of each 32-key tile)
  static constexpr float kNoOffset = -3.0e38f;
  // A tile whose exponentials sum to more than this in one lane was computed against an
  // offset too far below its scores: the offset is raised and the tile redone.
  static constexpr float kRaiseSum = 1099511627776.f;  // 2^40

  // Raise the offset of every row to at least its max mx (times c).  Returns the factor
  // for the earlier accumulators through alpha (0 before the first key: exp2 of a huge
  // negative number); l_run is scaled here, acc by the caller.
  __device__ __forceinline__ void raise(float mx, float c, float& alpha) {
    const float m_new = fmaxf(m_off, mx * c);
    alpha = __builtin_amdgcn_exp2f(m_off - m_new);
    m_off = m_new;
    l_run *= alpha;
  }
  // Lazy form for the unpipelined path: only when some row's max exceeds the offset by
  // more than 2^8 in exp2 units (so exp2 arguments stay <= 8); the common path is one
  // compare.
  __device__ __forceinline__ bool raise_lazy(float mx, float c, float& alpha) {
    const bool up = __any(mx * c > m_off + 8.f);
    alpha = 1.f;
    if (up) raise(mx, c, alpha);
    return up;
  }

  // S^T for the keys of one K half tile: keys acc_row(r, h2), query = this lane's row.
  // kb: this lane's K read address (bytes, LDS).
  __device__ __forceinline__ f32x16 scores(const char* kb, int len, int h2) const {
    u32x4 kop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kop[s] = *reinterpret_cast<const u32x4*>(kb + 512 * s);
    f32x16 sa = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) sa = mfma32(kop[s], qreg[s], sa);
    if (len < 32) {
      // rare (a frame's tail block): keep it a branch rather than 16 selects per tile
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, h2) >= len) sa[r] = -INFINITY;
    }
    return sa;
  }

  // O^T += V^T P^T for one V half tile; vb: this lane's transposing-read address.
  __device__ __forceinline__ void pv(const f32x16& p, const char* vb) {
    lds_u16* base = (lds_u16*)(vb);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      u32x4 vop[ND];
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const s16x4_ lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(base + (2048 * dt + 1024 * t2) / 2));
        const s16x4_ hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(base + (2048 * dt + 1024 * t2 + 512) / 2));
        const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
        vop[dt] = u32x4{x[0], x[1], y[0], y[1]};
      }
      const u32x4 pb = pack_step(&p, t2);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(vop[dt], pb, acc[dt]);
    }
  }

  // K operands of one half tile.
  __device__ __forceinline__ void kread(const char* kb, u32x4 (&kop)[NS]) const {
#pragma unroll
    for (int s = 0; s < NS; ++s) kop[s] = *reinterpret_cast<const u32x4*>(kb + 512 * s);
  }
  __device__ __forceinline__ f32x16 smma(const u32x4 (&kop)[NS]) const {
    f32x16 sa = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) sa = mfma32(kop[s], qreg[s], sa);
    return sa;
  }
  __device__ __forceinline__ static void mask(f32x16& sa, int len, int h2) {
    if (len < 32) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, h2) >= len) sa[r] = -INFINITY;
    }
  }
  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
  }
  // The transposing V reads of MFMA j (t2 = j / ND, dt = j % ND) of a PV step.
  __device__ __forceinline__ static u32x4 vread(const char* vb, int j) {
    const int t2 = j / ND, dt = j % ND;
    lds_u16* base = (lds_u16*)(vb);
    const s16x4_ lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + (2048 * dt + 1024 * t2) / 2));
    const s16x4_ hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + (2048 * dt + 1024 * t2 + 512) / 2));
    const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
    return u32x4{x[0], x[1], y[0], y[1]};
  }

  // Softmax of one score tile in stages, so that the stages can ride under MFMAs of the
  // other tile.  The exponentials use the current offset without looking at the tile's
  // max first: stage k takes the exponentials of pair k of this lane's 16 scores and adds
  // and packs (bf16) pair k - 1; finish() takes the last pair and then checks the sums: a
  // lane whose 16 exponentials sum to more than kRaiseSum (one of them overflowed, or the
  // offset lags the scores by more than 2^40) sends the whole wave down the rare branch,
  // which takes the row max (in-lane plus the other lane half through gfx950's permlane
  // swap), raises the offset and redoes the tile.  The first tile of every row takes that
  // branch.
  static constexpr int kStages = 8;
  struct Soft {
    float alpha, ps;
    float p[16];
    u32x4 pb[2];
    bool up;
  };
  __device__ __forceinline__ void sum_pack(int j, Soft& so) {
    const float s2 = so.p[2 * j] + so.p[2 * j + 1];
    so.ps = j == 0 ? s2 : so.ps + s2;
    so.pb[j >> 2][j & 3] = pack_bf16x2(so.p[2 * j], so.p[2 * j + 1]);
  }
  __device__ __forceinline__ void stage(int k, const f32x16& sa, Soft& so, float c) {
    so.p[2 * k] = __builtin_amdgcn_exp2f(fmaf(sa[2 * k], c, -m_off));
    so.p[2 * k + 1] = __builtin_amdgcn_exp2f(fmaf(sa[2 * k + 1], c, -m_off));
    if (k > 0) sum_pack(k - 1, so);
  }
  __device__ __forceinline__ void finish(const f32x16& sa, Soft& so, float c) {
    sum_pack(kStages - 1, so);
    // the packing stays in the stages' scheduling groups (not sunk into the common branch)
    asm volatile("" ::"v"(so.pb[0]), "v"(so.pb[1]), "v"(so.ps));
    so.up = __any(so.ps > kRaiseSum);
    so.alpha = 1.f;
    if (so.up) {
      __builtin_amdgcn_sched_barrier(0);
      float mx = sa[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sa[r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      raise(fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])), c, so.alpha);
#pragma unroll
      for (int k = 0; k < kStages; ++k) stage(k, sa, so, c);
      sum_pack(kStages - 1, so);
    }
    l_run += so.ps;
  }

  // The pipelined steps (head_dim 128) come in two halves around the step's mid barrier:
  // A = the S phase (reads K), B = the PV phase (reads V).  Scheduling groups are explicit
  // (sched_fence) and each carries one gather instruction (dma(i)) so that the gathers are
  // issued between MFMAs; issued in one burst they would stall the wave.
  struct Mid {
    f32x16 sy;  // S of the second half tile (pair)
    Soft so;    // softmax of the first half tile
  };

  // One half tile (a private step), S phase: S MFMAs with the gathers, then the softmax
  // (it cannot overlap this wave's own MFMAs here).
  template <class Dma>
  __device__ __forceinline__ void singleA(const char* kb, int len, float c, int h2, Dma&& dma,
                                          Mid& md) {
    u32x4 kop[NS];
    kread(kb, kop);
    prio_mfma();
    f32x16 sa = {};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      sa = mfma32(kop[i], qreg[i], sa);
      dma(i);
      sched_fence();
    }
    prio_rest();
    mask(sa, len, h2);
#pragma unroll
    for (int k = 0; k < kStages; ++k) stage(k, sa, md.so, c);
    finish(sa, md.so, c);
    asm volatile("" ::"v"(md.so.pb[0]), "v"(md.so.pb[1]));
  }
  // PV phase of a private step: the V reads run two MFMAs ahead.
  template <class Dma>
  __device__ __forceinline__ void singleB(const char* vb, Dma&& dma, Mid& md) {
    if (md.so.up) rescale(md.so.alpha);
    u32x4 vop[2 * ND];
    vop[0] = vread(vb, 0);
    vop[1] = vread(vb, 1);
    prio_mfma();
#pragma unroll
    for (int j = 0; j < 2 * ND; ++j) {
      acc[j % ND] = mfma32(vop[j], md.so.pb[j / ND], acc[j % ND]);
      if (j + 2 < 2 * ND) vop[j + 2] = vread(vb, j + 2);
      dma(j);
      sched_fence();
    }
    prio_rest();
  }

  // Two half tiles (X then Y, a shared step), S phase: the gathers and the K reads of Y
  // ride under the S MFMAs of X; each S MFMA of Y carries one softmax stage of X.
  template <class Dma>
  __device__ __forceinline__ void pairA(const char* kx, const char* ky, int lx, float c, int h2,
                                        Dma&& dma, Mid& md) {
    static_assert(NS == 8 && ND == 4, "the pipelined pair is laid out for head_dim 128");
    u32x4 kop[NS], kopy[NS];
    kread(kx, kop);
    prio_mfma();
    f32x16 sx = {};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      sx = mfma32(kop[i], qreg[i], sx);
      dma(i);
      kopy[i] = *reinterpret_cast<const u32x4*>(ky + 512 * i);
      sched_fence();
    }
    mask(sx, lx, h2);
    md.sy = f32x16{};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      md.sy = mfma32(kopy[i], qreg[i], md.sy);
      if (i < kStages) stage(i, sx, md.so, c);
      sched_fence();
    }
    prio_rest();
    finish(sx, md.so, c);
    // the exponentials of X stay in the groups above (not sunk past later branches)
    asm volatile("" ::"v"(md.so.pb[0]), "v"(md.so.pb[1]));
  }
  // PV phase of a shared step: each PV MFMA of X carries one softmax stage of Y and a
  // gather; the V reads run two MFMAs ahead.  The rare rescales sit between the phases.
  template <class Dma>
  __device__ __forceinline__ void pairB(const char* vx, const char* vy, int ly, float c, int h2,
                                        Dma&& dma, Mid& md) {
    if (md.so.up) rescale(md.so.alpha);
    mask(md.sy, ly, h2);
    Soft sv;
    u32x4 vop[4 * ND];  // V of X (0..7), then V of Y (8..15)
    vop[0] = vread(vx, 0);
    vop[1] = vread(vx, 1);
    prio_mfma();
#pragma unroll
    for (int j = 0; j < 2 * ND; ++j) {
      acc[j % ND] = mfma32(vop[j], md.so.pb[j / ND], acc[j % ND]);
      const int nx = j + 2;
      vop[nx] = nx < 2 * ND ? vread(vx, nx) : vread(vy, nx - 2 * ND);
      if (j < kStages) stage(j, md.sy, sv, c);
      dma(j);
      sched_fence();
    }
    finish(md.sy, sv, c);
    asm volatile("" ::"v"(sv.pb[0]), "v"(sv.pb[1]));
    if (sv.up) rescale(sv.alpha);
#pragma unroll
    for (int j = 0; j < 2 * ND; ++j) {
      acc[j % ND] = mfma32(vop[2 * ND + j], sv.pb[j / ND], acc[j % ND]);
      if (j + 2 < 2 * ND) vop[2 * ND + j + 2] = vread(vy, j + 2);
      sched_fence();
    }
    prio_rest();
  }

  // Online-softmax update with NT score tiles (32 keys each) and their V half tiles.
  // The offset only moves when some row's new max exceeds it by more than 2^8 in exp2
  // units, so the rescale of the accumulators is rare; exp2 arguments stay <= 8.
  template <int NT>
  __device__ __forceinline__ void update(f32x16* sacc, const char* v0, const char* v1, float c) {
    float mx = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float alpha;
    if (raise_lazy(mx, c, alpha)) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], c, -m_off));
        sacc[kt][r] = p;
        psum += p;
      }
    l_run += psum;
    pv(sacc[0], v0);
    if (NT > 1) pv(sacc[1], v1);
  }
};

}  // namespace

// 1-D grid of 8 * ceil(H * pairs / 8) workgroups of 256 threads.  GATHER_ONLY builds the
// gather probe: the same lists, gathers, waits and barriers with the math left out (no
// output is written).
template <int D, bool PERSIST, bool GATHER_ONLY = false, bool FP8 = false>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(FwdArgs a) {
  using HT = HalfTile<D>;
  // K and V half tiles (X and Y) of even and odd steps, gathered straight into LDS; four
  // distinct arrays so that the compiler can tell a gather's target from the tiles being
  // read.
  __shared__ __attribute__((aligned(1024))) char kb0[2][HT::BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[2][HT::BYTES];
  __shared__ __attribute__((aligned(1024))) char vb0[2][HT::BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[2][HT::BYTES];
  // Block lists: static (a dynamic LDS array defeats the compiler's alias analysis, which
  // then waits for every gather in flight before each list read).
  __shared__ uint32_t lists[kAttnListCap + 1];
  __shared__ int wave_cnt[4];
  __shared__ int part_cnt[4][3];
  __shared__ int n_list;

  // XCD-aware numbering: hardware workgroup i runs on XCD i % 8; give each XCD a
  // contiguous range of (head, pair) so a head's KV stays in one L2.
  const int per = gridDim.x / 8;
  const int L = static_cast<int>(blockIdx.x % 8) * per + static_cast<int>(blockIdx.x / 8);
  if (L >= a.H * a.pairs) return;
  const int h = L / a.pairs, pr = L - h * a.pairs;
  const int t = threadIdx.x, l = t & 63, h2 = l >> 5, c32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, scalar
  const int mine = w >> 1;  // 0: query block A, 1: query block B
  const int rA = 2 * pr, rB = 2 * pr + 1;
  const int r = mine ? rB : rA;
  const int qlen = r < a.nq ? block_len(r % a.nb, a.n) : 0;
  const int qrow = 32 * (w & 1) + c32;
  const int64_t t0 = r < a.nq ? block_token0(r, a.nb, a.n) : 0;
  const float c = a.scale * kLog2e;
  // (pids: union routing's lookups of persistent block ids, staged in a V tile; rawA/rawB:
  // the routed ids, staged in two K tiles; no gather has targeted them yet, and the V tiles
  // are cleared after the lists are built)
  const FwdLists fl = build_lists<PERSIST, false>(
      a, h, rA, rB, lists, wave_cnt, part_cnt, n_list, reinterpret_cast<int32_t*>(&kb0[0][0]),
      reinterpret_cast<int32_t*>(&kb1[0][0]), reinterpret_cast<int32_t*>(&vb1[0][0]));
  const int cntA = fl.cntA, cntB = fl.cntB, nPq = fl.nPq, nshared = fl.nshared;
  constexpr uint32_t kCacheBlockBytes = kBlock * D * (FP8 ? 1 : 2);
  const uint32_t xrow = static_cast<uint32_t>(a.xts * 2);
  // a shared step takes both halves of one shared block; a private step takes one half
  // of A's next routed block (X) and the same half of B's (Y).  The shared phase is
  // padded to an even number of steps (an empty step) so that both phases alternate the
  // two LDS buffers in a fixed order.
  const int nsh2 = nshared + (nshared & 1);
  const int nsteps = nsh2 + 2 * (cntA > cntB ? cntA : cntB);

  RowState<D> st;
  load_row_operand<D>(st.qreg, a.q + h * a.qhs + t0 * a.qts, a.qts, qrow, qlen, h2);
#pragma unroll
  for (int i = 0; i < RowState<D>::ND; ++i) st.acc[i] = f32x16{};
  st.m_off = RowState<D>::kNoOffset;
  st.l_run = 0.f;

  const char* ck_h = reinterpret_cast<const char*>(a.ck) +
                     static_cast<int64_t>(h) * a.slots * kCacheBlockBytes;
  const char* cv_h = reinterpret_cast<const char*>(a.cv) +
                     static_cast<int64_t>(h) * a.slots * kCacheBlockBytes;
  const char* xk_h = reinterpret_cast<const char*>(a.xk + h * a.xhs);
  const char* xv_h = reinterpret_cast<const char*>(a.xv + h * a.xhs);
  auto half_len = [](uint32_t e, int half) {  // valid rows of half tile `half` (0 if e = 0)
    const int len = static_cast<int>((e >> 24) & 0x7f) - 32 * half;
    return len < 0 ? 0 : (len < 32 ? len : 32);
  };
  auto ref_of = [&](uint32_t e, int half, HalfRef& hr) {
    const bool tok = (e >> 31) != 0;
    const uint32_t id = e & 0xffffffu;
    const uint32_t stride = tok ? xrow : (FP8 ? D : 2 * D);
    const uint32_t o = id * (tok ? xrow : kCacheBlockBytes) + 32 * half * stride;
    hr.len = half_len(e, half);
    hr.f8 = false;
    hr.ks = hr.vs = 1.f;
    if (hr.len > 0) {
      hr.off = o;
      hr.tok = tok;
      hr.stride = stride;
      if (FP8 && !tok) {
        hr.f8 = true;
        // (read through the constant address space: a wave-uniform load from it is a scalar
        // load, which the gathers' vmcnt waits do not count; a vector load here made the
        // compiler drain every gather in flight before using the scale)
        typedef __attribute__((address_space(4))) const float cfloat;
        const cfloat* sc = (const cfloat*)(a.kv_scale) + (static_cast<int64_t>(h) * a.slots + id) * 2;
        hr.ks = sc[0];
        hr.vs = sc[1];
      }
    } else {
      // an empty half tile still gets its gathers (of the head's first token row, so
      // that every step issues the same number and the waits stay fixed); its rows are
      // masked or weighted by zero
      hr.off = 0;
      hr.tok = 1;
      hr.stride = 0;
    }
  };
  // Raw list entries of step s for X and Y (0 = nothing).  They are read one step before
  // they are decoded, so the LDS read's latency is never waited for.
  // (Indices into `lists` itself, not pointers chosen at run time: the compiler then still
  // sees that these reads cannot touch a tile being gathered and adds no wait for them.)
  const int offA = fl.offA, offB = fl.offB;
  auto fetch = [&](int s, uint32_t& ex, uint32_t& ey) {
    // two reads, always issued (no branch, and no copy of a value still in flight); an
    // entry that does not exist reads the word past the lists, which holds 0
    const int blk = (s - nsh2) >> 1;
    const bool sh = s < nshared, pv = s >= nsh2 && s < nsteps;
    const int is = s < nPq ? s : offB - 1 - (s - nPq);
    const int ix = sh ? is : (pv && blk < cntA ? offA + blk : kAttnListCap);
    const int iy = sh ? is : (pv && blk < cntB ? offB + blk : kAttnListCap);
    ex = lists[ix];
    ey = lists[iy];
  };
  // This wave's half tile of step s (see the gathers below) and the lengths of X and Y.
  // Only this wave's half tile is decoded into addresses; of the other, its length.
  auto decode = [&](int s, uint32_t ex_, uint32_t ey_, HalfRef& mineref, int& lenX, int& lenY) {
    // list entries are wave-uniform: readfirstlane keeps them (and the gathers' offsets)
    // in scalar registers
    const uint32_t ex = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(ex_)));
    const uint32_t ey = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(ey_)));
    // a shared step takes halves 0 (X) and 1 (Y) of one block; a private step the same
    // half of A's (X) and B's (Y) next routed block
    const int hx = s < nshared ? 0 : ((s - nsh2) & 1);
    const int hy = s < nshared ? 1 : hx;
    lenX = half_len(ex, hx);
    lenY = half_len(ey, hy);
    const bool use_y = (w >> 1) != 0;
    ref_of(use_y ? ey : ex, use_y ? hy : hx, mineref);
  };

  // Gathers: waves 0, 1 gather half tile X of every step, waves 2, 3 half tile Y; each
  // wave takes half of the tile's K pieces and half of its V pieces, so that every wave
  // issues the same sequence (K(s), V(s), K(s+1), V(s+1), ...) and the waits below are
  // exact.  Rows past the valid length re-read the last valid row (finite data that the
  // mask or a zero probability removes).
  constexpr int HP = HT::PIECES / 2;  // pieces of K (and of V) per wave and step
  const int p0 = (w & 1) * HP;        // this wave's first piece
  const int tw = w >> 1;              // this wave's half tile: 0 = X, 1 = Y
  const uint32_t k_rowl = l & 15, k_colb = 16u * (l >> 4);
  const uint32_t v_rowl = l >> 2, v_colb = 16u * (l & 3);
  //   K piece p: rows 16 (p / HP) .., chunks 4 (p % HP) ..
  //   V piece p: rows 16 (p % 2) .., 32-channel segment p / 2
  // so this wave's K pieces all use rows 16 (w & 1) + (l & 15) (one lane offset per step)
  // and its V pieces rows (l >> 2) or 16 + (l >> 2) (two lane offsets per step); the
  // piece's chunk or segment is a scalar offset.
  // The wave's HP pieces of a tile form one run (lds_dma16_piece): one LDS base, the
  // head's buffer resource for the tensor (dma_base, 3 KB low; chosen per step between the
  // chunk's and the cache's), the half tile's position as the scalar offset, and per-piece
  // lane offsets raised by 3 KB and lowered by the piece's 1 KB immediate offset.
  struct Offs {
    __amdgpu_buffer_rsrc_t kb, vb;  // the head's K and V bases (chunk or cache)
    uint32_t soff;                  // the half tile's byte offset from them
    uint32_t k, v0, v1;   // lane offsets of K, and of V rows (l >> 2) and 16 + (l >> 2)
    uint32_t fk, fv;      // (FP8 slot) lane offsets of this lane's 32 K and 32 V codes
    uint32_t flast;       // (FP8 slot) the last valid row
  };
  const __amdgpu_buffer_rsrc_t rs_ck = dma_base(ck_h), rs_cv = dma_base(cv_h);
  const __amdgpu_buffer_rsrc_t rs_xk = dma_base(xk_h), rs_xv = dma_base(xv_h);
  auto offsets = [&](const HalfRef& hr) {
    const uint32_t last = static_cast<uint32_t>(hr.len > 0 ? hr.len - 1 : 0);
    Offs o;
    o.kb = hr.tok ? rs_xk : rs_ck;
    o.vb = hr.tok ? rs_xv : rs_cv;
    o.soff = hr.off;
    o.k = min(16u * (w & 1) + k_rowl, last) * hr.stride + k_colb + 3072u;
    // this wave's V pieces p0 + i lie in segments (p0 + i) / 2 = p0 / 2 + i / 2
    o.v0 = min(v_rowl, last) * hr.stride + v_colb + 32u * p0 + 3072u;
    o.v1 = min(16u + v_rowl, last) * hr.stride + v_colb + 32u * p0 + 3072u;
    if constexpr (FP8) {
      // the same rows and channels as the wave's bf16 pieces, as codes: K rows
      // 16 (w & 1) + (l & 15), channels 32 (l >> 4) + [0, 32); V rows (l >> 3) + 8 i
      // (load i), channels 64 (w & 1) + 8 (l & 7) + [0, 8), so that each decoded V store
      // of the wave fills two contiguous 512-byte runs of the tile
      o.fk = min(16u * (w & 1) + k_rowl, last) * hr.stride + 32u * (l >> 4) + 3072u;
      o.fv = 64u * (w & 1) + 8u * (l & 7) + 3072u;  // + row offset per load
      o.flast = last;
    }
    return o;
  };
  // (FP8) codes of this wave's pieces in flight: K of the step two ahead (loaded under a
  // PV phase, decoded into LDS at the end of the next S phase), V of the next step (loaded
  // under an S phase, decoded at the end of the same step's PV phase)
  u32x2 kpend[HP], vpend[HP];
  float kscale = 1.f, vscale = 1.f;
  bool kp8 = false, vp8 = false;
  auto gather_k = [&](char (*buf)[HT::BYTES], const HalfRef& hr, const Offs& o, int i) {
    if constexpr (FP8) {
      if (i == 0) {
        kp8 = hr.f8;
        kscale = hr.ks;
      }
      if (hr.f8) {
        // as many instructions as the bf16 pieces, so the waits below stay exact
        kpend[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                 o.kb, o.fk + 8u * i, o.soff, 0));
        return;
      }
    }
    lds_dma16_piece(i, o.kb, o.k + 64u * i - 1024u * i, o.soff, buf[tw] + 1024 * p0);
  };
  auto gather_v = [&](char (*buf)[HT::BYTES], const HalfRef& hr, const Offs& o, int i) {
    if constexpr (FP8) {
      if (i == 0) {
        vp8 = hr.f8;
        vscale = hr.vs;
      }
      if (hr.f8) {
        const uint32_t row = min(static_cast<uint32_t>(l >> 3) + 8u * i, o.flast);
        vpend[i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                                 o.vb, o.fv + row * hr.stride, o.soff, 0));
        return;
      }
    }
    lds_dma16_piece(i, o.vb, (i % 2 ? o.v1 : o.v0) + 64u * (i / 2) - 1024u * i, o.soff,
                    buf[tw] + 1024 * p0);
  };
  // (FP8) decode the pending codes (exact in bf16: a power-of-two scale) and store them
  // into the tile layouts the bf16 gathers fill
  auto store_k = [&](char (*buf)[HT::BYTES]) {
    if constexpr (FP8) {
      if (kp8) {
        u32x4 d[4];
        decode_e4m3x16(u32x4{kpend[0][0], kpend[0][1], kpend[1][0], kpend[1][1]}, kscale,
                       d[0], d[1]);
        decode_e4m3x16(u32x4{kpend[2][0], kpend[2][1], kpend[3][0], kpend[3][1]}, kscale,
                       d[2], d[3]);
        const int R = 16 * (w & 1) + (l & 15);
        char* base = buf[tw] + (R >> 4) * HT::KRG + 16 * (R & 15) + 256 * 4 * (l >> 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(base + 256 * j) = d[j];
      }
    }
  };
  auto store_v = [&](char (*buf)[HT::BYTES]) {
    if constexpr (FP8) {
      if (vp8) {
        u32x4 d[4];
        decode_e4m3x16(u32x4{vpend[0][0], vpend[0][1], vpend[1][0], vpend[1][1]}, vscale,
                       d[0], d[1]);
        decode_e4m3x16(u32x4{vpend[2][0], vpend[2][1], vpend[3][0], vpend[3][1]}, vscale,
                       d[2], d[3]);
        // row (l >> 3) + 8 j, segment 2 (w & 1) + ((l & 7) >> 2), 16-byte chunk l & 3
        char* base = buf[tw] + 2048 * (2 * (w & 1) + ((l & 7) >> 2)) + 64 * (l >> 3) +
                     16 * (l & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(base + 512 * j) = d[j];
      }
    }
  };
  // Waits before the barriers that publish gathered tiles.  Each wave's gathers in issue
  // order: K(s), V(s), K(s+1), V(s+1), ... (HP instructions each).  Before the top barrier
  // of step s, K(s) must have landed (V(s) and K(s+1) may be in flight); before the mid
  // barrier V(s) (K(s+1) and V(s+1) may be in flight).
  auto wait_keep_next = [&]() { vm_wait<2 * HP>(); };

  // this lane's LDS read offsets inside a half tile
  const int kofs = (c32 >> 4) * HT::KRG + 256 * h2 + 16 * (c32 & 15);
  const int g16 = l >> 4, i16 = l & 15;
  const int vofs = (4 * (g16 >> 1) + (i16 >> 2)) * 64 + 32 * (g16 & 1) + 8 * (i16 & 3);

  // V buffers start zeroed: a V half tile that a step leaves empty is still read (with
  // zero probabilities) and must hold finite values.  (Empty K half tiles are masked.)
  {
    u32x4* z0 = reinterpret_cast<u32x4*>(&vb0[0][0]);
    u32x4* z1 = reinterpret_cast<u32x4*>(&vb1[0][0]);
    for (int i = t; i < 2 * HT::BYTES / 16; i += 256) {
      z0[i] = u32x4{0, 0, 0, 0};
      z1[i] = u32x4{0, 0, 0, 0};
    }
  }
  // r1, r2: this wave's half tile of steps s+1 and s+2; (lx0, ly0) .. (lx2, ly2): the
  // lengths of X and Y in steps s, s+1, s+2.
  HalfRef r0{0, 1, 0, 0}, r1{0, 1, 0, 0}, r2{0, 1, 0, 0};
  int lx0 = 0, ly0 = 0, lx1 = 0, ly1 = 0, lx2 = 0, ly2 = 0;
  uint32_t ex = 0, ey = 0;
  fetch(0, ex, ey);
  decode(0, ex, ey, r0, lx0, ly0);
  fetch(1, ex, ey);
  decode(1, ex, ey, r1, lx1, ly1);
  fetch(2, ex, ey);
  vm_wait<0>();  // Q (and the list inputs) have landed: the loop's waits count gathers only
  __syncthreads();
  {
    const Offs o0 = offsets(r0), o1 = offsets(r1);
#pragma unroll
    for (int i = 0; i < HP; ++i) gather_k(kb0, r0, o0, i);
    store_k(kb0);
#pragma unroll
    for (int i = 0; i < HP; ++i) gather_v(vb0, r0, o0, i);
    store_v(vb0);
#pragma unroll
    for (int i = 0; i < HP; ++i) gather_k(kb1, r1, o1, i);
    store_k(kb1);
    kp8 = false;  // (K of step 1 is stored)
  }
  // Step s (kc/vc: its K and V buffers, vn: V buffer of step s+1):
  //   top barrier (K(s) published) -> V(s+1) gathers under the S phase -> mid barrier
  //   (V(s) published; every wave is done with K(s)) -> K(s+2) gathers into kc under the
  //   PV phase.
  // A shared step gives every wave both half tiles (64 keys); a private step gives each
  // wave pair its own query block's half tile.
  // (FP8: kn is K of step s+1, decoded into LDS at the end of the S phase; V of step s+1
  // is decoded into vn at the end of the PV phase)
  auto step = [&](char (*kc)[HT::BYTES], char (*kn)[HT::BYTES], char (*vc)[HT::BYTES],
                  char (*vn)[HT::BYTES], int s, bool kShared) {
    wait_keep_next();
    lds_barrier();
    decode(s + 2, ex, ey, r2, lx2, ly2);
    fetch(s + 3, ex, ey);
    const int lx = lx0, ly = ly0;
    const int len = kShared ? lx : (mine ? ly : lx);
    // Every wave runs the math of every step (a wave without rows or without a tile
    // computes on masked data and writes nothing), so that the gathers can sit between its
    // MFMAs without any branch around them.
    const Offs o1 = offsets(r1), o2 = offsets(r2);
    auto dma_v = [&](int g) {
      if (g % 2 == 0 && g / 2 < HP) {
        sched_fence();
        gather_v(vn, r1, o1, g / 2);
      }
    };
    auto dma_k = [&](int g) {
      if (g % 2 == 0 && g / 2 < HP) {
        sched_fence();
        gather_k(kc, r2, o2, g / 2);
      }
    };
    typename RowState<D>::Mid md;
    f32x16 sacc[2];
    if constexpr (GATHER_ONLY) {
#pragma unroll
      for (int i = 0; i < HP; ++i) gather_v(vn, r1, o1, i);
      wait_keep_next();
      lds_barrier();
#pragma unroll
      for (int i = 0; i < HP; ++i) gather_k(kc, r2, o2, i);
      (void)md;
      (void)sacc;
      (void)len;
      (void)dma_v;
      (void)dma_k;
    } else {
    // S phase
    if constexpr (D == 128) {
      if (kShared) st.pairA(kc[0] + kofs, kc[1] + kofs, lx, c, h2, dma_v, md);
      else st.singleA(kc[mine] + kofs, len, c, h2, dma_v, md);
    } else {
#pragma unroll
      for (int i = 0; i < HP; ++i) gather_v(vn, r1, o1, i);
      if (kShared) {
        sacc[0] = st.scores(kc[0] + kofs, lx, h2);
        sacc[1] = st.scores(kc[1] + kofs, ly, h2);
      } else {
        sacc[0] = st.scores(kc[mine] + kofs, len, h2);
      }
    }
    store_k(kn);
    wait_keep_next();
    lds_barrier();
    // PV phase
    if constexpr (D == 128) {
      if (kShared) st.pairB(vc[0] + vofs, vc[1] + vofs, ly, c, h2, dma_k, md);
      else st.singleB(vc[mine] + vofs, dma_k, md);
    } else {
#pragma unroll
      for (int i = 0; i < HP; ++i) gather_k(kc, r2, o2, i);
      if (kShared) st.template update<2>(sacc, vc[0] + vofs, vc[1] + vofs, c);
      else st.template update<1>(sacc, vc[mine] + vofs, vc[mine] + vofs, c);
    }
    store_v(vn);
    }
    r1 = r2;
    lx0 = lx1;
    ly0 = ly1;
    lx1 = lx2;
    ly1 = ly2;
  };
  int s = 0;
  for (; s < nsh2; s += 2) {
    step(kb0, kb1, vb0, vb1, s, true);
    step(kb1, kb0, vb1, vb0, s + 1, true);
  }
  for (; s < nsteps; s += 2) {
    step(kb0, kb1, vb0, vb1, s, false);
    step(kb1, kb0, vb1, vb0, s + 1, false);
  }
  vm_wait<0>();  // no gather may still be writing this workgroup's LDS when it exits

  if constexpr (GATHER_ONLY) return;
  const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
  if (qrow < qlen) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.o + h * a.ohs + (t0 + qrow) * a.ots;
#pragma unroll
    for (int dt = 0; dt < RowState<D>::ND; ++dt)
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

namespace {

template <int D, bool PERSIST, bool GATHER_ONLY = false>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  const int G = a.H * a.pairs;
  const int grid = 8 * cdiv(G, 8);
  hipLaunchKernelGGL((attn_fwd_kernel<D, PERSIST, GATHER_ONLY>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_persistent(const pbsa_dims& d, TokIn q, const pbsa_cache& c,
                                      TokIn ck, TokIn cv, const int32_t* sel, TokOut o,
                                      float* lse, hipStream_t s, bool gather_only) {
  FwdArgs a{};
  const int nb = nb_of(d);
  a.q = q.p; a.qts = q.ts; a.qhs = q.hs;
  a.o = o.p; a.ots = o.ts; a.ohs = o.hs;
  a.lse = lse;
  a.lse_hs = static_cast<int64_t>(d.chunk_frames) * d.frame_tokens;
  a.ck = static_cast<const uint16_t*>(c.k);
  a.cv = static_cast<const uint16_t*>(c.v);
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
  if (gather_only)
    return d.head_dim == 128 ? launch<128, true, true>(a, s) : launch<64, true, true>(a, s);
  return d.head_dim == 128 ? launch<128, true>(a, s) : launch<64, true>(a, s);
}

hipError_t launch_attn_fwd_fp8(const pbsa_dims& d, TokIn q, const pbsa_cache& c, TokIn ck,
                               TokIn cv, const int32_t* sel, TokOut o, float* lse,
                               hipStream_t s) {
  FwdArgs a{};
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
  const int G = a.H * a.pairs;
  hipLaunchKernelGGL((attn_fwd_kernel<128, true, false, true>), dim3(8 * cdiv(G, 8)), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_2lvl(const pbsa_dims& d, int chunks, TokIn q, TokIn k, TokIn v,
                                const int32_t* sel, const int32_t* nsel, int max_sel, TokOut o,
                                float* lse, hipStream_t s) {
  FwdArgs a{};
  const int nb = nb_of(d);
  a.q = q.p; a.qts = q.ts; a.qhs = q.hs;
  a.o = o.p; a.ots = o.ts; a.ohs = o.hs;
  a.lse = lse;
  a.lse_hs = static_cast<int64_t>(chunks) * d.chunk_frames * d.frame_tokens;
  a.xk = k.p; a.xv = v.p; a.xts = k.ts; a.xhs = k.hs;
  a.sel = sel;
  a.nsel = nsel;
  a.sel_stride = max_sel;
  a.nq = chunks * d.chunk_frames * nb;
  a.n = d.frame_tokens;
  a.nb = nb;
  a.H = d.heads;
  a.pairs = cdiv(a.nq, 2);
  a.scale = d.scale;
  a.slots = 0;
  return d.head_dim == 128 ? launch<128, false>(a, s) : launch<64, false>(a, s);
}

}  // namespace pbsa
