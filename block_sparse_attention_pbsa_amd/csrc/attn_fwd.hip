// Attention over selected KV blocks with an online softmax (fine stage of PBSA).
//
// Sparse Forcing (gist.science) 2.C and the Chinese page's 2.2: each query attends to all
// persistent blocks and to its query block's top-K window blocks (plus, here, the current
// chunk); with the selection fixed this is softmax attention restricted by a block mask,
// computed block by block with a running max and sum (flash-style).  The trainable
// two-level mode attends to a per-query-block list over the whole clip instead.
//
// gfx950 design.  One workgroup = two 64-token query blocks of one head (A and B), four
// waves of 32 query rows.  The KV blocks every query block of the head attends (the
// persistent memory and the chunk itself) are gathered once for both; then each query
// block's own routed window blocks.  Each step gathers two KV blocks (two shared ones, or
// A's and B's routed ones).  Workgroups are numbered so that the eight XCDs each take a
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
//   * the next step's global loads are issued before the current step's math.
// Softmax runs in base 2 with scale*log2(e) folded in (v_exp_f32), P is packed to bf16 with
// v_cvt_pk_bf16_f32, and the running max is raised lazily; accumulators are fp32.
#include "attn_common.h"

namespace pbsa {

struct FwdArgs {
  const uint16_t* q;
  int64_t qts, qhs;
  uint16_t* o;
  int64_t ots, ohs;
  float* lse;
  int64_t lse_hs;      // tokens per head in lse
  // persistent-mode cache (unused in the two-level mode)
  const uint16_t* ck;
  const uint16_t* cv;
  const int32_t* bid;
  const int32_t* blen;
  int slots, C, W;
  // token-layout K/V: the current chunk (persistent mode) or the clip (two-level mode)
  const uint16_t* xk;
  const uint16_t* xv;
  int64_t xts, xhs;
  const int32_t* sel;   // [H][nq][sel_stride]
  const int32_t* nsel;  // two-level: [H][nq]
  int sel_stride;
  int nq, n, nb, H, pairs;
  float scale;
};

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

// A half tile to gather: wave-uniform base (bytes), row stride (bytes) and valid rows.
// Full scheduling fence (the compiler may not move instructions across it).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait until this wave's gathers into LDS have landed.  The barrier that follows makes
// them visible to the other waves; the compiler does not add this wait by itself (a
// barrier's release only covers LDS instructions), so every step barrier needs it.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// 16 bytes per lane from global memory straight into LDS (lane l writes lds + 16 l; the
// LDS address must be wave-uniform).
__device__ __forceinline__ void lds_dma16(const char* src, char* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

struct HalfRef {
  const char* k;
  const char* v;
  uint32_t stride;
  int len;  // 0 = nothing to gather
};

// Online-softmax state of one wave (32 query rows, this lane's row = column c32).
template <int D>
struct RowState {
  static constexpr int NS = D / 16, ND = D / 32;
  u32x4 qreg[NS];
  f32x16 acc[ND];
  float m_run, l_run;

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
  // Online softmax of one score tile without touching the accumulators: raises the running
  // max when some row's new max exceeds it by more than 2^8 in exp2 units (so exp2
  // arguments stay <= 8), folds the factor into l_run and returns it through alpha (the
  // caller rescales acc when the result is true), and packs P to bf16 for the PV step.
  __device__ __forceinline__ bool softmax(const f32x16& sa, float c, u32x4 (&pb)[2],
                                          float& alpha) {
    float mx = sa[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sa[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool up = __any(mx * c > m_run * c + 8.f);
    const float m_new = up ? fmaxf(m_run, mx) : m_run;
    alpha = up ? __builtin_amdgcn_exp2f(m_run * c - m_new * c) : 1.f;
    m_run = m_new;
    const float m_off = m_new * c;
    float p[16];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(sa[r], c, -m_off));
      psum += p[r];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 4; ++e) pb[t2][e] = pack_bf16x2(p[8 * t2 + 2 * e], p[8 * t2 + 2 * e + 1]);
    return up;
  }
  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
  }
  __device__ __forceinline__ void pvmma(const u32x4 (&pb)[2], const char* vb) {
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
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(vop[dt], pb[t2], acc[dt]);
    }
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
  // other tile.  Stage 0: in-lane row max; 1: max with lane l^32 (gfx950 permlane swap, no
  // LDS round trip), lazy raise of the running max (by more than 2^8 in exp2 units) and
  // the factor alpha folded into l_run; 2..5: four exponentials each; 6: bf16 packing
  // and the row sum.
  struct Soft {
    float mx, m_off, alpha, psum;
    float p[16];
    u32x4 pb[2];
    bool up;
  };
  __device__ __forceinline__ void stage(int k, const f32x16& sa, Soft& so, float c) {
    if (k == 0) {
      float mx = fmaxf(sa[0], sa[1]);
#pragma unroll
      for (int r = 2; r < 16; ++r) mx = fmaxf(mx, sa[r]);
      so.mx = mx;
    } else if (k == 1) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(so.mx),
                                                       __float_as_uint(so.mx), false, false);
      const float mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      so.up = __any(mx * c > m_run * c + 8.f);
      const float m_new = so.up ? fmaxf(m_run, mx) : m_run;
      so.alpha = so.up ? __builtin_amdgcn_exp2f(m_run * c - m_new * c) : 1.f;
      m_run = m_new;
      so.m_off = m_new * c;
    } else if (k <= 5) {
      const int r0 = 4 * (k - 2);
#pragma unroll
      for (int r = r0; r < r0 + 4; ++r) so.p[r] = __builtin_amdgcn_exp2f(fmaf(sa[r], c, -so.m_off));
    } else {
      float ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) ps += so.p[r];
      l_run = l_run * so.alpha + ps;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          so.pb[t2][e] = pack_bf16x2(so.p[8 * t2 + 2 * e], so.p[8 * t2 + 2 * e + 1]);
    }
  }

  // One half tile (a private step): the next step's gather instructions and the V reads
  // ride under the S MFMAs; the softmax cannot overlap this wave's own MFMAs.
  template <class Dma>
  __device__ __forceinline__ void single(const char* kb, const char* vb, int len, float c,
                                         int h2, Dma&& dma) {
    u32x4 kop[NS];
    kread(kb, kop);
    f32x16 sa = {};
    u32x4 vop[2 * ND];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      sa = mfma32(kop[i], qreg[i], sa);
      dma(i);
      if (i < 2 * ND) vop[i] = vread(vb, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask(sa, len, h2);
    Soft so;
#pragma unroll
    for (int k = 0; k < 7; ++k) stage(k, sa, so, c);
    asm volatile("" ::"v"(so.pb[0]), "v"(so.pb[1]));
    if (so.up) rescale(so.alpha);
#pragma unroll
    for (int j = 0; j < 2 * ND; ++j) acc[j % ND] = mfma32(vop[j], so.pb[j / ND], acc[j % ND]);
  }

  // Two half tiles (X then Y) software-pipelined inside the wave, in explicit groups the
  // scheduler may not merge: the next step's gather instructions (dma(i)) and the K reads
  // of Y ride under the S MFMAs of X (issued in one burst they would stall the wave); each
  // S MFMA of Y carries one softmax stage of X and the V reads of X; each PV MFMA of X
  // carries one softmax stage of Y and the V reads of Y.  The rare accumulator rescales
  // and tail masks sit between the phases.
  template <class Dma>
  __device__ __forceinline__ void pair(const char* kx, const char* ky, const char* vx,
                                       const char* vy, int lx, int ly, float c, int h2,
                                       Dma&& dma) {
    static_assert(NS == 8 && ND == 4, "the pipelined pair is laid out for head_dim 128");
    u32x4 kop[NS], kopy[NS];
    kread(kx, kop);
    f32x16 sx = {};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      sx = mfma32(kop[i], qreg[i], sx);
      dma(i);
      kopy[i] = *reinterpret_cast<const u32x4*>(ky + 512 * i);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask(sx, lx, h2);
    Soft so;
    u32x4 vop[2 * ND];
    f32x16 sy = {};
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      sy = mfma32(kopy[i], qreg[i], sy);
      if (i < 7) stage(i, sx, so, c);
      vop[i] = vread(vx, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the exponentials of X stay in the groups above (not sunk past the branch)
    asm volatile("" ::"v"(so.pb[0]), "v"(so.pb[1]));
    if (so.up) rescale(so.alpha);
    mask(sy, ly, h2);
    Soft sv;
    u32x4 vopy[2 * ND];
#pragma unroll
    for (int j = 0; j < 2 * ND; ++j) {
      acc[j % ND] = mfma32(vop[j], so.pb[j / ND], acc[j % ND]);
      if (j < 7) stage(j, sy, sv, c);
      vopy[j] = vread(vy, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"v"(sv.pb[0]), "v"(sv.pb[1]));
    if (sv.up) rescale(sv.alpha);
#pragma unroll
    for (int j = 0; j < 2 * ND; ++j) acc[j % ND] = mfma32(vopy[j], sv.pb[j / ND], acc[j % ND]);
  }

  // Online-softmax update with NT score tiles (32 keys each) and their V half tiles.
  // The running max only moves when some row's new max exceeds it by more than 2^8 in
  // exp2 units, so the rescale of the accumulators is rare; exp2 arguments stay <= 8.
  template <int NT>
  __device__ __forceinline__ void update(f32x16* sacc, const char* v0, const char* v1, float c) {
    float mx = sacc[0][0];
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__any(mx * c > m_run * c + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run * c - m_new * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
    }
    const float m_off = m_run * c;
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

// 1-D grid of 8 * ceil(H * pairs / 8) workgroups of 256 threads.
template <int D, bool PERSIST>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(FwdArgs a) {
  using HT = HalfTile<D>;
  // Two buffers of four half tiles each (K of X, K of Y, V of X, V of Y): one step's
  // tiles are gathered straight into LDS while the previous step's are used.
  __shared__ __attribute__((aligned(1024))) char buf0[4][HT::BYTES];
  __shared__ __attribute__((aligned(1024))) char buf1[4][HT::BYTES];
  extern __shared__ int2 lists[];
  __shared__ int wave_cnt[4];
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
  int cntA, cntB;

  // Block lists in LDS as (byte offset, valid rows | kind << 16): kind 0 is a cache slot
  // (offset from the head's cache base), kind 1 a block of the token tensors xk/xv
  // (offset from the head's base there).  Shared list (persistent mode): occupied P slots
  // in slot order, then the chunk's blocks.  Private lists: A's and B's routed blocks.
  constexpr uint32_t kCacheBlockBytes = kBlock * D * 2;
  const uint32_t xrow = static_cast<uint32_t>(a.xts * 2);
  auto tok_entry = [&](int g) {
    const int f = g / a.nb, jj = g - f * a.nb;
    const uint32_t tok = static_cast<uint32_t>(f) * a.n + kBlock * jj;
    return int2{static_cast<int>(tok * xrow), block_len(jj, a.n) | (1 << 16)};
  };
  int2* shared_list = lists;
  int2* listA = lists + (PERSIST ? a.C + a.nq : 0);
  int2* listB = listA + a.sel_stride;
  int nshared = 0;
  if (PERSIST) {
    if (t == 0) n_list = 0;
    __syncthreads();
    const int32_t* bh = a.bid + static_cast<int64_t>(h) * a.slots;
    const int32_t* lh = a.blen + static_cast<int64_t>(h) * a.slots;
    for (int s0 = 0; s0 < a.C; s0 += 256) {
      const int s = s0 + t;
      const bool valid = s < a.C && bh[s] >= 0;
      const unsigned long long m = __ballot(valid);
      if (l == 0) wave_cnt[w] = __popcll(m);
      __syncthreads();
      int off = n_list;
      for (int u = 0; u < w; ++u) off += wave_cnt[u];
      if (valid)
        shared_list[off + __popcll(m & ((1ull << l) - 1ull))] =
            int2{static_cast<int>(s * kCacheBlockBytes), lh[s]};
      __syncthreads();
      if (t == 0) n_list += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
      __syncthreads();
    }
    const int nP = __builtin_amdgcn_readfirstlane(n_list);
    for (int b = t; b < a.nq; b += 256) shared_list[nP + b] = tok_entry(b);
    nshared = nP + a.nq;
  }
  // private lists; routed ids are ascending with -1 padding at the end (persistent) or
  // counted by nsel (two-level)
  {
    const int32_t* sa = a.sel + (static_cast<int64_t>(h) * a.nq + rA) * a.sel_stride;
    const int32_t* sb = a.sel + (static_cast<int64_t>(h) * a.nq + rB) * a.sel_stride;
    const int na = PERSIST ? a.sel_stride : a.nsel[static_cast<int64_t>(h) * a.nq + rA];
    const int nbb = rB >= a.nq ? 0 : PERSIST ? a.sel_stride
                                             : a.nsel[static_cast<int64_t>(h) * a.nq + rB];
    auto entry = [&](int g) {
      if (!PERSIST) return tok_entry(g);
      const int f = g / a.nb, jj = g - f * a.nb;
      const int slot = a.C + (f % a.W) * a.nb + jj;
      return int2{static_cast<int>(slot * kCacheBlockBytes),
                  a.blen[static_cast<int64_t>(h) * a.slots + slot]};
    };
    for (int j = t; j < a.sel_stride; j += 256) {
      const int ga = j < na ? sa[j] : -1;
      const int gb = j < nbb ? sb[j] : -1;
      listA[j] = ga >= 0 ? entry(ga) : int2{0, 0};
      listB[j] = gb >= 0 ? entry(gb) : int2{0, 0};
    }
    int ca = 0, cb = 0;
    for (int j = l; j < a.sel_stride; j += 64) {
      ca += (j < na) && sa[j] >= 0;
      cb += (j < nbb) && sb[j] >= 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      ca += __shfl_xor(ca, o, 64);
      cb += __shfl_xor(cb, o, 64);
    }
    cntA = __builtin_amdgcn_readfirstlane(ca);
    cntB = __builtin_amdgcn_readfirstlane(cb);
  }
  __syncthreads();
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
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  const char* ck_h = reinterpret_cast<const char*>(a.ck) +
                     static_cast<int64_t>(h) * a.slots * kCacheBlockBytes;
  const char* cv_h = reinterpret_cast<const char*>(a.cv) +
                     static_cast<int64_t>(h) * a.slots * kCacheBlockBytes;
  const char* xk_h = reinterpret_cast<const char*>(a.xk + h * a.xhs);
  const char* xv_h = reinterpret_cast<const char*>(a.xv + h * a.xhs);
  // list entries are wave-uniform: readfirstlane keeps them (and the gather base
  // addresses) in scalar registers
  auto ref_of = [&](int2 e, int half, HalfRef& hr) {
    const uint32_t off = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(e.x));
    const int y = __builtin_amdgcn_readfirstlane(e.y);
    const bool tok = (y >> 16) != 0;
    const uint32_t stride = tok ? xrow : 2 * D;
    const uint32_t o = off + 32 * half * stride;
    const int len = (y & 0xffff) - 32 * half;
    hr.k = (tok ? xk_h : ck_h) + o;
    hr.v = (tok ? xv_h : cv_h) + o;
    hr.stride = stride;
    hr.len = len < 0 ? 0 : (len < 32 ? len : 32);
  };
  // This wave's half tile of step s (see the gather below) and the lengths of X and Y.
  auto refs = [&](int s, HalfRef& mineref, int& lenX, int& lenY) {
    HalfRef x{nullptr, nullptr, 0, 0}, y{nullptr, nullptr, 0, 0};
    if (s < nshared) {
      const int2 e = shared_list[s];
      ref_of(e, 0, x);
      ref_of(e, 1, y);
    } else if (s >= nsh2) {
      const int j = s - nsh2, half = j & 1, blk = j >> 1;
      if (blk < cntA) ref_of(listA[blk], half, x);
      if (blk < cntB) ref_of(listB[blk], half, y);
    }
    lenX = x.len;
    lenY = y.len;
    const bool use_y = (w & 1) != 0;
    mineref.k = use_y ? y.k : x.k;
    mineref.v = use_y ? y.v : x.v;
    mineref.stride = use_y ? y.stride : x.stride;
    mineref.len = use_y ? y.len : x.len;
  };

  // Gather: wave w fills half tile w of a buffer (0: K of X, 1: K of Y, 2: V of X, 3: V of
  // Y).  Rows past the valid length re-read the last valid row (finite data that the mask
  // or a zero probability removes).
  const bool kwave = w < 2;
  const uint32_t rowl = kwave ? (l & 15) : (l >> 2);
  const uint32_t colb = 16u * (kwave ? (l >> 4) : (l & 3));
  // One gather instruction (piece p of this wave's half tile).
  auto gather_piece = [&](char (*bufp)[HT::BYTES], const HalfRef& hr, int p) {
    if (hr.len == 0) return;
    const char* g = kwave ? hr.k : hr.v;
    const uint32_t last = static_cast<uint32_t>(hr.len - 1);
    const int kr = p / (HT::PIECES / 2), kc = 64 * (p % (HT::PIECES / 2));
    const int vr = p % 2, vc = 64 * (p / 2);
    const uint32_t row = ((kwave ? kr : vr) ? 16u : 0u) + rowl;
    const uint32_t vo = min(row, last) * hr.stride + colb;
    lds_dma16(g + (kwave ? kc : vc) + vo, bufp[w] + 1024 * p);
  };
  auto gather = [&](char (*bufp)[HT::BYTES], const HalfRef& hr) {
    if (hr.len == 0) return;
    const char* g = kwave ? hr.k : hr.v;
    const uint32_t last = static_cast<uint32_t>(hr.len - 1);
    const uint32_t v0 = min(rowl, last) * hr.stride + colb;
    const uint32_t v1 = min(16u + rowl, last) * hr.stride + colb;
    char* dst = bufp[w];
#pragma unroll
    for (int p = 0; p < HT::PIECES; ++p) {
      // K piece p: rows 16 (p / (PIECES/2)) .., chunks 4 (p % (PIECES/2)) ..
      // V piece p: rows 16 (p % 2) .., segment p / 2
      const int kr = p / (HT::PIECES / 2), kc = 64 * (p % (HT::PIECES / 2));
      const int vr = p % 2, vc = 64 * (p / 2);
      const uint32_t vo = (kwave ? kr : vr) ? v1 : v0;
      const char* src = g + (kwave ? kc : vc) + vo;
      lds_dma16(src, dst + 1024 * p);
    }
  };

  // this lane's LDS read offsets inside a half tile
  const int kofs = (c32 >> 4) * HT::KRG + 256 * h2 + 16 * (c32 & 15);
  const int g16 = l >> 4, i16 = l & 15;
  const int vofs = (4 * (g16 >> 1) + (i16 >> 2)) * 64 + 32 * (g16 & 1) + 8 * (i16 & 3);

  // Buffers start zeroed: a half tile that a step leaves empty is still read (its scores
  // are masked and its probabilities are zero) and must hold finite values.
  {
    u32x4* z0 = reinterpret_cast<u32x4*>(&buf0[0][0]);
    u32x4* z1 = reinterpret_cast<u32x4*>(&buf1[0][0]);
    for (int i = t; i < 4 * HT::BYTES / 16; i += 256) {
      z0[i] = u32x4{0, 0, 0, 0};
      z1[i] = u32x4{0, 0, 0, 0};
    }
  }
  HalfRef next{nullptr, nullptr, 0, 0};
  int nX = 0, nY = 0;
  __syncthreads();
  if (nsteps > 0) {
    refs(0, next, nX, nY);
    gather(buf0, next);
  }
  // One step: wait for this step's tiles (buffer cur), start the next step's gathers into
  // the other buffer (whose readers, the previous step, have all passed the barrier), then
  // the math.  A shared step gives every wave both half tiles (64 keys); a private step
  // gives each wave pair its own query block's half tile.
  auto step = [&](char (*cur)[HT::BYTES], char (*nxt)[HT::BYTES], int s, bool kShared) {
    dma_wait();
    __syncthreads();
    const int lx = nX, ly = nY;
    const bool more = s + 1 < nsteps;
    if (more) refs(s + 1, next, nX, nY);
    const int len = kShared ? lx : (mine ? ly : lx);
    // with head_dim 128 the gathers ride inside the math (dma below); otherwise, or when
    // this wave has no math in this step, they are issued here
    const bool inside = D == 128 && qlen > 0 && len > 0;
    if (more && !inside) gather(nxt, next);
    if (!inside && D == 128) return;
    if (qlen <= 0) return;
    auto dma = [&](int p) {
      if (more && p < HT::PIECES) {
        sched_fence();
        gather_piece(nxt, next, p);
      }
    };
    if (kShared) {
      if (lx > 0) {
        if constexpr (D == 128) {
          st.pair(cur[0] + kofs, cur[1] + kofs, cur[2] + vofs, cur[3] + vofs, lx, ly, c, h2, dma);
        } else {
          f32x16 sacc[2];
          sacc[0] = st.scores(cur[0] + kofs, lx, h2);
          sacc[1] = st.scores(cur[1] + kofs, ly, h2);
          st.template update<2>(sacc, cur[2] + vofs, cur[3] + vofs, c);
        }
      }
    } else {
      if (len > 0) {
        if constexpr (D == 128) {
          st.single(cur[mine] + kofs, cur[2 + mine] + vofs, len, c, h2, dma);
        } else {
          f32x16 sacc[1];
          sacc[0] = st.scores(cur[mine] + kofs, len, h2);
          st.template update<1>(sacc, cur[2 + mine] + vofs, cur[2 + mine] + vofs, c);
        }
      }
    }
  };
  int s = 0;
  for (; s < nsh2; s += 2) {
    step(buf0, buf1, s, true);
    step(buf1, buf0, s + 1, true);
  }
  for (; s < nsteps; s += 2) {
    step(buf0, buf1, s, false);
    step(buf1, buf0, s + 1, false);
  }

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
    if (h2 == 0) a.lse[h * a.lse_hs + t0 + qrow] = st.m_run * a.scale + logf(l_tot);
  }
}

namespace {

template <int D, bool PERSIST>
hipError_t launch(const FwdArgs& a, size_t lds, hipStream_t s) {
  const int G = a.H * a.pairs;
  const int grid = 8 * cdiv(G, 8);
  hipLaunchKernelGGL((attn_fwd_kernel<D, PERSIST>), dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_persistent(const pbsa_dims& d, TokIn q, const pbsa_cache& c,
                                      TokIn ck, TokIn cv, const int32_t* sel, TokOut o,
                                      float* lse, hipStream_t s) {
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
  const size_t lds = static_cast<size_t>(d.capacity + a.nq + 2 * d.topk) * sizeof(int2);
  return d.head_dim == 128 ? launch<128, true>(a, lds, s) : launch<64, true>(a, lds, s);
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
  const size_t lds = static_cast<size_t>(2 * max_sel) * sizeof(int2);
  return d.head_dim == 128 ? launch<128, false>(a, lds, s) : launch<64, false>(a, lds, s);
}

}  // namespace pbsa
