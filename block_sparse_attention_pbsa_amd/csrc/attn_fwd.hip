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

struct KvRef {
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;  // elements between token rows
  int len;         // valid rows; 0 = no block
};

// Online-softmax state of one wave (32 query rows, this lane's row = column c32).
template <int D>
struct RowState {
  static constexpr int NS = D / 16, ND = D / 32;
  u32x4 qreg[NS];
  f32x16 acc[ND];
  float m_run, l_run;

  // S^T for the keys of one 32-row K half tile: keys acc_row(r, h2), query = this lane's row.
  __device__ __forceinline__ f32x16 scores(const uint16_t* Ks, int len, int c32, int h2) const {
    // all K operands are read before the MFMA chain so the LDS latency is paid once
    u32x4 kop[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) kop[s] = rd_rows<D>(Ks, 0, s, c32, h2);
    f32x16 sa = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) sa = mfma32(kop[s], qreg[s], sa);
    if (len < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (acc_row(r, h2) >= len) sa[r] = -INFINITY;
    }
    return sa;
  }

  // Online-softmax update with NT score tiles (32 keys each) and their V half tiles.
  // The running max only moves when some row's new max exceeds it by more than 2^8 in
  // exp2 units, so the rescale of the accumulators is rare; exp2 arguments stay <= 8.
  template <int NT>
  __device__ __forceinline__ void update(f32x16* sacc, const uint16_t* V0, const uint16_t* V1,
                                         float c, int l) {
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
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
      const uint16_t* Vs = kt ? V1 : V0;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        u32x4 vop[ND];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vop[dt] = rd_rows_tr<D>(Vs, dt, t2, l);
        const u32x4 pb = pack_step(sacc + kt, t2);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(vop[dt], pb, acc[dt]);
      }
    }
  }
};

}  // namespace

// 1-D grid of 8 * ceil(H * pairs / 8) workgroups of 256 threads.
template <int D, bool PERSIST>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(FwdArgs a) {
  // two 32-key half tiles per step: X and Y, K and V row-major
  constexpr int HT = 32 * Lds<D>::RS;
  __shared__ __attribute__((aligned(16))) uint16_t KsX[HT];
  __shared__ __attribute__((aligned(16))) uint16_t VsX[HT];
  __shared__ __attribute__((aligned(16))) uint16_t KsY[HT];
  __shared__ __attribute__((aligned(16))) uint16_t VsY[HT];
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

  // Block lists in LDS as (handle, valid rows): handle < slots is a cache slot, otherwise
  // block (handle - slots) of the token tensors xk/xv.  Shared list (persistent mode):
  // occupied P slots in slot order, then the chunk's blocks.  Private lists: A's and B's
  // routed blocks.
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
      if (valid) shared_list[off + __popcll(m & ((1ull << l) - 1ull))] = int2{s, lh[s]};
      __syncthreads();
      if (t == 0) n_list += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
      __syncthreads();
    }
    const int nP = __builtin_amdgcn_readfirstlane(n_list);
    for (int b = t; b < a.nq; b += 256)
      shared_list[nP + b] = int2{a.slots + b, block_len(b % a.nb, a.n)};
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
    for (int j = t; j < a.sel_stride; j += 256) {
      int2 ea{-1, 0}, eb{-1, 0};
      const int ga = j < na ? sa[j] : -1;
      const int gb = j < nbb ? sb[j] : -1;
      if (ga >= 0) {
        const int f = ga / a.nb, jj = ga - f * a.nb;
        ea = PERSIST ? int2{a.C + (f % a.W) * a.nb + jj, 0} : int2{a.slots + ga, block_len(jj, a.n)};
        if (PERSIST) ea.y = a.blen[static_cast<int64_t>(h) * a.slots + ea.x];
      }
      if (gb >= 0) {
        const int f = gb / a.nb, jj = gb - f * a.nb;
        eb = PERSIST ? int2{a.C + (f % a.W) * a.nb + jj, 0} : int2{a.slots + gb, block_len(jj, a.n)};
        if (PERSIST) eb.y = a.blen[static_cast<int64_t>(h) * a.slots + eb.x];
      }
      listA[j] = ea;
      listB[j] = eb;
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
  // of A's next routed block (X) and the same half of B's (Y)
  const int nsteps = nshared + 2 * (cntA > cntB ? cntA : cntB);

  RowState<D> st;
  load_row_operand<D>(st.qreg, a.q + h * a.qhs + t0 * a.qts, a.qts, qrow, qlen, h2);
#pragma unroll
  for (int i = 0; i < RowState<D>::ND; ++i) st.acc[i] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  // handles are wave-uniform: readfirstlane keeps them (and the gather base addresses)
  // in scalar registers
  auto ref_of = [&](int2 e, int half) {
    KvRef o;
    const int hd = __builtin_amdgcn_readfirstlane(e.x);
    const int len = __builtin_amdgcn_readfirstlane(e.y) - 32 * half;
    if (hd < a.slots) {
      const int64_t off = (static_cast<int64_t>(h) * a.slots + hd) * kBlock * D + 32 * half * D;
      o = KvRef{a.ck + off, a.cv + off, D, 0};
    } else {
      const int64_t t0b = block_token0(hd - a.slots, a.nb, a.n) + 32 * half;
      const int64_t off = h * a.xhs + t0b * a.xts;
      o = KvRef{a.xk + off, a.xv + off, a.xts, 0};
    }
    o.len = len < 0 ? 0 : (len < 32 ? len : 32);
    return o;
  };
  auto refs = [&](int s, KvRef& x, KvRef& y) {
    x.len = 0;
    y.len = 0;
    if (s < nshared) {
      const int2 e = shared_list[s];
      x = ref_of(e, 0);
      y = ref_of(e, 1);
    } else {
      const int j = s - nshared, half = j & 1, blk = j >> 1;
      if (blk < cntA) x = ref_of(listA[blk], half);
      if (blk < cntB) y = ref_of(listB[blk], half);
    }
  };

  Tile<D, 256, 32> kx, vx, ky, vy;
  KvRef x, y;
  if (nsteps > 0) {
    refs(0, x, y);
    kx.load(x.k, x.stride, x.len, t);
    vx.load(x.v, x.stride, x.len, t);
    ky.load(y.k, y.stride, y.len, t);
    vy.load(y.v, y.stride, y.len, t);
  }
  for (int s = 0; s < nsteps; ++s) {
    __syncthreads();  // the previous step's LDS reads are done
    kx.store_rows(KsX, t);
    vx.store_rows(VsX, t);
    ky.store_rows(KsY, t);
    vy.store_rows(VsY, t);
    const int lenX = x.len, lenY = y.len;
    __syncthreads();
    if (s + 1 < nsteps) {  // next step's gathers are in flight during this step's math
      refs(s + 1, x, y);
      kx.load(x.k, x.stride, x.len, t);
      vx.load(x.v, x.stride, x.len, t);
      ky.load(y.k, y.stride, y.len, t);
      vy.load(y.v, y.stride, y.len, t);
    }
    if (qlen > 0) {
      // a shared step gives every wave both half tiles; a private step gives each wave
      // pair its own query block's half tile
      const bool shared_step = s < nshared;
#pragma unroll 1
      for (int it = 0; it < 2; ++it) {
        const bool use_y = shared_step ? it == 1 : mine == 1;
        const int len = (shared_step || it == 0) ? (use_y ? lenY : lenX) : 0;
        if (len > 0) {
          f32x16 sacc[1];
          sacc[0] = st.scores(use_y ? KsY : KsX, len, c32, h2);
          const uint16_t* Vs = use_y ? VsY : VsX;
          st.template update<1>(sacc, Vs, Vs, c, l);
        }
      }
    }
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
