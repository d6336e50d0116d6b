// Attention over selected KV blocks with an online softmax (fine stage of PBSA).
//
// Sparse Forcing (gist.science) 2.C and the Chinese page's 2.2: each query attends to all
// persistent blocks and to its query block's top-K window blocks (plus, here, the current
// chunk); with the selection fixed this is softmax attention restricted by a block mask,
// computed block by block with a running max and sum (flash-style).  The trainable
// two-level mode attends to a per-query-block list over the whole clip instead.
//
// gfx950 design.  One workgroup = one (head, 64-token query block), two waves of 32 query
// rows.  Per KV block (64 keys, possibly fewer in a frame's tail block):
//   * the block is gathered from HBM/L2 with 16-byte loads into LDS: K row-major, V
//     transposed (channel-major) so both MFMA operands read 16 contiguous bytes;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (Q lives in registers as the B operand), so
//     each lane holds 32 scores of ONE query row: the row max/sum are in-lane plus one
//     exchange with lane l^32;
//   * O^T += V^T P^T on the same MFMA, P converted to bf16 straight from the S^T
//     accumulators (the contraction order over keys is permuted identically in both
//     operands, which leaves the sum unchanged);
//   * the next block's global loads are issued before the current block's math.
// Softmax runs in base 2 with scale*log2(e) folded in; accumulators are fp32.
#include "attn_common.h"

namespace pbsa {

namespace {

struct KvRef {
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;  // elements between token rows
  int len;         // valid rows (1..64)
};

// Persistent mode: P slots, then the routed window blocks, then the chunk's own blocks.
struct PersistentSrc {
  const uint16_t* ck;    // cache K of this head, slot-major
  const uint16_t* cv;
  const int32_t* bid;    // block_id of this head
  const int32_t* blen;   // len of this head
  const int32_t* sel;    // routed ids of this query block
  const uint16_t* xk;    // chunk K/V of this head
  const uint16_t* xv;
  int64_t xts;
  int C, K, W, nb, n, nq, D;
  __device__ int count() const { return C + K + nq; }
  __device__ bool get(int i, KvRef& o) const {
    if (i < C) {
      if (bid[i] < 0) return false;
      const int64_t off = static_cast<int64_t>(i) * kBlock * D;
      o = KvRef{ck + off, cv + off, D, blen[i]};
      return true;
    }
    i -= C;
    if (i < K) {
      const int g = sel[i];
      if (g < 0) return false;
      const int f = g / nb, j = g - f * nb;
      const int slot = C + (f % W) * nb + j;
      const int64_t off = static_cast<int64_t>(slot) * kBlock * D;
      o = KvRef{ck + off, cv + off, D, blen[slot]};
      return true;
    }
    i -= K;
    const int f = i / nb, j = i - f * nb;
    const int64_t t0 = static_cast<int64_t>(f) * n + kBlock * j;
    o = KvRef{xk + t0 * xts, xv + t0 * xts, xts, block_len(j, n)};
    return true;
  }
};

// Two-level mode: sel[0..cnt) global ids into the clip's token tensors.
struct ListSrc {
  const uint16_t* xk;
  const uint16_t* xv;
  int64_t xts;
  const int32_t* sel;
  int cnt, nb, n;
  __device__ int count() const { return cnt; }
  __device__ bool get(int i, KvRef& o) const {
    const int g = sel[i];
    const int f = g / nb, j = g - f * nb;
    const int64_t t0 = static_cast<int64_t>(f) * n + kBlock * j;
    o = KvRef{xk + t0 * xts, xv + t0 * xts, xts, block_len(j, n)};
    return true;
  }
};

template <class Src>
__device__ __forceinline__ int next_valid(const Src& src, int i, KvRef& kv) {
  const int cnt = src.count();
  while (i < cnt && !src.get(i, kv)) ++i;
  return i;
}

}  // namespace

// One workgroup per (query block, head).  blockDim = 128.
template <int D, class Src>
__device__ __forceinline__ void attn_fwd_block(const Src& src, const uint16_t* q, int64_t qts,
                                               int qlen, float scale, uint16_t* o, int64_t ots,
                                               float* lse) {
  constexpr int NS = D / 16;  // k-steps over channels
  constexpr int ND = D / 32;  // 32-channel output tiles
  __shared__ __attribute__((aligned(16))) uint16_t Ks[Lds<D>::ROWS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[Lds<D>::COLS];

  const int t = threadIdx.x;
  const int w = t >> 6, l = t & 63, h2 = l >> 5, c32 = l & 31;
  const int qrow = 32 * w + c32;  // this lane's query row inside the block
  const float c = scale * kLog2e;

  // Q as the B operand of S^T = K Q^T: lane holds row qrow, channels 16s + 8*h2 + [0, 8).
  u32x4 qreg[NS];
  load_row_operand<D>(qreg, q, qts, qrow, qlen, h2);

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of raw q.k for this lane's row
  float l_run = 0.f;        // this lane's share of the running sum

  Tile<D> tk, tv;
  KvRef cur;
  int i = next_valid(src, 0, cur);
  if (i < src.count()) {
    tk.load(cur.k, cur.stride, cur.len, t);
    tv.load(cur.v, cur.stride, cur.len, t);
  }
  while (i < src.count()) {
    __syncthreads();  // previous block's LDS reads are done
    tk.store_rows(Ks, t);
    tv.store_cols(Vt, t);
    const int len = cur.len;
    KvRef nxt;
    const int inext = next_valid(src, i + 1, nxt);
    __syncthreads();
    if (inext < src.count()) {  // next block's loads are in flight during the math below
      tk.load(nxt.k, nxt.stride, nxt.len, t);
      tv.load(nxt.v, nxt.stride, nxt.len, t);
    }

    // S^T tiles: keys 32*kt + acc_row(r), query column = this lane's row.
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) sacc[kt] = mfma32(rd_rows<D>(Ks, kt, s, c32, h2), qreg[s], sacc[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (32 * kt + acc_row(r, h2) >= len) sacc[kt][r] = -INFINITY;
        mx = fmaxf(mx, sacc[kt][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_off = m_new == -INFINITY ? 0.f : m_new * c;
    const float alpha = exp2f(m_run * c - m_off);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(sacc[kt][r], c, -m_off));
        sacc[kt][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;

    // O^T += V^T P^T over 4 k-steps of 16 keys.
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const u32x4 pb = pack_step(sacc, t4);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(rd_cols<D>(Vt, dt, t4, c32, h2), pb, acc[dt]);
    }
    cur = nxt;
    i = inext;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qrow < qlen) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = o + qrow * ots;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = 32 * dt + 8 * j + 4 * h2;
        u32x2 pk = {pack_bf16x2(acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv),
                    pack_bf16x2(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + ch) = pk;
      }
    if (h2 == 0) lse[qrow] = m_run * scale + logf(l_tot);
  }
}

struct FwdCommon {
  const uint16_t* q;
  int64_t qts, qhs;
  uint16_t* o;
  int64_t ots, ohs;
  float* lse;
  int64_t lse_hs;  // tokens per head in lse
  int n, nb;
  float scale;
};

template <int D>
__global__ void __launch_bounds__(128)
    attn_fwd_persistent_kernel(FwdCommon cm, const uint16_t* ck, const uint16_t* cv,
                               const int32_t* bid, const int32_t* blen, const int32_t* sel,
                               const uint16_t* xk, const uint16_t* xv, int64_t xts, int64_t xhs,
                               int slots, int C, int K, int W, int nq) {
  const int r = blockIdx.x, h = blockIdx.y;
  const int f = r / cm.nb, j = r - f * cm.nb;
  const int64_t t0 = static_cast<int64_t>(f) * cm.n + kBlock * j;
  PersistentSrc src;
  src.ck = ck + static_cast<int64_t>(h) * slots * kBlock * D;
  src.cv = cv + static_cast<int64_t>(h) * slots * kBlock * D;
  src.bid = bid + static_cast<int64_t>(h) * slots;
  src.blen = blen + static_cast<int64_t>(h) * slots;
  src.sel = sel + (static_cast<int64_t>(h) * nq + r) * K;
  src.xk = xk + h * xhs;
  src.xv = xv + h * xhs;
  src.xts = xts;
  src.C = C;
  src.K = K;
  src.W = W;
  src.nb = cm.nb;
  src.n = cm.n;
  src.nq = nq;
  src.D = D;
  attn_fwd_block<D>(src, cm.q + h * cm.qhs + t0 * cm.qts, cm.qts, block_len(j, cm.n), cm.scale,
                    cm.o + h * cm.ohs + t0 * cm.ots, cm.ots, cm.lse + h * cm.lse_hs + t0);
}

template <int D>
__global__ void __launch_bounds__(128)
    attn_fwd_2lvl_kernel(FwdCommon cm, const uint16_t* xk, const uint16_t* xv, int64_t xts,
                         int64_t xhs, const int32_t* sel, const int32_t* nsel, int max_sel,
                         int nq) {
  const int r = blockIdx.x, h = blockIdx.y;
  const int f = r / cm.nb, j = r - f * cm.nb;
  const int64_t t0 = static_cast<int64_t>(f) * cm.n + kBlock * j;
  ListSrc src;
  src.xk = xk + h * xhs;
  src.xv = xv + h * xhs;
  src.xts = xts;
  src.sel = sel + (static_cast<int64_t>(h) * nq + r) * max_sel;
  src.cnt = nsel[static_cast<int64_t>(h) * nq + r];
  src.nb = cm.nb;
  src.n = cm.n;
  attn_fwd_block<D>(src, cm.q + h * cm.qhs + t0 * cm.qts, cm.qts, block_len(j, cm.n), cm.scale,
                    cm.o + h * cm.ohs + t0 * cm.ots, cm.ots, cm.lse + h * cm.lse_hs + t0);
}

hipError_t launch_attn_fwd_persistent(const pbsa_dims& d, TokIn q, const pbsa_cache& c,
                                      TokIn ck, TokIn cv, const int32_t* sel, TokOut o,
                                      float* lse, hipStream_t s) {
  const int nb = nb_of(d);
  const int nq = d.chunk_frames * nb;
  const int slots = static_cast<int>(slots_of(d));
  FwdCommon cm{q.p, q.ts, q.hs, o.p, o.ts, o.hs, lse,
               static_cast<int64_t>(d.chunk_frames) * d.frame_tokens, d.frame_tokens, nb, d.scale};
  dim3 grid(nq, d.heads);
  const uint16_t* kk = static_cast<const uint16_t*>(c.k);
  const uint16_t* vv = static_cast<const uint16_t*>(c.v);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_persistent_kernel<128>, grid, dim3(128), 0, s, cm, kk, vv,
                       c.block_id, c.len, sel, ck.p, cv.p, ck.ts, ck.hs, slots, d.capacity,
                       d.topk, d.window_frames, nq);
  else
    hipLaunchKernelGGL(attn_fwd_persistent_kernel<64>, grid, dim3(128), 0, s, cm, kk, vv,
                       c.block_id, c.len, sel, ck.p, cv.p, ck.ts, ck.hs, slots, d.capacity,
                       d.topk, d.window_frames, nq);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_2lvl(const pbsa_dims& d, int chunks, TokIn q, TokIn k, TokIn v,
                                const int32_t* sel, const int32_t* nsel, int max_sel, TokOut o,
                                float* lse, hipStream_t s) {
  const int nb = nb_of(d);
  const int nq = chunks * d.chunk_frames * nb;
  FwdCommon cm{q.p, q.ts, q.hs, o.p, o.ts, o.hs, lse,
               static_cast<int64_t>(chunks) * d.chunk_frames * d.frame_tokens, d.frame_tokens, nb,
               d.scale};
  dim3 grid(nq, d.heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(attn_fwd_2lvl_kernel<128>, grid, dim3(128), 0, s, cm, k.p, v.p, k.ts,
                       k.hs, sel, nsel, max_sel, nq);
  else
    hipLaunchKernelGGL(attn_fwd_2lvl_kernel<64>, grid, dim3(128), 0, s, cm, k.p, v.p, k.ts, k.hs,
                       sel, nsel, max_sel, nq);
  return hipGetLastError();
}

}  // namespace pbsa
