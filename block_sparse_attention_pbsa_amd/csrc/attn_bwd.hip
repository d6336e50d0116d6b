// Backward of attention over selected blocks (trainable path), deterministic.
//
// Sparse Forcing (gist.science) 2.D / 3: the same sparse attention is used while training,
// so the kernel family must also give gradients.  With the selection held constant, the
// gradient of softmax attention is the textbook one: with P = exp(scale*S - LSE),
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// gfx950 design (no atomics, so results are bit-reproducible):
//   dq pass  -- one workgroup per (query block, head): walks its selected KV blocks like the
//               forward, recomputes S^T and dP^T on MFMA, accumulates dQ^T in registers;
//               it also writes D for its rows.
//   inverse  -- one workgroup per (KV block, head): lists, in ascending order, the query
//               blocks that selected the KV block (binary search in their sorted lists).
//   dkdv pass -- one workgroup per (KV block, head): walks that list, recomputes S and dP
//               with keys as MFMA columns, accumulates dK^T and dV^T in registers.
#include "attn_common.h"

namespace pbsa {

namespace {

struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;
  int64_t qts, qhs, kts, khs, vts, vhs, ots, ohs, dts, dhs;
  uint16_t *dq, *dk, *dv;
  int64_t dqts, dqhs, dkts, dkhs, dvts, dvhs;
  const float* lse;     // [H][T]
  const int32_t* sel;   // [H][nq][max_sel]
  const int32_t* nsel;  // [H][nq]
  float* Dw;            // workspace [H][T]
  int32_t* inv_cnt;     // workspace [H][nq]
  int32_t* inv;         // workspace [H][nq][nq]
  int64_t T;
  int nq, nb, n, F, max_sel;
  float scale;
};

}  // namespace

// ------------------------------------------------------------------ dQ pass (+ D)
template <int D>
__global__ void __launch_bounds__(128) attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[Lds<D>::ROWS];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[Lds<D>::COLS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[Lds<D>::ROWS];
  const int r = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int w = t >> 6, l = t & 63, h2 = l >> 5, c32 = l & 31;
  const int qrow = 32 * w + c32;
  const int64_t t0 = block_token0(r, a.nb, a.n);
  const int qlen = block_len(r % a.nb, a.n);
  const float c = a.scale * kLog2e;

  u32x4 qreg[NS], dreg[NS];
  load_row_operand<D>(qreg, a.q + h * a.qhs + t0 * a.qts, a.qts, qrow, qlen, h2);
  load_row_operand<D>(dreg, a.dout + h * a.dhs + t0 * a.dts, a.dts, qrow, qlen, h2);
  // D = rowsum(dO * O): this lane holds half the channels of its row, lane l^32 the rest.
  float dsum = 0.f;
  {
    u32x4 oreg[NS];
    load_row_operand<D>(oreg, a.o + h * a.ohs + t0 * a.ots, a.ots, qrow, qlen, h2);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dsum = fmaf(__uint_as_float(oreg[s][e] << 16), __uint_as_float(dreg[s][e] << 16), dsum);
        dsum = fmaf(__uint_as_float(oreg[s][e] & 0xffff0000u),
                    __uint_as_float(dreg[s][e] & 0xffff0000u), dsum);
      }
  }
  dsum += __shfl_xor(dsum, 32, 64);
  const float* lse_h = a.lse + h * a.T + t0;
  const float lse2 = qrow < qlen ? lse_h[qrow] * kLog2e : 0.f;
  if (qrow < qlen && h2 == 0) a.Dw[h * a.T + t0 + qrow] = dsum;

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

  const int32_t* sel = a.sel + (static_cast<int64_t>(h) * a.nq + r) * a.max_sel;
  const int cnt = a.nsel[static_cast<int64_t>(h) * a.nq + r];
  const uint16_t* kh = a.k + h * a.khs;
  const uint16_t* vh = a.v + h * a.vhs;
  Tile<D> tk, tv;
  int g = cnt > 0 ? sel[0] : 0;
  if (cnt > 0) {
    const int64_t k0 = block_token0(g, a.nb, a.n);
    const int len = block_len(g % a.nb, a.n);
    tk.load(kh + k0 * a.kts, a.kts, len, t);
    tv.load(vh + k0 * a.vts, a.vts, len, t);
  }
  for (int i = 0; i < cnt; ++i) {
    __syncthreads();
    tk.store_rows(Ks, t);
    tk.store_cols(Kt, t);
    tv.store_rows(Vs, t);
    const int len = block_len(g % a.nb, a.n);
    __syncthreads();
    if (i + 1 < cnt) {
      g = sel[i + 1];
      const int64_t k0 = block_token0(g, a.nb, a.n);
      const int ln = block_len(g % a.nb, a.n);
      tk.load(kh + k0 * a.kts, a.kts, ln, t);
      tv.load(vh + k0 * a.vts, a.vts, ln, t);
    }
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x16{};
      pacc[kt] = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sacc[kt] = mfma32(rd_rows<D>(Ks, kt, s, c32, h2), qreg[s], sacc[kt]);
        pacc[kt] = mfma32(rd_rows<D>(Vs, kt, s, c32, h2), dreg[s], pacc[kt]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const bool ok = 32 * kt + acc_row(rr, h2) < len;
        const float p = ok ? exp2f(fmaf(sacc[kt][rr], c, -lse2)) : 0.f;
        sacc[kt][rr] = p * (pacc[kt][rr] - dsum);  // dS^T
      }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const u32x4 pb = pack_step(sacc, t4);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(rd_cols<D>(Kt, dt, t4, c32, h2), pb, acc[dt]);
    }
  }
  if (qrow < qlen) {
    uint16_t* out = a.dq + h * a.dqhs + (t0 + qrow) * a.dqts;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = 32 * dt + 8 * j + 4 * h2;
        u32x2 pk = {pack_bf16x2(acc[dt][4 * j] * a.scale, acc[dt][4 * j + 1] * a.scale),
                    pack_bf16x2(acc[dt][4 * j + 2] * a.scale, acc[dt][4 * j + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(out + ch) = pk;
      }
  }
}

// ------------------------------------------------------------------ inverse lists
// grid (nq, H), 256 threads: inv[h][g] = ascending query blocks whose list holds g.
__global__ void __launch_bounds__(256) attn_bwd_inverse_kernel(BwdArgs a) {
  __shared__ int wave_cnt[4];
  const int g = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int w = t >> 6, l = t & 63;
  // a query block of chunk i (1-based) sees frames < F*i, so frame f is first visible to
  // chunk f/F + 1
  const int f = g / a.nb;
  const int r0 = (f / a.F) * a.F * a.nb;
  int32_t* out = a.inv + (static_cast<int64_t>(h) * a.nq + g) * a.nq;
  int total = 0;
  for (int base = r0; base < a.nq; base += 256) {
    const int r = base + t;
    bool found = false;
    if (r < a.nq) {
      const int32_t* s = a.sel + (static_cast<int64_t>(h) * a.nq + r) * a.max_sel;
      int lo = 0, hi = a.nsel[static_cast<int64_t>(h) * a.nq + r];
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s[mid] < g) lo = mid + 1;
        else hi = mid;
      }
      found = lo < a.nsel[static_cast<int64_t>(h) * a.nq + r] && s[lo] == g;
    }
    const unsigned long long m = __ballot(found);
    const int below = __popcll(m & ((1ull << l) - 1ull));
    if (l == 0) wave_cnt[w] = __popcll(m);
    __syncthreads();
    int off = total;
    for (int u = 0; u < w; ++u) off += wave_cnt[u];
    if (found) out[off + below] = r;
    total += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    __syncthreads();
  }
  if (t == 0) a.inv_cnt[static_cast<int64_t>(h) * a.nq + g] = total;
}

// ------------------------------------------------------------------ dK/dV pass
template <int D>
__global__ void __launch_bounds__(128) attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[Lds<D>::ROWS];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[Lds<D>::COLS];
  __shared__ __attribute__((aligned(16))) uint16_t Os[Lds<D>::ROWS];  // dO row-major
  __shared__ __attribute__((aligned(16))) uint16_t Ot[Lds<D>::COLS];  // dO channel-major
  __shared__ float lse2_s[kBlock], d_s[kBlock];
  const int g = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int w = t >> 6, l = t & 63, h2 = l >> 5, c32 = l & 31;
  const int key = 32 * w + c32;  // this lane's key (MFMA column) inside the block
  const int64_t k0 = block_token0(g, a.nb, a.n);
  const int klen = block_len(g % a.nb, a.n);
  const float c = a.scale * kLog2e;

  u32x4 kreg[NS], vreg[NS];
  load_row_operand<D>(kreg, a.k + h * a.khs + k0 * a.kts, a.kts, key, klen, h2);
  load_row_operand<D>(vreg, a.v + h * a.vhs + k0 * a.vts, a.vts, key, klen, h2);

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const int32_t* lst = a.inv + (static_cast<int64_t>(h) * a.nq + g) * a.nq;
  const int cnt = a.inv_cnt[static_cast<int64_t>(h) * a.nq + g];
  const uint16_t* qh = a.q + h * a.qhs;
  const uint16_t* dh = a.dout + h * a.dhs;
  Tile<D> tq, td;
  float lse_r = 0.f, d_r = 0.f;
  int r = cnt > 0 ? lst[0] : 0;
  auto fetch = [&](int rb) {
    const int64_t q0 = block_token0(rb, a.nb, a.n);
    const int ql = block_len(rb % a.nb, a.n);
    tq.load(qh + q0 * a.qts, a.qts, ql, t);
    td.load(dh + q0 * a.dts, a.dts, ql, t);
    if (t < kBlock) {
      lse_r = t < ql ? a.lse[h * a.T + q0 + t] * kLog2e : INFINITY;
      d_r = t < ql ? a.Dw[h * a.T + q0 + t] : 0.f;
    }
  };
  if (cnt > 0) fetch(r);
  for (int i = 0; i < cnt; ++i) {
    __syncthreads();
    tq.store_rows(Qs, t);
    tq.store_cols(Qt, t);
    td.store_rows(Os, t);
    td.store_cols(Ot, t);
    if (t < kBlock) {
      lse2_s[t] = lse_r;
      d_s[t] = d_r;
    }
    __syncthreads();
    if (i + 1 < cnt) fetch(lst[i + 1]);
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      sacc[qt] = f32x16{};
      pacc[qt] = f32x16{};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        sacc[qt] = mfma32(rd_rows<D>(Qs, qt, s, c32, h2), kreg[s], sacc[qt]);
        pacc[qt] = mfma32(rd_rows<D>(Os, qt, s, c32, h2), vreg[s], pacc[qt]);
      }
    }
    // rows beyond the query block's length carry lse = +inf, so their P is 0
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int qi = 32 * qt + acc_row(rr, h2);
        const float p = exp2f(fmaf(sacc[qt][rr], c, -lse2_s[qi]));
        sacc[qt][rr] = p;
        pacc[qt][rr] = p * (pacc[qt][rr] - d_s[qi]);
      }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const u32x4 pb = pack_step(sacc, t4);
      const u32x4 sb = pack_step(pacc, t4);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        dv[dt] = mfma32(rd_cols<D>(Ot, dt, t4, c32, h2), pb, dv[dt]);
        dk[dt] = mfma32(rd_cols<D>(Qt, dt, t4, c32, h2), sb, dk[dt]);
      }
    }
  }
  if (key < klen) {
    uint16_t* ko = a.dk + h * a.dkhs + (k0 + key) * a.dkts;
    uint16_t* vo = a.dv + h * a.dvhs + (k0 + key) * a.dvts;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = 32 * dt + 8 * j + 4 * h2;
        u32x2 pk = {pack_bf16x2(dk[dt][4 * j] * a.scale, dk[dt][4 * j + 1] * a.scale),
                    pack_bf16x2(dk[dt][4 * j + 2] * a.scale, dk[dt][4 * j + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(ko + ch) = pk;
        u32x2 pv = {pack_bf16x2(dv[dt][4 * j], dv[dt][4 * j + 1]),
                    pack_bf16x2(dv[dt][4 * j + 2], dv[dt][4 * j + 3])};
        *reinterpret_cast<u32x2*>(vo + ch) = pv;
      }
  }
}

size_t attn_bwd_workspace(const pbsa_dims& d, int chunks, int max_sel) {
  (void)max_sel;
  const int64_t nq = static_cast<int64_t>(chunks) * d.chunk_frames * nb_of(d);
  const int64_t T = static_cast<int64_t>(chunks) * d.chunk_frames * d.frame_tokens;
  const int64_t H = d.heads;
  return static_cast<size_t>(H * T * 4 + H * nq * 4 + H * nq * nq * 4 + 256);
}

hipError_t launch_attn_bwd(const pbsa_dims& d, int chunks, TokIn q, TokIn k, TokIn v, TokIn o,
                           const float* lse, TokIn dout, const int32_t* sel,
                           const int32_t* nsel, int max_sel, TokOut dq, TokOut dk, TokOut dv,
                           void* ws, hipStream_t s) {
  const int nb = nb_of(d);
  const int nq = chunks * d.chunk_frames * nb;
  const int64_t T = static_cast<int64_t>(chunks) * d.chunk_frames * d.frame_tokens;
  BwdArgs a;
  a.q = q.p; a.qts = q.ts; a.qhs = q.hs;
  a.k = k.p; a.kts = k.ts; a.khs = k.hs;
  a.v = v.p; a.vts = v.ts; a.vhs = v.hs;
  a.o = o.p; a.ots = o.ts; a.ohs = o.hs;
  a.dout = dout.p; a.dts = dout.ts; a.dhs = dout.hs;
  a.dq = dq.p; a.dqts = dq.ts; a.dqhs = dq.hs;
  a.dk = dk.p; a.dkts = dk.ts; a.dkhs = dk.hs;
  a.dv = dv.p; a.dvts = dv.ts; a.dvhs = dv.hs;
  a.lse = lse;
  a.sel = sel;
  a.nsel = nsel;
  char* p = static_cast<char*>(ws);
  a.Dw = reinterpret_cast<float*>(p);
  p += static_cast<size_t>(d.heads) * T * 4;
  a.inv_cnt = reinterpret_cast<int32_t*>(p);
  p += static_cast<size_t>(d.heads) * nq * 4;
  a.inv = reinterpret_cast<int32_t*>(p);
  a.T = T;
  a.nq = nq;
  a.nb = nb;
  a.n = d.frame_tokens;
  a.F = d.chunk_frames;
  a.max_sel = max_sel;
  a.scale = d.scale;
  dim3 grid(nq, d.heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, grid, dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_inverse_kernel, grid, dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d.head_dim == 128)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, grid, dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace pbsa
