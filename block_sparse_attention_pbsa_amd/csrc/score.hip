// Coarse block scoring and top-K routing.
//
// Persistent mode -- Sparse Forcing (gist.science) 2.C: the block-level score of a query
// block against a history block is the scaled inner product of their representatives;
// each query block keeps the K best blocks of the local window; persistent blocks are
// scored too (their scores feed the memory update) but always attended.
// Two-level mode -- Light Forcing (papernotes.org), hierarchical sparse attention steps 2
// and 3: frame-level top-K over pooled frame representatives united with forced frames,
// then block-level top-K inside the chosen frames.
//
// Latency-bound (~1e8 FLOP per chunk): scores are fp32 FMA dot products on the vector ALUs,
// which keeps them within ~1e-7 of the exact value, so selections agree with an exact
// reference wherever score gaps are larger.  Candidates are 64-bit (score, ~id) keys, so
// that ties go to the lower id; NaN scores order as -inf.  Every top-K is an exact radix
// select over the keys held by one wave (one ballot per bit).
#include "common.h"
#include "launch.h"
#include "select.h"

namespace pbsa {


// Row-parallel scores of QB query blocks against `cnt` representative rows.  Groups of
// LPR = D/8 lanes read one row with 16-byte loads (whole rows per instruction), multiply
// by the query blocks' matching 8 channels, and reduce across the group; the group's first
// lane writes the QB scores of its row to out[qb * stride + row].  U row groups are loaded
// before any is used, so a pass over the rows waits for memory cnt / (U * step) times.
template <int D, int QB, int U>
__device__ __forceinline__ void score_rows(const float (&qv)[QB][8], const float* __restrict__ rep,
                                           const int32_t* __restrict__ bid, int cnt, float scale,
                                           float* out, int stride, int l, int first, int step) {
  constexpr int LPR = D / 8;
  const int g = l / LPR, sub = l % LPR;
  for (int s0 = first; s0 < cnt; s0 += U * step) {
    f32x4 a[U], b[U];
    int id[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * step + g;
      const int sr = s < cnt ? s : 0;  // rows past the end re-read row 0, unused
      const float* row = rep + static_cast<int64_t>(sr) * D + 8 * sub;
      a[u] = *reinterpret_cast<const f32x4*>(row);
      b[u] = *reinterpret_cast<const f32x4*>(row + 4);
      id[u] = bid[sr];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc[QB];
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        acc[q] = qv[q][0] * a[u][0] + qv[q][1] * a[u][1] + qv[q][2] * a[u][2] +
                 qv[q][3] * a[u][3] + qv[q][4] * b[u][0] + qv[q][5] * b[u][1] +
                 qv[q][6] * b[u][2] + qv[q][7] * b[u][3];
      }
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1)
#pragma unroll
        for (int q = 0; q < QB; ++q) acc[q] += __shfl_xor(acc[q], o, 64);
      const int s = s0 + u * step + g;
      if (s < cnt && sub == 0) {
#pragma unroll
        for (int q = 0; q < QB; ++q) out[q * stride + s] = id[u] >= 0 ? scale * acc[q] : -INFINITY;
      }
    }
  }
}

// grid (ceil(Nq / QB), H), 2 QB waves scoring QB query blocks together: every
// representative row is read once per QB query blocks, whole rows per load instruction, the
// waves taking interleaved row groups (two waves per query block halve each wave's chain of
// loads: 3.8 us less at 406 slots).  Then wave q < QB selects query block q's top K window
// candidates and writes their ids in ascending order (each id's position = the number of
// selected ids below it).  Dynamic LDS: [QB][slots] floats (a wave's row is reused for its
// selected ids).  POOL: wave q < QB first pools query block q from the query tokens xq (the same arithmetic as
// pool_blocks_kernel) and, if q_rep is not null, stores the mean there; otherwise q_rep is
// read.
template <int D, int E, int QB, bool POOL>
__global__ void __launch_bounds__(128 * QB)
    score_topk_kernel(TokIn xq, int n, int nb, float* q_rep, const float* __restrict__ rep,
                      const int32_t* __restrict__ block_id, int slots, int C, int S, int K,
                      int nq, float scale, float* __restrict__ scores,
                      int32_t* __restrict__ sel, int cand0) {
  extern __shared__ float sc_lds[];  // [QB][slots]
  const int r0 = blockIdx.x * QB, h = blockIdx.y, t = threadIdx.x, w = t >> 6, l = t & 63;
  const int nrows = nq - r0 < QB ? nq - r0 : QB;
  constexpr int LPR = D / 8, RPI = 64 / LPR;
  float qv[QB][8];
  if constexpr (POOL) {
    __shared__ float qp[QB][D];
    if (w < nrows) {
      const int r = r0 + w;
      const int f = r / nb, j = r - f * nb;
      const int len = block_len(j, n);
      const int64_t t0 = static_cast<int64_t>(f) * n + static_cast<int64_t>(kBlock) * j;
      const uint16_t* base = xq.p + h * xq.hs + t0 * xq.ts + 8 * (l % LPR);
      u32x4 v[kBlock / RPI];
#pragma unroll
      for (int i = 0; i < kBlock / RPI; ++i) {
        const int row = l / LPR + RPI * i;
        v[i] = row < len ? *reinterpret_cast<const u32x4*>(base + row * xq.ts) : u32x4{0, 0, 0, 0};
      }
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int i = 0; i < kBlock / RPI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(v[i][e] << 16);
          acc[2 * e + 1] += __uint_as_float(v[i][e] & 0xffff0000u);
        }
#pragma unroll
      for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
      const float inv = 1.f / static_cast<float>(len);
      if (l < LPR) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qp[w][8 * l + e] = acc[e] * inv;
        if (q_rep) {
          float* out = q_rep + (static_cast<int64_t>(h) * nq + r) * D + 8 * l;
          reinterpret_cast<f32x4*>(out)[0] = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
          reinterpret_cast<f32x4*>(out)[1] = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[q][e] = qp[q < nrows ? q : 0][8 * (l % LPR) + e];
  } else {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int r = r0 + (q < nrows ? q : 0);
      const float* qr = q_rep + (static_cast<int64_t>(h) * nq + r) * D + 8 * (l % LPR);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[q][e] = qr[e];
    }
  }
  const int32_t* bid = block_id + static_cast<int64_t>(h) * slots;
  const float* rp = rep + static_cast<int64_t>(h) * slots * D;
  score_rows<D, QB, 8>(qv, rp, bid, slots, scale, sc_lds, slots, l, w * RPI, 2 * QB * RPI);
  __syncthreads();
  // scores out (coalesced rows)
  for (int q = 0; q < nrows; ++q) {
    float* srow = scores + (static_cast<int64_t>(h) * nq + r0 + q) * slots;
    for (int s = t; s < slots; s += 128 * QB) srow[s] = sc_lds[q * slots + s];
  }
  // candidates: occupied slots from cand0 on holding non-sink blocks (cand0 = C: the
  // window's ring slots; cand0 = 0: the persistent slots too)
  const int q = w;
  const int nwin = slots - cand0;
  uint64_t key[E];
  int nvalid = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int wi = l + 64 * e;
    key[e] = 0;
    if (q < nrows && wi < nwin) {
      const int id = bid[cand0 + wi];
      if (id >= S) {
        key[e] = rank_key(sc_lds[q * slots + cand0 + wi], id);
        ++nvalid;
      }
    }
  }
  __syncthreads();  // every row has been read: a wave may now reuse its own
  if (q >= nrows) return;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nvalid += __shfl_xor(nvalid, o, 64);
  const int nsel = K < nvalid ? K : nvalid;
  int32_t* out = sel + (static_cast<int64_t>(h) * nq + r0 + q) * K;
  if (nsel > 0) {
    bool on[E];
    wave_topk<E>(key, nsel, on);
    int* ids = reinterpret_cast<int*>(sc_lds + q * slots);  // nsel <= nwin < slots
    int myid[E];
    int base = 0;
    const unsigned long long below = (1ull << l) - 1ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      myid[e] = rank_key_id(key[e]);
      const unsigned long long m = __ballot(on[e]);
      if (on[e]) ids[base + __popcll(m & below)] = myid[e];
      base += __popcll(m);
    }
    // (one wave's LDS accesses complete in order: the reads below see the writes above)
    int rk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) rk[e] = 0;
    for (int j = 0; j < nsel; ++j) {
      const int v = ids[j];
#pragma unroll
      for (int e = 0; e < E; ++e) rk[e] += v < myid[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (on[e]) out[rk[e]] = myid[e];
  }
  for (int p = nsel + l; p < K; p += 64) out[p] = -1;
}

template <int D, bool POOL>
static hipError_t launch_score_d(const pbsa_dims& d, TokIn xq, float* q_rep, const pbsa_cache& c,
                                 float* scores, int32_t* sel, hipStream_t s) {
  constexpr int QB = 4;
  const int nb = nb_of(d);
  const int nq = d.chunk_frames * nb;
  const int slots = static_cast<int>(slots_of(d));
  const int cand0 = d.route_mode == PBSA_ROUTE_UNION ? 0 : d.capacity;
  const int nwin = slots - cand0;
  const size_t lds = static_cast<size_t>(QB) * slots * sizeof(float);
  dim3 grid(cdiv(nq, QB), d.heads);
#define PBSA_SCORE_E(EE)                                                                     \
  hipLaunchKernelGGL((score_topk_kernel<D, EE, QB, POOL>), grid, dim3(128 * QB), lds, s, xq,    \
                     d.frame_tokens, nb, q_rep, c.rep, c.block_id, slots, d.capacity, d.sinks, \
                     d.topk, nq, d.scale, scores, sel, cand0)
  if (nwin <= 64) PBSA_SCORE_E(1);
  else if (nwin <= 128) PBSA_SCORE_E(2);
  else if (nwin <= 256) PBSA_SCORE_E(4);
  else if (nwin <= 512) PBSA_SCORE_E(8);
  else PBSA_SCORE_E(16);  // candidates <= 1024 (checked at the boundary)
#undef PBSA_SCORE_E
  return hipGetLastError();
}

hipError_t launch_score_topk(const pbsa_dims& d, const float* q_rep, const pbsa_cache& c,
                             float* scores, int32_t* sel, hipStream_t s) {
  const TokIn none{nullptr, 0, 0};
  float* qr = const_cast<float*>(q_rep);  // read only when not pooling
  return d.head_dim == 128 ? launch_score_d<128, false>(d, none, qr, c, scores, sel, s)
                           : launch_score_d<64, false>(d, none, qr, c, scores, sel, s);
}

hipError_t launch_route(const pbsa_dims& d, TokIn q, float* q_rep, const pbsa_cache& c,
                        float* scores, int32_t* sel, hipStream_t s) {
  return d.head_dim == 128 ? launch_score_d<128, true>(d, q, q_rep, c, scores, sel, s)
                           : launch_score_d<64, true>(d, q, q_rep, c, scores, sel, s);
}

// ---------------------------------------------------------------- two-level selection

constexpr int kMaxChunks = 256;
constexpr size_t kScoreMfmaLds = 150 * 1024;  // dynamic LDS of the matrix-core selection
struct ChunkBudgets {
  int32_t k[kMaxChunks];
};

// scale * <q_rep row, rep row> for rows [0, cnt) (row_ptr(i): row i's D floats) into
// out[i], by the 256 threads of a workgroup: groups of D/8 lanes take one row each (whole
// rows per load instruction), U row groups loaded before any is used.  qv: this lane's 8
// channels of the query representative.
template <int D, int U, class RowPtr>
__device__ __forceinline__ void rows_dot(const float (&qv)[8], int cnt, RowPtr row_ptr,
                                         float scale, float* out, int t) {
  constexpr int LPR = D / 8, RPI = 64 / LPR, STEP = 4 * RPI;
  const int w = t >> 6, l = t & 63, sub = l % LPR, g = l / LPR;
  for (int r0 = w * RPI; r0 < cnt; r0 += U * STEP) {
    f32x4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = r0 + u * STEP + g;
      const float* p = row_ptr(row < cnt ? row : 0) + 8 * sub;
      a[u] = *reinterpret_cast<const f32x4*>(p);
      b[u] = *reinterpret_cast<const f32x4*>(p + 4);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = qv[0] * a[u][0] + qv[1] * a[u][1] + qv[2] * a[u][2] + qv[3] * a[u][3] +
                  qv[4] * b[u][0] + qv[5] * b[u][1] + qv[6] * b[u][2] + qv[7] * b[u][3];
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
      const int row = r0 + u * STEP + g;
      if (row < cnt && sub == 0) out[row] = scale * acc;
    }
  }
}

// grid (Nq_total, H), 256 threads per query block.  Frame stage: the history frames' scores
// (rows_dot), then wave 0 selects the top_frames by radix select; chosen and forced frames
// are flagged in LDS and listed in ascending order.  Block stage: every block of the listed
// frames is a candidate (ascending ids); their scores (rows_dot), then wave 0 selects the
// top k and writes them in candidate order, which is ascending.  Dynamic LDS: frame scores,
// flags and list ([frames_total] each), candidate scores [64 E].
template <int D, int EF, int E>
__global__ void __launch_bounds__(256)
    score_topk_2lvl_kernel(const float* __restrict__ q_rep, const float* __restrict__ block_rep,
                           const float* __restrict__ frame_rep, int F, int nb, int chunks,
                           int top_frames, ChunkBudgets budgets, float scale, int max_sel,
                           int32_t* __restrict__ sel, int32_t* __restrict__ nsel_out) {
  extern __shared__ float sel_lds[];
  __shared__ int s_nfr;
  const int r = blockIdx.x, h = blockIdx.y, t = threadIdx.x, w = t >> 6, l = t & 63;
  const int nq = chunks * F * nb;
  const int frames_total = chunks * F;
  float* fsc = sel_lds;                                          // [frames_total]
  int* fflag = reinterpret_cast<int*>(fsc + frames_total);       // [frames_total]
  int* flist = fflag + frames_total;                             // [frames_total]
  float* bsc = reinterpret_cast<float*>(flist + frames_total);   // [64 E]
  const int i = r / (F * nb) + 1;  // 1-based chunk of this query block
  int32_t* out = sel + (static_cast<int64_t>(h) * nq + r) * max_sel;
  if (i == 1) {
    for (int g = t; g < F * nb; g += 256) out[g] = g;
    if (t == 0) nsel_out[static_cast<int64_t>(h) * nq + r] = F * nb;
    return;
  }
  constexpr int LPR = D / 8;
  float qv[8];
  {
    const float* qr = q_rep + (static_cast<int64_t>(h) * nq + r) * D + 8 * (l % LPR);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = qr[e];
  }
  const int hist = F * (i - 1);
  const int vis = hist + F;  // frames this chunk can see
  // forced: sink frame, latest history frame, the chunk's own frames
  for (int f = t; f < vis; f += 256) fflag[f] = (f == 0 || f >= hist - 1);
  const float* fr = frame_rep + static_cast<int64_t>(h) * frames_total * D;
  rows_dot<D, 4>(qv, hist, [&](int f) { return fr + static_cast<int64_t>(f) * D; }, scale, fsc, t);
  __syncthreads();
  const int ntop = top_frames < hist ? top_frames : hist;
  if (w == 0 && ntop > 0) {
    uint64_t fk[EF];
#pragma unroll
    for (int e = 0; e < EF; ++e) {
      const int f = l + 64 * e;
      fk[e] = f < hist ? rank_key(fsc[f], f) : 0;
    }
    bool on[EF];
    wave_topk<EF>(fk, ntop, on);
#pragma unroll
    for (int e = 0; e < EF; ++e)
      if (on[e]) fflag[l + 64 * e] = 1;
  }
  __syncthreads();
  if (w == 0) {
    // chosen frames in ascending order (ballot compaction over the visible frames)
    int nfr = 0;
    for (int f0 = 0; f0 < vis; f0 += 64) {
      const int f = f0 + l;
      const bool on = f < vis && fflag[f];
      const unsigned long long m = __ballot(on);
      if (on) flist[nfr + __popcll(m & ((1ull << l) - 1ull))] = f;
      nfr += __popcll(m);
    }
    if (l == 0) s_nfr = nfr;
  }
  __syncthreads();
  const int ncand = s_nfr * nb;
  const float* br = block_rep + static_cast<int64_t>(h) * nq * D;
  auto cand_id = [&](int c) { return flist[c / nb] * nb + (c % nb); };
  rows_dot<D, 8>(qv, ncand, [&](int c) { return br + static_cast<int64_t>(cand_id(c)) * D; },
                 scale, bsc, t);
  __syncthreads();
  if (w == 0) {
    uint64_t key[E];
    int gid[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = l + 64 * e;
      gid[e] = c < ncand ? cand_id(c) : -1;
      key[e] = c < ncand ? rank_key(bsc[c], gid[e]) : 0;
    }
    int k = budgets.k[i - 1];
    if (k > ncand) k = ncand;
    if (k < 1) k = 1;
    bool on[E];
    wave_topk<E>(key, k, on);
    int base = 0;
    const unsigned long long below = (1ull << l) - 1ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const unsigned long long m = __ballot(on[e]);
      if (on[e]) out[base + __popcll(m & below)] = gid[e];
      base += __popcll(m);
    }
    if (l == 0) nsel_out[static_cast<int64_t>(h) * nq + r] = k;
  }
}

// Matrix-core form of the same selection for clips whose scores fit in LDS.  One
// workgroup (512 threads) per group of up to 32 query blocks of one chunk and head: first
// the scores of the group against every history frame and every block the chunk can see,
// as 32 x 32 tiles of fp32 MFMAs (v_mfma_f32_32x32x2_f32: the products and sums stay in
// fp32, like the dot products above, only in another order), each representative row read
// once per group instead of once per query block; then each wave selects for its query
// blocks from the scores in LDS, with the same radix selects and order as
// score_topk_2lvl_kernel.  Dynamic LDS: block scores [32][nvis_pad], frame scores
// [32][hist_pad], and per wave the frame flags and list ([frames_total] each).
template <int D, int EF, int E>
__global__ void __launch_bounds__(512, 1)
    score_2lvl_mfma_kernel(const float* __restrict__ q_rep, const float* __restrict__ block_rep,
                           const float* __restrict__ frame_rep, int F, int nb, int chunks,
                           int top_frames, ChunkBudgets budgets, float scale, int max_sel,
                           int groups_per_chunk, int nvis_pad, int hist_pad,
                           int32_t* __restrict__ sel, int32_t* __restrict__ nsel_out) {
  extern __shared__ float sel_lds[];
  constexpr int KH = D / 2;  // channels per lane half: MFMA k-step s pairs channel s (lanes
                             // 0..31) with channel KH + s (lanes 32..63)
  const int h = blockIdx.y, t = threadIdx.x, w = t >> 6, l = t & 63;
  const int h2 = l >> 5, c32 = l & 31;
  const int nqc = F * nb;                        // query blocks per chunk
  const int nq = chunks * nqc;
  const int frames_total = chunks * F;
  const int ci = blockIdx.x / groups_per_chunk;  // 0-based chunk
  const int i = ci + 1;
  const int r0 = ci * nqc + 32 * (blockIdx.x % groups_per_chunk);
  const int G = nqc - 32 * static_cast<int>(blockIdx.x % groups_per_chunk) < 32
                    ? nqc - 32 * static_cast<int>(blockIdx.x % groups_per_chunk)
                    : 32;
  if (i == 1) {
    for (int j = t; j < G * nqc; j += 512) {
      const int q = j / nqc, g = j - q * nqc;
      sel[(static_cast<int64_t>(h) * nq + r0 + q) * max_sel + g] = g;
    }
    if (t < G) nsel_out[static_cast<int64_t>(h) * nq + r0 + t] = nqc;
    return;
  }
  const int hist = F * (i - 1);
  const int vis = hist + F;           // frames this chunk can see
  const int nvis = vis * nb;          // blocks this chunk can see
  float* bsc = sel_lds;                                      // [32][nvis_pad]
  float* fsc = bsc + 32 * nvis_pad;                          // [32][hist_pad]
  int* fflag = reinterpret_cast<int*>(fsc + 32 * hist_pad) + 2 * frames_total * w;
  int* flist = fflag + frames_total;

  // ---- scores: tiles of 32 rows (frames, then blocks) against the group's 32 query blocks
  {
    float qa[KH];
    const float* qr = q_rep + (static_cast<int64_t>(h) * nq + r0 + c32) * D + KH * h2;
#pragma unroll
    for (int s4 = 0; s4 < KH / 4; ++s4) {
      const f32x4 v = c32 < G ? *reinterpret_cast<const f32x4*>(qr + 4 * s4) : f32x4{0, 0, 0, 0};
      qa[4 * s4] = v[0];
      qa[4 * s4 + 1] = v[1];
      qa[4 * s4 + 2] = v[2];
      qa[4 * s4 + 3] = v[3];
    }
    const int ntf = (hist + 31) / 32, ntb = (nvis + 31) / 32;
    const float* fr = frame_rep + static_cast<int64_t>(h) * frames_total * D;
    const float* br = block_rep + static_cast<int64_t>(h) * nq * D;
    for (int tt = w; tt < ntf + ntb; tt += 8) {
      const bool is_f = tt < ntf;
      const int row0 = 32 * (is_f ? tt : tt - ntf);
      const int nrow = is_f ? hist : nvis;
      const int row = row0 + c32;
      const float* rp = (is_f ? fr : br) + static_cast<int64_t>(row < nrow ? row : 0) * D + KH * h2;
      float kb[KH];
#pragma unroll
      for (int s4 = 0; s4 < KH / 4; ++s4) {
        const f32x4 v = row < nrow ? *reinterpret_cast<const f32x4*>(rp + 4 * s4)
                                   : f32x4{0, 0, 0, 0};
        kb[4 * s4] = v[0];
        kb[4 * s4 + 1] = v[1];
        kb[4 * s4 + 2] = v[2];
        kb[4 * s4 + 3] = v[3];
      }
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < KH; ++s)
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s], kb[s], acc, 0, 0, 0);
      // lane: column (row of the tile) c32, query blocks acc_row(e, h2)
      float* dst = is_f ? fsc : bsc;
      const int pitch = is_f ? hist_pad : nvis_pad;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int qb = 8 * (e >> 2) + 4 * h2 + (e & 3);
        dst[qb * pitch + row0 + c32] = scale * acc[e];
      }
    }
  }
  __syncthreads();

  // ---- selection: wave w takes query blocks w, w + 8, ... of the group
  for (int q = w; q < G; q += 8) {
    const int r = r0 + q;
    int32_t* out = sel + (static_cast<int64_t>(h) * nq + r) * max_sel;
    const float* fq = fsc + q * hist_pad;
    const float* bq = bsc + q * nvis_pad;
    // forced: sink frame, latest history frame, the chunk's own frames
    for (int f = l; f < vis; f += 64) fflag[f] = (f == 0 || f >= hist - 1);
    const int ntop = top_frames < hist ? top_frames : hist;
    if (ntop > 0) {
      uint64_t fk[EF];
#pragma unroll
      for (int e = 0; e < EF; ++e) {
        const int f = l + 64 * e;
        fk[e] = f < hist ? rank_key(fq[f], f) : 0;
      }
      bool on[EF];
      wave_topk<EF>(fk, ntop, on);
#pragma unroll
      for (int e = 0; e < EF; ++e)
        if (on[e]) fflag[l + 64 * e] = 1;
    }
    // chosen frames in ascending order (ballot compaction over the visible frames)
    int nfr = 0;
    for (int f0 = 0; f0 < vis; f0 += 64) {
      const int f = f0 + l;
      const bool on = f < vis && fflag[f];
      const unsigned long long m = __ballot(on);
      if (on) flist[nfr + __popcll(m & ((1ull << l) - 1ull))] = f;
      nfr += __popcll(m);
    }
    const int ncand = nfr * nb;
    auto cand_id = [&](int cc) { return flist[cc / nb] * nb + (cc % nb); };
    uint64_t key[E];
    int gid[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int cc = l + 64 * e;
      gid[e] = cc < ncand ? cand_id(cc) : -1;
      key[e] = cc < ncand ? rank_key(bq[gid[e]], gid[e]) : 0;
    }
    int k = budgets.k[i - 1];
    if (k > ncand) k = ncand;
    if (k < 1) k = 1;
    bool on[E];
    wave_topk<E>(key, k, on);
    int base = 0;
    const unsigned long long below = (1ull << l) - 1ull;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const unsigned long long m = __ballot(on[e]);
      if (on[e]) out[base + __popcll(m & below)] = gid[e];
      base += __popcll(m);
    }
    if (l == 0) nsel_out[static_cast<int64_t>(h) * nq + r] = k;
  }
}

template <int D, int EF>
static hipError_t launch_2lvl_mfma_e(int E, dim3 grid, size_t lds, hipStream_t s,
                                     const float* q_rep, const float* block_rep,
                                     const float* frame_rep, int F, int nb, int chunks,
                                     int top_frames, const ChunkBudgets& b, float scale,
                                     int max_sel, int gpc, int nvis_pad, int hist_pad,
                                     int32_t* sel, int32_t* nsel) {
#define PBSA_2LVL_M(EE)                                                                       \
  hipLaunchKernelGGL((score_2lvl_mfma_kernel<D, EF, EE>), grid, dim3(512), lds, s, q_rep,      \
                     block_rep, frame_rep, F, nb, chunks, top_frames, b, scale, max_sel, gpc, \
                     nvis_pad, hist_pad, sel, nsel)
  if (E <= 1) PBSA_2LVL_M(1);
  else if (E <= 2) PBSA_2LVL_M(2);
  else if (E <= 4) PBSA_2LVL_M(4);
  else if (E <= 8) PBSA_2LVL_M(8);
  else PBSA_2LVL_M(16);
#undef PBSA_2LVL_M
  return hipGetLastError();
}

template <int D, int EF>
static hipError_t launch_2lvl_e(int E, dim3 grid, size_t lds, hipStream_t s, const float* q_rep,
                                const float* block_rep, const float* frame_rep, int F, int nb,
                                int chunks, int top_frames, const ChunkBudgets& b, float scale,
                                int max_sel, int32_t* sel, int32_t* nsel) {
#define PBSA_2LVL_E(EE)                                                                      \
  hipLaunchKernelGGL((score_topk_2lvl_kernel<D, EF, EE>), grid, dim3(256), lds, s, q_rep,      \
                     block_rep, frame_rep, F, nb, chunks, top_frames, b, scale, max_sel, sel, \
                     nsel)
  if (E <= 1) PBSA_2LVL_E(1);
  else if (E <= 2) PBSA_2LVL_E(2);
  else if (E <= 4) PBSA_2LVL_E(4);
  else if (E <= 8) PBSA_2LVL_E(8);
  else PBSA_2LVL_E(16);
#undef PBSA_2LVL_E
  return hipGetLastError();
}

template <int D>
static hipError_t launch_2lvl_d(const pbsa_dims& d, int chunks, int top_frames,
                                const ChunkBudgets& b, const float* q_rep,
                                const float* block_rep, const float* frame_rep, int max_sel,
                                int32_t* sel, int32_t* nsel, hipStream_t s) {
  const int nb = nb_of(d);
  const int F = d.chunk_frames;
  const int nq = chunks * F * nb;
  const int frames_total = chunks * F;
  // candidates: at most (top_frames + 2 + F) frames of nb blocks, and never more than
  // the frames a chunk can see
  const int fr_max = top_frames + 2 + F < frames_total ? top_frames + 2 + F : frames_total;
  const int ncand = fr_max * nb;
  const int E = (ncand + 63) / 64;
  const int EF = (frames_total + 63) / 64;
  // the matrix-core form when the group's scores fit in LDS
  const int nvis_pad = 32 * ((frames_total * nb + 31) / 32);
  const int hist_pad = 32 * ((frames_total - F + 31) / 32 > 0 ? (frames_total - F + 31) / 32 : 1);
  const size_t lds_m = (static_cast<size_t>(32) * (nvis_pad + hist_pad) +
                        static_cast<size_t>(8) * 2 * frames_total) * sizeof(float);
  if (lds_m <= kScoreMfmaLds) {
    const int gpc = (F * nb + 31) / 32;
    dim3 grid_m(chunks * gpc, d.heads);
    if (EF <= 1)
      return launch_2lvl_mfma_e<D, 1>(E, grid_m, lds_m, s, q_rep, block_rep, frame_rep, F, nb,
                                      chunks, top_frames, b, d.scale, max_sel, gpc, nvis_pad,
                                      hist_pad, sel, nsel);
    if (EF <= 2)
      return launch_2lvl_mfma_e<D, 2>(E, grid_m, lds_m, s, q_rep, block_rep, frame_rep, F, nb,
                                      chunks, top_frames, b, d.scale, max_sel, gpc, nvis_pad,
                                      hist_pad, sel, nsel);
    return launch_2lvl_mfma_e<D, 4>(E, grid_m, lds_m, s, q_rep, block_rep, frame_rep, F, nb,
                                    chunks, top_frames, b, d.scale, max_sel, gpc, nvis_pad,
                                    hist_pad, sel, nsel);
  }
  const size_t lds = static_cast<size_t>(3 * frames_total + 64 * E) * sizeof(int);
  dim3 grid(nq, d.heads);
  if (EF <= 1)
    return launch_2lvl_e<D, 1>(E, grid, lds, s, q_rep, block_rep, frame_rep, F, nb, chunks,
                               top_frames, b, d.scale, max_sel, sel, nsel);
  if (EF <= 2)
    return launch_2lvl_e<D, 2>(E, grid, lds, s, q_rep, block_rep, frame_rep, F, nb, chunks,
                               top_frames, b, d.scale, max_sel, sel, nsel);
  return launch_2lvl_e<D, 4>(E, grid, lds, s, q_rep, block_rep, frame_rep, F, nb, chunks,
                             top_frames, b, d.scale, max_sel, sel, nsel);
}

hipError_t launch_score_topk_2lvl(const pbsa_dims& d, int chunks, int top_frames,
                                  const int32_t* k_per_chunk, const float* q_rep,
                                  const float* block_rep, const float* frame_rep, int max_sel,
                                  int32_t* sel, int32_t* nsel, hipStream_t s) {
  ChunkBudgets b;
  for (int i = 0; i < kMaxChunks; ++i) b.k[i] = i < chunks ? k_per_chunk[i] : 0;
  return d.head_dim == 128
             ? launch_2lvl_d<128>(d, chunks, top_frames, b, q_rep, block_rep, frame_rep, max_sel,
                                  sel, nsel, s)
             : launch_2lvl_d<64>(d, chunks, top_frames, b, q_rep, block_rep, frame_rep, max_sel,
                                 sel, nsel, s);
}

}  // namespace pbsa
