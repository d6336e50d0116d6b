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
// reference wherever score gaps are larger.  Top-K is a rank count per candidate in LDS:
// rank(j) = #{i : i ahead of j in (score desc, id asc)}; NaN scores order as -inf.
#include "common.h"
#include "launch.h"

namespace pbsa {

namespace {

__device__ __forceinline__ float order_key(float x) {  // NaN -> -inf
  return x != x ? -INFINITY : x;
}
__device__ __forceinline__ bool ahead(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

template <int D>
__device__ __forceinline__ float dot_rep(const float* __restrict__ q_lds,
                                         const float* __restrict__ rep) {
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; c += 4) {
    f32x4 r = *reinterpret_cast<const f32x4*>(rep + c);
    a0 = fmaf(q_lds[c], r[0], a0);
    a1 = fmaf(q_lds[c + 1], r[1], a1);
    a2 = fmaf(q_lds[c + 2], r[2], a2);
    a3 = fmaf(q_lds[c + 3], r[3], a3);
  }
  return (a0 + a1) + (a2 + a3);
}

}  // namespace

// grid (Nq, H), 256 threads.  Dynamic LDS: slots floats + slots ints + slots ints.
template <int D>
__global__ void __launch_bounds__(256)
    score_topk_kernel(const float* __restrict__ q_rep, const float* __restrict__ rep,
                      const int32_t* __restrict__ block_id, int slots, int C, int S, int K,
                      int nq, float scale, float* __restrict__ scores, int32_t* __restrict__ sel) {
  extern __shared__ float smem[];
  __shared__ float q_lds[D];
  __shared__ int n_win;
  float* sc = smem;                                        // [slots]
  int* ids = reinterpret_cast<int*>(sc + slots);           // [slots]
  int* keep = ids + slots;                                 // [slots]
  const int r = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const float* qr = q_rep + (static_cast<int64_t>(h) * nq + r) * D;
  for (int c = t; c < D; c += 256) q_lds[c] = qr[c];
  if (t == 0) n_win = 0;
  __syncthreads();
  const int32_t* bid = block_id + static_cast<int64_t>(h) * slots;
  const float* rp = rep + static_cast<int64_t>(h) * slots * D;
  float* srow = scores + (static_cast<int64_t>(h) * nq + r) * slots;
  int my_win = 0;
  for (int s = t; s < slots; s += 256) {
    const int id = bid[s];
    float v = -INFINITY;
    if (id >= 0) v = scale * dot_rep<D>(q_lds, rp + static_cast<int64_t>(s) * D);
    srow[s] = v;
    sc[s] = order_key(v);
    // window candidates: occupied ring slots holding non-sink blocks
    const bool cand = s >= C && id >= S;
    ids[s] = cand ? id : -1;
    my_win += cand;
  }
  atomicAdd(&n_win, my_win);
  __syncthreads();
  const int nsel = K < n_win ? K : n_win;
  for (int s = C + t; s < slots; s += 256) {
    int k = 0;
    const int id = ids[s];
    if (id >= 0) {
      const float v = sc[s];
      int rank = 0;
      for (int u = C; u < slots; ++u) rank += (ids[u] >= 0) && ahead(sc[u], ids[u], v, id);
      k = rank < nsel;
    }
    keep[s] = k;
  }
  __syncthreads();
  int32_t* out = sel + (static_cast<int64_t>(h) * nq + r) * K;
  for (int s = C + t; s < slots; s += 256) {
    if (keep[s]) {
      const int id = ids[s];
      int pos = 0;
      for (int u = C; u < slots; ++u) pos += keep[u] && ids[u] < id;
      out[pos] = id;
    }
  }
  for (int p = nsel + t; p < K; p += 256) out[p] = -1;
}

hipError_t launch_score_topk(const pbsa_dims& d, const float* q_rep, const pbsa_cache& c,
                             float* scores, int32_t* sel, hipStream_t s) {
  const int nb = nb_of(d);
  const int nq = d.chunk_frames * nb;
  const int slots = static_cast<int>(slots_of(d));
  const size_t lds = static_cast<size_t>(slots) * 12;
  dim3 grid(nq, d.heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(score_topk_kernel<128>, grid, dim3(256), lds, s, q_rep, c.rep, c.block_id,
                       slots, d.capacity, d.sinks, d.topk, nq, d.scale, scores, sel);
  else
    hipLaunchKernelGGL(score_topk_kernel<64>, grid, dim3(256), lds, s, q_rep, c.rep, c.block_id,
                       slots, d.capacity, d.sinks, d.topk, nq, d.scale, scores, sel);
  return hipGetLastError();
}

// ---------------------------------------------------------------- two-level selection

constexpr int kMaxChunks = 256;
struct ChunkBudgets {
  int32_t k[kMaxChunks];
};

// grid (Nq_total, H), 256 threads.  Dynamic LDS sized for the largest candidate set:
// frames floats + frames ints (frame stage), cand floats + cand ints + cand ints.
template <int D>
__global__ void __launch_bounds__(256)
    score_topk_2lvl_kernel(const float* __restrict__ q_rep, const float* __restrict__ block_rep,
                           const float* __restrict__ frame_rep, int F, int nb, int chunks,
                           int top_frames, ChunkBudgets budgets, float scale, int max_sel,
                           int32_t* __restrict__ sel, int32_t* __restrict__ nsel_out) {
  extern __shared__ float smem[];
  __shared__ float q_lds[D];
  __shared__ int n_frames_sel;
  const int r = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int nq = chunks * F * nb;
  const int frames_total = chunks * F;
  const int i = r / (F * nb) + 1;  // 1-based chunk of this query block
  int32_t* out = sel + (static_cast<int64_t>(h) * nq + r) * max_sel;
  if (i == 1) {
    for (int g = t; g < F * nb; g += 256) out[g] = g;
    if (t == 0) nsel_out[static_cast<int64_t>(h) * nq + r] = F * nb;
    return;
  }
  const float* qr = q_rep + (static_cast<int64_t>(h) * nq + r) * D;
  for (int c = t; c < D; c += 256) q_lds[c] = qr[c];
  const int hist = F * (i - 1);
  const int vis = hist + F;  // frames this chunk can see
  float* fsc = smem;                                   // [frames_total]
  int* fsel = reinterpret_cast<int*>(fsc + frames_total);  // [frames_total]
  float* csc = reinterpret_cast<float*>(fsel + frames_total);  // [frames_total*nb]
  int* cid = reinterpret_cast<int*>(csc + frames_total * nb);   // [frames_total*nb]
  int* ckeep = cid + frames_total * nb;                         // [frames_total*nb]
  __syncthreads();
  const float* fr = frame_rep + static_cast<int64_t>(h) * frames_total * D;
  for (int f = t; f < hist; f += 256) fsc[f] = order_key(scale * dot_rep<D>(q_lds, fr + static_cast<int64_t>(f) * D));
  __syncthreads();
  for (int f = t; f < vis; f += 256) {
    int chosen;
    if (f >= hist - 1 || f == 0) {
      chosen = 1;  // forced: sink frame, latest history frame, the chunk's own frames
    } else {
      int rank = 0;
      const float v = fsc[f];
      for (int u = 0; u < hist; ++u) rank += ahead(fsc[u], u, v, f);
      chosen = rank < top_frames;
    }
    fsel[f] = chosen;
  }
  // frame 0 and the latest history frame may also have been chosen by score; a frame is in
  // the set either way.
  __syncthreads();
  if (t == 0) {
    // list the chosen frames in ascending order (at most a few hundred frames)
    int m = 0;
    for (int f = 0; f < vis; ++f)
      if (fsel[f]) fsel[m++] = f;
    n_frames_sel = m;
  }
  __syncthreads();
  const int ncand = n_frames_sel * nb;
  const float* br = block_rep + static_cast<int64_t>(h) * nq * D;
  for (int c = t; c < ncand; c += 256) {
    const int g = fsel[c / nb] * nb + (c % nb);
    cid[c] = g;
    csc[c] = order_key(scale * dot_rep<D>(q_lds, br + static_cast<int64_t>(g) * D));
  }
  __syncthreads();
  int k = budgets.k[i - 1];
  if (k > ncand) k = ncand;
  if (k < 1) k = 1;
  for (int c = t; c < ncand; c += 256) {
    const float v = csc[c];
    const int g = cid[c];
    int rank = 0;
    for (int u = 0; u < ncand; ++u) rank += ahead(csc[u], cid[u], v, g);
    ckeep[c] = rank < k;
  }
  __syncthreads();
  // candidates are listed in ascending id order, so a prefix count gives the position
  for (int c = t; c < ncand; c += 256) {
    if (ckeep[c]) {
      int pos = 0;
      for (int u = 0; u < c; ++u) pos += ckeep[u];
      out[pos] = cid[c];
    }
  }
  if (t == 0) nsel_out[static_cast<int64_t>(h) * nq + r] = k;
}

hipError_t launch_score_topk_2lvl(const pbsa_dims& d, int chunks, int top_frames,
                                  const int32_t* k_per_chunk, const float* q_rep,
                                  const float* block_rep, const float* frame_rep, int max_sel,
                                  int32_t* sel, int32_t* nsel, hipStream_t s) {
  const int nb = nb_of(d);
  const int nq = chunks * d.chunk_frames * nb;
  const int frames_total = chunks * d.chunk_frames;
  ChunkBudgets b;
  for (int i = 0; i < kMaxChunks; ++i) b.k[i] = i < chunks ? k_per_chunk[i] : 0;
  const size_t lds = static_cast<size_t>(frames_total) * 8 + static_cast<size_t>(frames_total) * nb * 12;
  dim3 grid(nq, d.heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(score_topk_2lvl_kernel<128>, grid, dim3(256), lds, s, q_rep, block_rep,
                       frame_rep, d.chunk_frames, nb, chunks, top_frames, b, d.scale, max_sel,
                       sel, nsel);
  else
    hipLaunchKernelGGL(score_topk_2lvl_kernel<64>, grid, dim3(256), lds, s, q_rep, block_rep,
                       frame_rep, d.chunk_frames, nb, chunks, top_frames, b, d.scale, max_sel,
                       sel, nsel);
  return hipGetLastError();
}

}  // namespace pbsa
