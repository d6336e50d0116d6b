// Persistent-memory update (Top-C retention) and window append.
//
// Sparse Forcing (gist.science) 2.B: the persistent memory P_t has a fixed capacity and
// always keeps the sink blocks; 2.C "dynamic update": when the window slides, the blocks
// leaving it are scored from their compressed representatives, the most relevant are
// promoted into P_t and the rest dropped.  Reading: the memory score of a candidate is the
// sum over the chunk's query blocks of its coarse score; candidates are the non-sink
// blocks of P_t and the leaving blocks; the C - S best by (score desc, id asc) are kept.
//
// Two launches on the caller's stream:
//   select (one workgroup per head): column sums, rank, new P_t table, copy list;
//   copy   (one workgroup per chunk block and head): move each promoted block from its
//          window slot into its new persistent slot, then overwrite that window slot with
//          the chunk's block (tokens, zero-padded rows, representative, id, length).
// The window slot a chunk block lands in is exactly the slot of a leaving block (or an
// empty one), and the same workgroup does both moves, so reads precede writes.
#include "common.h"
#include "launch.h"

namespace pbsa {

struct MemArgs {
  const float* scores;  // [H][nq][slots]
  uint16_t* ck;         // cache K [H][slots][64][D]
  uint16_t* cv;
  float* rep;           // [H][slots][D]
  int32_t* bid;         // [H][slots]
  int32_t* blen;        // [H][slots]
  int32_t* copy_dst;    // workspace [H][F*nb]
  int slots, C, S, W, F, nb, n, nq;
  int64_t chunk;        // chunk index being appended
};

namespace {
__device__ __forceinline__ bool ahead(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}
__device__ __forceinline__ float order_key(float x) { return x != x ? -INFINITY : x; }
}  // namespace

// grid H, 256 threads.  Dynamic LDS: the head's block_id and len tables (2 * slots ints)
// followed by 4 arrays of ncand_max = (C - S) + F*nb candidate entries.  Serial steps
// (ordered enumeration, slot assignment) run on one thread over LDS only.
__global__ void __launch_bounds__(256) memory_select_kernel(MemArgs a) {
  extern __shared__ int mem_smem[];
  const int h = blockIdx.x, t = threadIdx.x;
  const int ncand_max = (a.C - a.S) + a.F * a.nb;
  int* sbid = mem_smem;                        // [slots]
  int* slen = sbid + a.slots;                  // [slots]
  int* cslot = slen + a.slots;                 // candidate's slot
  int* cid = cslot + ncand_max;                // candidate's block id
  float* cm = reinterpret_cast<float*>(cid + ncand_max);  // memory score
  int* ckeep = reinterpret_cast<int*>(cm + ncand_max);    // kept?
  __shared__ int nP, nE;
  __shared__ int free_slots[1024];
  int32_t* bid = a.bid + static_cast<int64_t>(h) * a.slots;
  int32_t* blen = a.blen + static_cast<int64_t>(h) * a.slots;
  int32_t* dst = a.copy_dst + static_cast<int64_t>(h) * a.F * a.nb;
  const int64_t hF = a.chunk * a.F;  // frames appended so far

  for (int b = t; b < a.F * a.nb; b += 256) dst[b] = -1;
  if (a.chunk == 0) {
    // empty cache: P_t becomes the sinks, written by the copy pass
    for (int s = t; s < a.C; s += 256) {
      bid[s] = -1;
      blen[s] = 0;
    }
    return;
  }
  for (int s = t; s < a.slots; s += 256) {
    sbid[s] = bid[s];
    slen[s] = blen[s];
  }
  __syncthreads();
  if (t == 0) {
    // enumerate candidates in a fixed order: persistent non-sink slots, then leaving blocks
    int m = 0;
    for (int s = a.S; s < a.C; ++s)
      if (sbid[s] >= a.S) {
        cslot[m] = s;
        cid[m] = sbid[s];
        ++m;
      }
    nP = m;
    for (int b = 0; b < a.F * a.nb; ++b) {
      const int64_t f_new = hF + b / a.nb;  // chunk frame landing in this window slot
      if (f_new < a.W) continue;           // slot was empty: nothing leaves
      const int s = a.C + static_cast<int>(f_new % a.W) * a.nb + b % a.nb;
      if (sbid[s] >= a.S) {
        cslot[m] = s;
        cid[m] = sbid[s];
        ++m;
      }
    }
    nE = m - nP;
  }
  __syncthreads();
  const int ncand = nP + nE;
  const float* sc = a.scores + static_cast<int64_t>(h) * a.nq * a.slots;
  for (int c = t; c < ncand; c += 256) {
    const int s = cslot[c];
    float acc = 0.f;
    for (int r = 0; r < a.nq; ++r) acc += sc[static_cast<int64_t>(r) * a.slots + s];
    cm[c] = order_key(acc);
  }
  __syncthreads();
  const int keep_n = a.C - a.S;
  for (int c = t; c < ncand; c += 256) {
    int rank = 0;
    const float v = cm[c];
    const int id = cid[c];
    for (int u = 0; u < ncand; ++u) rank += ahead(cm[u], cid[u], v, id);
    ckeep[c] = rank < keep_n;
  }
  __syncthreads();
  if (t == 0) {
    // free persistent slots (ascending): empty, or holding a block that is not kept
    int nf = 0;
    int c = 0;
    for (int s = a.S; s < a.C; ++s) {
      bool occupied_kept = false;
      if (c < nP && cslot[c] == s) {
        occupied_kept = ckeep[c];
        ++c;
      }
      if (!occupied_kept) free_slots[nf++] = s;
    }
    // promoted leaving blocks in ascending id order take free slots in ascending order
    int np = 0;
    for (;;) {
      int best = -1;
      for (int e = nP; e < ncand; ++e)
        if (ckeep[e] == 1 && (best < 0 || cid[e] < cid[best])) best = e;
      if (best < 0) break;
      ckeep[best] = 2;  // assigned
      const int s = free_slots[np++];
      const int b_rel = cslot[best] - a.C;
      // chunk block whose window slot is cslot[best]
      const int rf = b_rel / a.nb, j = b_rel % a.nb;
      const int fb = static_cast<int>(((rf - hF % a.W) % a.W + a.W) % a.W);
      dst[fb * a.nb + j] = s;
      sbid[s] = cid[best];
      slen[s] = slen[cslot[best]];
    }
    for (int k = np; k < nf; ++k) {
      sbid[free_slots[k]] = -1;
      slen[free_slots[k]] = 0;
    }
  }
  __syncthreads();
  for (int s = a.S + t; s < a.C; s += 256) {
    bid[s] = sbid[s];
    blen[s] = slen[s];
  }
}

// grid (F*nb, H), 256 threads.
template <int D>
__global__ void __launch_bounds__(256) memory_copy_kernel(MemArgs a, TokIn xk, TokIn xv,
                                                          const float* __restrict__ chunk_rep) {
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int64_t hF = a.chunk * a.F;
  const int fl = b / a.nb, j = b - fl * a.nb;  // chunk-local frame, block
  const int64_t f = hF + fl;
  const int ring = a.C + static_cast<int>(f % a.W) * a.nb + j;
  const int64_t g64 = f * a.nb + j;
  const int g = static_cast<int>(g64);
  const int len = block_len(j, a.n);
  const int64_t hs = static_cast<int64_t>(h) * a.slots;
  uint16_t* ck = a.ck + hs * kBlock * D;
  uint16_t* cv = a.cv + hs * kBlock * D;
  float* rep = a.rep + hs * D;
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int PER = kBlock * CH / 256;    // chunks per thread
  const int dst = a.copy_dst[static_cast<int64_t>(h) * a.F * a.nb + b];
  if (dst >= 0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int q = t + 256 * p;
      const int64_t so = static_cast<int64_t>(ring) * kBlock * D + 8 * q;
      const int64_t dof = static_cast<int64_t>(dst) * kBlock * D + 8 * q;
      *reinterpret_cast<u32x4*>(ck + dof) = *reinterpret_cast<const u32x4*>(ck + so);
      *reinterpret_cast<u32x4*>(cv + dof) = *reinterpret_cast<const u32x4*>(cv + so);
    }
    for (int c = t; c < D; c += 256)
      rep[static_cast<int64_t>(dst) * D + c] = rep[static_cast<int64_t>(ring) * D + c];
  }
  __syncthreads();
  // chunk 0's sink blocks go straight to their persistent slots; the window slot stays empty
  const bool sink = a.chunk == 0 && g < a.S;
  const int target = sink ? g : ring;
  const int64_t tok0 = static_cast<int64_t>(fl) * a.n + static_cast<int64_t>(kBlock) * j;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int q = t + 256 * p;
    const int row = q / CH, cc = q % CH;
    u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (row < len) {
      kv = *reinterpret_cast<const u32x4*>(xk.p + h * xk.hs + (tok0 + row) * xk.ts + 8 * cc);
      vv = *reinterpret_cast<const u32x4*>(xv.p + h * xv.hs + (tok0 + row) * xv.ts + 8 * cc);
    }
    const int64_t o = static_cast<int64_t>(target) * kBlock * D + 8 * q;
    *reinterpret_cast<u32x4*>(ck + o) = kv;
    *reinterpret_cast<u32x4*>(cv + o) = vv;
  }
  const float* cr = chunk_rep + (static_cast<int64_t>(h) * a.nq + b) * D;
  for (int c = t; c < D; c += 256) rep[static_cast<int64_t>(target) * D + c] = cr[c];
  if (t == 0) {
    a.bid[hs + target] = g;
    a.blen[hs + target] = len;
    if (sink) {
      a.bid[hs + ring] = -1;
      a.blen[hs + ring] = 0;
    }
  }
}

size_t memory_update_workspace(const pbsa_dims& d) {
  return sizeof(int32_t) * static_cast<size_t>(d.heads) * d.chunk_frames * nb_of(d);
}

hipError_t launch_memory_update(const pbsa_dims& d, const float* scores, const pbsa_cache& c,
                                TokIn ck, TokIn cv, const float* chunk_rep, void* ws,
                                hipStream_t s) {
  const int nb = nb_of(d);
  MemArgs a;
  a.scores = scores;
  a.ck = static_cast<uint16_t*>(c.k);
  a.cv = static_cast<uint16_t*>(c.v);
  a.rep = c.rep;
  a.bid = c.block_id;
  a.blen = c.len;
  a.copy_dst = static_cast<int32_t*>(ws);
  a.slots = static_cast<int>(slots_of(d));
  a.C = d.capacity;
  a.S = d.sinks;
  a.W = d.window_frames;
  a.F = d.chunk_frames;
  a.nb = nb;
  a.n = d.frame_tokens;
  a.nq = d.chunk_frames * nb;
  a.chunk = c.chunk_index;
  const int ncand_max = (d.capacity - d.sinks) + d.chunk_frames * nb;
  const size_t lds = static_cast<size_t>(ncand_max) * 16 + static_cast<size_t>(a.slots) * 8;
  hipLaunchKernelGGL(memory_select_kernel, dim3(d.heads), dim3(256), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(d.chunk_frames * nb, d.heads);
  if (d.head_dim == 128)
    hipLaunchKernelGGL(memory_copy_kernel<128>, grid, dim3(256), 0, s, a, ck, cv, chunk_rep);
  else
    hipLaunchKernelGGL(memory_copy_kernel<64>, grid, dim3(256), 0, s, a, ck, cv, chunk_rep);
  return hipGetLastError();
}

}  // namespace pbsa

namespace pbsa {

__global__ void cache_reset_kernel(int32_t* bid, int32_t* blen, int64_t total) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < total) {
    bid[i] = -1;
    blen[i] = 0;
  }
}

hipError_t launch_cache_reset(const pbsa_dims& d, const pbsa_cache& c, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(d.heads) * slots_of(d);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_reset_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, s, c.block_id, c.len, total);
  return hipGetLastError();
}

}  // namespace pbsa
