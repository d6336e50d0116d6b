// Persistent-memory update (Top-C retention) and window append.
//
// Sparse Forcing (gist.science) 2.B: the persistent memory P_t has a fixed capacity and
// always keeps the sink blocks; 2.C "dynamic update": when the window slides, the blocks
// leaving it are scored from their compressed representatives, the most relevant are
// promoted into P_t and the rest dropped.  Reading: the memory score of a candidate is the
// sum over the chunk's query blocks of its coarse score; candidates are the non-sink
// blocks of P_t and the leaving blocks; the C - S best by (score desc, id asc) are kept.
//
// Two launches:
//   select (one workgroup per head): column sums, rank, new P_t table and copy list, both
//          into the workspace; it only reads the cache, so it may run on another stream
//          while the chunk's attention still reads the cache (pbsa_memory_select);
//   copy   (one workgroup per chunk block and head; pbsa_memory_apply): write the new P_t
//          table, move each promoted block from its window slot into its new persistent
//          slot, then overwrite that window slot with the chunk's block (tokens,
//          zero-padded rows, representative, id, length).
// The window slot a chunk block lands in is exactly the slot of a leaving block (or an
// empty one), and the same workgroup does both moves, so reads precede writes.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "fp8.h"
#include "launch.h"
#include "select.h"

namespace pbsa {

struct MemArgs {
  const float* scores;  // [H][nq][slots]
  uint16_t* ck;         // cache K [H][slots][64][D]
  uint16_t* cv;
  float* rep;           // [H][slots][D]
  int32_t* bid;         // [H][slots]
  int32_t* blen;        // [H][slots]
  int32_t* copy_dst;    // workspace [H][F*nb]: persistent slot of each leaving block kept
  int32_t* pbid;        // workspace [H][C]: the new persistent table (block ids) ...
  int32_t* plen;        // ... and lengths, written by the select, applied by the copy
  int slots, C, S, W, F, nb, n, nq;
  int64_t chunk;        // chunk index being appended (host copy)
  // Optional device chunk counter (NULL: the host copy above is used).  The select reads
  // it and records the value it used in ws_chunk; the copy pass reads ws_chunk and one of
  // its threads advances the counter when done, so a captured update replays correctly
  // for successive chunks.
  int64_t* chunk_dev;
  int64_t* ws_chunk;    // workspace: the chunk index the select used
  float* kv_scale;      // FP8 cache: [H][slots][2] K and V scale of each slot
};

// The chunk index of this update, as the select sees it.
__device__ __forceinline__ int64_t select_chunk(const MemArgs& a) {
  return a.chunk_dev ? *a.chunk_dev : a.chunk;
}
// ... and as the copy pass sees it (what the select recorded).
__device__ __forceinline__ int64_t copy_chunk(const MemArgs& a) {
  return a.chunk_dev ? *a.ws_chunk : a.chunk;
}

// grid H, 1024 threads per head (256 when the candidate count needs more sort registers).  Candidates are listed in a fixed order (persistent
// non-sink slots ascending, then the leaving blocks in chunk-block order, which is
// ascending id); their memory scores are column sums of the chunk's score matrix, computed
// by all 16 waves with coalesced row reads (row group g = t / 256 sums rows g, g+4, ... of
// the full groups of four, group 0 also the remaining rows; the four partials are added as
// (g0 + g1) + (g2 + g3)).  Wave 0 then selects the C - S best (score, ~id) keys with an
// exact radix select (a candidate is kept iff it is among them).  Freed persistent slots
// (ascending) are handed to the promoted leaving blocks in ascending id order.  Dynamic
// LDS: block_id and len of the head ([slots] each), candidate slot [ncand_max], free-slot
// list [C], partial sums [4][ncand_max].
// NT threads: 1024 when the selection runs alone (more rows of the column sums in flight),
// 256 when it runs beside the attention (four waves and a few KB of LDS fit next to two
// attention workgroups on a CU, so it takes no attention workgroup's place); 256 also when
// wave 0's sort keys need the registers.  The sums are the same either way.
template <int E>
constexpr int select_threads(bool beside) { return E <= 8 && !beside ? 1024 : 256; }

template <int E, int NT>
__global__ void __launch_bounds__(NT) memory_select_kernel(MemArgs a) {
  extern __shared__ int mem_smem[];
  __shared__ int s_cnt[2];  // nP, ncand
  const int h = blockIdx.x, t = threadIdx.x, l = t & 63, w = t >> 6;
  const int ncand_max = (a.C - a.S) + a.F * a.nb;
  int* sbid = mem_smem;          // [slots]
  int* slen = sbid + a.slots;    // [slots]
  int* cslot = slen + a.slots;   // [ncand_max]
  int* freel = cslot + ncand_max;  // [C]
  float* part = reinterpret_cast<float*>(freel + a.C);  // [4][ncand_max]
  const int32_t* bid = a.bid + static_cast<int64_t>(h) * a.slots;
  const int32_t* blen = a.blen + static_cast<int64_t>(h) * a.slots;
  int32_t* dst = a.copy_dst + static_cast<int64_t>(h) * a.F * a.nb;
  const int64_t chunk = select_chunk(a);
  if (a.chunk_dev && h == 0 && t == 0) *a.ws_chunk = chunk;
  const int64_t hF = chunk * a.F;  // frames appended so far
  const int fnb = a.F * a.nb;

  for (int b = t; b < fnb; b += NT) dst[b] = -1;
  int32_t* pbid = a.pbid + static_cast<int64_t>(h) * a.C;
  int32_t* plen = a.plen + static_cast<int64_t>(h) * a.C;
  if (chunk == 0) {
    // empty cache: P_t becomes the sinks (block g in slot g; the copy pass moves them)
    for (int s = t; s < a.C; s += NT) {
      pbid[s] = s < a.S ? s : -1;
      plen[s] = s < a.S ? block_len(s % a.nb, a.n) : 0;
    }
    return;
  }
  for (int s = t; s < a.slots; s += NT) {
    sbid[s] = bid[s];
    slen[s] = blen[s];
  }
  __syncthreads();
  if (w == 0) {
    // candidate list (ballot compaction keeps the order)
    int nP = 0;
    for (int s0 = a.S; s0 < a.C; s0 += 64) {
      const int s = s0 + l;
      const bool on = s < a.C && sbid[s] >= a.S;
      const unsigned long long m = __ballot(on);
      if (on) cslot[nP + __popcll(m & ((1ull << l) - 1ull))] = s;
      nP += __popcll(m);
    }
    int ncand = nP;
    for (int b0 = 0; b0 < fnb; b0 += 64) {
      const int b = b0 + l;
      int s = -1;
      if (b < fnb) {
        const int64_t f_new = hF + b / a.nb;  // chunk frame landing in this window slot
        if (f_new >= a.W) {                   // otherwise the slot was empty: nothing leaves
          s = a.C + static_cast<int>(f_new % a.W) * a.nb + b % a.nb;
          if (sbid[s] < a.S) s = -1;
        }
      }
      const unsigned long long m = __ballot(s >= 0);
      if (s >= 0) cslot[ncand + __popcll(m & ((1ull << l) - 1ull))] = s;
      ncand += __popcll(m);
    }
    if (l == 0) {
      s_cnt[0] = nP;
      s_cnt[1] = ncand;
    }
  }
  __syncthreads();
  const int nP = s_cnt[0], ncand = s_cnt[1];
  // partial column sums
  {
    const float* sc = a.scores + static_cast<int64_t>(h) * a.nq * a.slots;
    const int full = a.nq & ~3;
    // the head's first `full` score rows as a buffer: a load past them returns 0
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sc), (short)0, full * a.slots * 4, 0x00020000);
    for (int c = t & 255; c < ncand; c += 256) {
      const int s = cslot[c];
      for (int g = t >> 8; g < 4; g += NT / 256) {
        float acc = 0.f;
        // 24 rows loaded before they are added, rows past `full` as 0 (adding +0 leaves the
        // sum as it is; the order of the additions is kept): up to 96 query blocks take a
        // single round trip
        for (int r = g; r < full; r += 96) {
          float v[24];
#pragma unroll
          for (int u = 0; u < 24; ++u)
            v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rs, 4u * static_cast<uint32_t>((r + 4 * u) * a.slots + s), 0, 0));
#pragma unroll
          for (int u = 0; u < 24; ++u) acc += v[u];
        }
        if (g == 0)
          for (int r = full; r < a.nq; ++r) acc += sc[static_cast<int64_t>(r) * a.slots + s];
        part[g * ncand_max + c] = acc;
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    // memory scores and keys (in candidate order)
    uint64_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int c = l + 64 * e;
      key[e] = 0;
      if (c < ncand) {
        const float msum = (part[c] + part[ncand_max + c]) +
                           (part[2 * ncand_max + c] + part[3 * ncand_max + c]);
        key[e] = rank_key(msum, sbid[cslot[c]]);
      }
    }
    const int keep_n = a.C - a.S < ncand ? a.C - a.S : ncand;
    if (keep_n > 0) {
      bool on[E];
      wave_topk<E>(key, keep_n, on);
      // kept flags per candidate (in candidate order), written over cslot's sign bit
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int c = l + 64 * e;
        if (c < ncand && on[e]) cslot[c] = ~cslot[c];  // kept: negative
      }
    }
    // kept flags per persistent slot, over the partial sums (read above by this wave only;
    // one wave's LDS accesses complete in order)
    int* keptf = reinterpret_cast<int*>(part);
    for (int s = l; s < a.C; s += 64) keptf[s] = 0;
    for (int c = l; c < nP; c += 64)
      if (cslot[c] < 0) keptf[~cslot[c]] = 1;
  }
  __syncthreads();
  if (w == 0) {
    // free list: persistent non-sink slots whose block is not kept (or that are empty)
    int nfree = 0;
    for (int s0 = a.S; s0 < a.C; s0 += 64) {
      const int s = s0 + l;
      bool fr = false;
      if (s < a.C) {
        const int* keptf = reinterpret_cast<const int*>(part);
        fr = sbid[s] < a.S || keptf[s] == 0;  // empty, or its block is not kept
      }
      const unsigned long long m = __ballot(fr);
      if (fr) freel[nfree + __popcll(m & ((1ull << l) - 1ull))] = s;
      nfree += __popcll(m);
    }
    // (the free list is read back by other lanes of this wave only)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // promoted leaving blocks (kept candidates past nP), in candidate order = ascending id
    int npro = 0;
    for (int c0 = nP; c0 < ncand; c0 += 64) {
      const int c = c0 + l;
      const bool pro = c < ncand && cslot[c] < 0;
      const unsigned long long m = __ballot(pro);
      if (pro) {
        const int k = npro + __popcll(m & ((1ull << l) - 1ull));
        const int src = ~cslot[c];
        const int s = freel[k];
        const int b_rel = src - a.C;
        const int rf = b_rel / a.nb, j = b_rel % a.nb;
        const int fb = static_cast<int>(((rf - hF % a.W) % a.W + a.W) % a.W);
        dst[fb * a.nb + j] = s;
        // (persistent slots only: the window slots read above are not written)
        sbid[s] = sbid[src];
        slen[s] = slen[src];
      }
      npro += __popcll(m);
    }
    // freed slots left over become empty
    for (int k = npro + l; k < nfree; k += 64) {
      sbid[freel[k]] = -1;
      slen[freel[k]] = 0;
    }
  }
  __syncthreads();
  // the new persistent table goes to the workspace; the cache itself is not written here,
  // so this selection may run while other kernels still read the cache
  for (int s = t; s < a.C; s += NT) {
    pbid[s] = sbid[s];
    plen[s] = slen[s];
  }
}

// grid (F*nb, H), 256 threads.  chunk_rep may be null: the block means of chunk_k are then
// computed here from the rows being copied (fp32 sums).
template <int D>
__global__ void __launch_bounds__(256) memory_copy_kernel(MemArgs a, TokIn xk, TokIn xv,
                                                          const float* __restrict__ chunk_rep) {
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int64_t chunk = copy_chunk(a);
  const int64_t hF = chunk * a.F;
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
  // (a persistent slot or -1; checked so that a workspace that holds no selection of this
  // cache cannot send the copy outside the persistent slots)
  if (dst >= 0 && dst < a.C) {
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
  const bool sink = chunk == 0 && g < a.S;
  const int target = sink ? g : ring;
  const int64_t tok0 = static_cast<int64_t>(fl) * a.n + static_cast<int64_t>(kBlock) * j;
  // thread t holds channels 8 (t % CH) .. of rows t / CH + (256 / CH) p; their K sums give
  // the block's representative when the caller passes none
  float ksum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ksum[e] = 0.f;
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
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ksum[2 * e] += __uint_as_float(kv[e] << 16);
      ksum[2 * e + 1] += __uint_as_float(kv[e] & 0xffff0000u);
    }
  }
  if (chunk_rep) {
    const float* cr = chunk_rep + (static_cast<int64_t>(h) * a.nq + b) * D;
    for (int c = t; c < D; c += 256) rep[static_cast<int64_t>(target) * D + c] = cr[c];
  } else {
    // lanes l, l ^ CH, ... of a wave share channels; then the four waves through LDS
    __shared__ float wsum[4][D];
    const int l = t & 63, w = t >> 6;
#pragma unroll
    for (int o = CH; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) ksum[e] += __shfl_xor(ksum[e], o, 64);
    if (l < CH)
#pragma unroll
      for (int e = 0; e < 8; ++e) wsum[w][8 * l + e] = ksum[e];
    __syncthreads();
    const float inv = 1.f / static_cast<float>(len);
    for (int c = t; c < D; c += 256)
      rep[static_cast<int64_t>(target) * D + c] =
          ((wsum[0][c] + wsum[1][c]) + (wsum[2][c] + wsum[3][c])) * inv;
  }
  // the persistent table (selected by the select pass, sinks included) by one workgroup
  // per head; every other id written here is a window slot's
  if (b == 0)
    for (int s = t; s < a.C; s += 256) {
      a.bid[hs + s] = a.pbid[static_cast<int64_t>(h) * a.C + s];
      a.blen[hs + s] = a.plen[static_cast<int64_t>(h) * a.C + s];
    }
  if (t == 0) {
    a.bid[hs + ring] = sink ? -1 : g;
    a.blen[hs + ring] = sink ? 0 : len;
    // the device counter moves on (only this workgroup writes it; the others read the
    // index the select recorded)
    if (a.chunk_dev && b == 0 && h == 0) *a.chunk_dev = chunk + 1;
  }
}

// The copy pass for an FP8 cache (same grid and duties as memory_copy_kernel): promoted
// blocks move as codes with their scales; the chunk's blocks are quantized on the way in:
// per block and tensor the power-of-two scale of its largest |value|, then each value's
// nearest E4M3 code (rows past the block length stay code 0).  The representative is the
// mean of the chunk's bf16 keys, as in the bf16 cache.
template <int D>
__global__ void __launch_bounds__(256) memory_copy_fp8_kernel(MemArgs a, TokIn xk, TokIn xv,
                                                              const float* __restrict__ chunk_rep) {
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int l = t & 63, w = t >> 6;
  const int64_t chunk = copy_chunk(a);
  const int64_t hF = chunk * a.F;
  const int fl = b / a.nb, j = b - fl * a.nb;
  const int64_t f = hF + fl;
  const int ring = a.C + static_cast<int>(f % a.W) * a.nb + j;
  const int g = static_cast<int>(f * a.nb + j);
  const int len = block_len(j, a.n);
  const int64_t hs = static_cast<int64_t>(h) * a.slots;
  uint8_t* ck = reinterpret_cast<uint8_t*>(a.ck) + hs * kBlock * D;
  uint8_t* cv = reinterpret_cast<uint8_t*>(a.cv) + hs * kBlock * D;
  float* rep = a.rep + hs * D;
  float* ksc = a.kv_scale + hs * 2;
  constexpr int CH = D / 8;               // 8-value chunks per row
  constexpr int PER = kBlock * CH / 256;  // chunks per thread
  constexpr int CB = kBlock * D / 16;     // 16-byte pieces of a slot's codes
  const int dst = a.copy_dst[static_cast<int64_t>(h) * a.F * a.nb + b];
  if (dst >= 0 && dst < a.C) {
    for (int q = t; q < CB; q += 256) {
      const int64_t so = static_cast<int64_t>(ring) * kBlock * D + 16 * q;
      const int64_t dof = static_cast<int64_t>(dst) * kBlock * D + 16 * q;
      *reinterpret_cast<u32x4*>(ck + dof) = *reinterpret_cast<const u32x4*>(ck + so);
      *reinterpret_cast<u32x4*>(cv + dof) = *reinterpret_cast<const u32x4*>(cv + so);
    }
    for (int c = t; c < D; c += 256)
      rep[static_cast<int64_t>(dst) * D + c] = rep[static_cast<int64_t>(ring) * D + c];
    if (t < 2) ksc[2 * dst + t] = ksc[2 * ring + t];
  }
  __syncthreads();
  const bool sink = chunk == 0 && g < a.S;
  const int target = sink ? g : ring;
  const int64_t tok0 = static_cast<int64_t>(fl) * a.n + static_cast<int64_t>(kBlock) * j;
  u32x4 kv[PER], vv[PER];
  float ksum[8], kmax = 0.f, vmax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ksum[e] = 0.f;
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
      const float k0 = __uint_as_float(kv[p][e] << 16), k1 = __uint_as_float(kv[p][e] & 0xffff0000u);
      const float v0 = __uint_as_float(vv[p][e] << 16), v1 = __uint_as_float(vv[p][e] & 0xffff0000u);
      ksum[2 * e] += k0;
      ksum[2 * e + 1] += k1;
      kmax = fmaxf(kmax, fmaxf(fabsf(k0), fabsf(k1)));
      vmax = fmaxf(vmax, fmaxf(fabsf(v0), fabsf(v1)));
    }
  }
  // block maxima: the wave, then the four waves through LDS
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
    const int64_t o = static_cast<int64_t>(target) * kBlock * D + static_cast<int64_t>(row) * D + 8 * cc;
    *reinterpret_cast<u32x2*>(ck + o) = kc;
    *reinterpret_cast<u32x2*>(cv + o) = vc;
  }
  if (t == 0) {
    ksc[2 * target] = ldexpf(1.f, ek);
    ksc[2 * target + 1] = ldexpf(1.f, ev);
  }
  if (chunk_rep) {
    const float* cr = chunk_rep + (static_cast<int64_t>(h) * a.nq + b) * D;
    for (int c = t; c < D; c += 256) rep[static_cast<int64_t>(target) * D + c] = cr[c];
  } else {
    __shared__ float wsum[4][D];
#pragma unroll
    for (int o = CH; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) ksum[e] += __shfl_xor(ksum[e], o, 64);
    if (l < CH)
#pragma unroll
      for (int e = 0; e < 8; ++e) wsum[w][8 * l + e] = ksum[e];
    __syncthreads();
    const float inv = 1.f / static_cast<float>(len);
    for (int c = t; c < D; c += 256)
      rep[static_cast<int64_t>(target) * D + c] =
          ((wsum[0][c] + wsum[1][c]) + (wsum[2][c] + wsum[3][c])) * inv;
  }
  if (b == 0)
    for (int s = t; s < a.C; s += 256) {
      a.bid[hs + s] = a.pbid[static_cast<int64_t>(h) * a.C + s];
      a.blen[hs + s] = a.plen[static_cast<int64_t>(h) * a.C + s];
    }
  if (t == 0) {
    a.bid[hs + ring] = sink ? -1 : g;
    a.blen[hs + ring] = sink ? 0 : len;
    if (a.chunk_dev && b == 0 && h == 0) *a.chunk_dev = chunk + 1;
  }
}

namespace {

// Workspace: copy list [H][F*nb], then the new persistent table [H][C] (ids, lengths),
// then the chunk index the select used, each piece 256-byte aligned.
size_t ws_up(size_t x) { return (x + 255) & ~size_t{255}; }

MemArgs mem_args(const pbsa_dims& d, const float* scores, const pbsa_cache& c, void* ws) {
  const int nb = nb_of(d);
  MemArgs a;
  a.scores = scores;
  a.ck = static_cast<uint16_t*>(c.k);
  a.cv = static_cast<uint16_t*>(c.v);
  a.rep = c.rep;
  a.bid = c.block_id;
  a.blen = c.len;
  char* p = static_cast<char*>(ws);
  const size_t ncopy = ws_up(sizeof(int32_t) * static_cast<size_t>(d.heads) * d.chunk_frames * nb);
  const size_t ntab = ws_up(sizeof(int32_t) * static_cast<size_t>(d.heads) * d.capacity);
  a.copy_dst = reinterpret_cast<int32_t*>(p);
  a.pbid = reinterpret_cast<int32_t*>(p + ncopy);
  a.plen = reinterpret_cast<int32_t*>(p + ncopy + ntab);
  a.ws_chunk = reinterpret_cast<int64_t*>(p + ncopy + 2 * ntab);
  a.chunk_dev = c.chunk_index_dev;
  a.kv_scale = c.kv_scale;
  a.slots = static_cast<int>(slots_of(d));
  a.C = d.capacity;
  a.S = d.sinks;
  a.W = d.window_frames;
  a.F = d.chunk_frames;
  a.nb = nb;
  a.n = d.frame_tokens;
  a.nq = d.chunk_frames * nb;
  a.chunk = c.chunk_index;
  return a;
}

}  // namespace

size_t memory_update_workspace(const pbsa_dims& d) {
  return ws_up(sizeof(int32_t) * static_cast<size_t>(d.heads) * d.chunk_frames * nb_of(d)) +
         2 * ws_up(sizeof(int32_t) * static_cast<size_t>(d.heads) * d.capacity) +
         ws_up(sizeof(int64_t));
}

hipError_t launch_memory_select(const pbsa_dims& d, const float* scores, const pbsa_cache& c,
                                void* ws, bool beside, hipStream_t s) {
  const MemArgs a = mem_args(d, scores, c, ws);
  const int ncand_max = (d.capacity - d.sinks) + d.chunk_frames * a.nb;
  const size_t lds = static_cast<size_t>(2 * a.slots + 5 * ncand_max + d.capacity) * sizeof(int);
  const int E = (ncand_max + 63) / 64;
  auto go = [&](auto e_tag) {
    constexpr int EE = decltype(e_tag)::value;
    if (beside)
      hipLaunchKernelGGL((memory_select_kernel<EE, select_threads<EE>(true)>), dim3(d.heads),
                         dim3(select_threads<EE>(true)), lds, s, a);
    else
      hipLaunchKernelGGL((memory_select_kernel<EE, select_threads<EE>(false)>), dim3(d.heads),
                         dim3(select_threads<EE>(false)), lds, s, a);
  };
  if (E <= 1) go(std::integral_constant<int, 1>{});
  else if (E <= 2) go(std::integral_constant<int, 2>{});
  else if (E <= 4) go(std::integral_constant<int, 4>{});
  else if (E <= 8) go(std::integral_constant<int, 8>{});
  else if (E <= 16) go(std::integral_constant<int, 16>{});
  else go(std::integral_constant<int, 32>{});
  return hipGetLastError();
}

hipError_t launch_memory_apply(const pbsa_dims& d, const pbsa_cache& c, TokIn ck, TokIn cv,
                               const float* chunk_rep, void* ws, hipStream_t s) {
  const MemArgs a = mem_args(d, nullptr, c, ws);
  dim3 grid(d.chunk_frames * a.nb, d.heads);
  if (d.kv_format == PBSA_KV_FP8) {  // head_dim 128 (checked at the boundary)
    hipLaunchKernelGGL(memory_copy_fp8_kernel<128>, grid, dim3(256), 0, s, a, ck, cv, chunk_rep);
    return hipGetLastError();
  }
  if (d.head_dim == 128)
    hipLaunchKernelGGL(memory_copy_kernel<128>, grid, dim3(256), 0, s, a, ck, cv, chunk_rep);
  else
    hipLaunchKernelGGL(memory_copy_kernel<64>, grid, dim3(256), 0, s, a, ck, cv, chunk_rep);
  return hipGetLastError();
}

hipError_t launch_memory_update(const pbsa_dims& d, const float* scores, const pbsa_cache& c,
                                TokIn ck, TokIn cv, const float* chunk_rep, void* ws,
                                hipStream_t s) {
  const hipError_t e = launch_memory_select(d, scores, c, ws, false, s);
  if (e != hipSuccess) return e;
  return launch_memory_apply(d, c, ck, cv, chunk_rep, ws, s);
}

// Library-held workspace of the allocation-free update: each GPU holds its own copy of
// this array for the life of the process.  Host code never uses the array's name as an
// address: memory_scratch() looks the device address up (once per device, with that
// device current) and every launch gets that address.
__device__ __align__(256) char scratch[kMemoryScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t memory_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pbsa

namespace pbsa {

__global__ void cache_reset_kernel(int32_t* bid, int32_t* blen, int64_t total,
                                   int64_t* chunk_dev) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < total) {
    bid[i] = -1;
    blen[i] = 0;
  }
  if (chunk_dev && i == 0) *chunk_dev = 0;
}

hipError_t launch_cache_reset(const pbsa_dims& d, const pbsa_cache& c, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(d.heads) * slots_of(d);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_reset_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, s, c.block_id, c.len, total, c.chunk_index_dev);
  return hipGetLastError();
}

}  // namespace pbsa
