// Block lists of the attention forward: one workgroup takes two 64-token query blocks A, B
// of one head and walks the KV blocks both attend ("shared") and then each one's own
// ("private").
#pragma once

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
  // persistent mode, top-K over the persistent and window blocks together: only the sink
  // slots [0, S) are attended whole, routed ids may name persistent blocks
  int route_union, S;
  // FP8 cache: ck / cv hold E4M3 codes [H][slots][64][D] (one byte each), kv_scale the
  // power-of-two scale of every slot's K and V ([H][slots][2])
  const float* kv_scale;
};

// Lists of one workgroup.  Entries (32 bits): bit 31 = a block of the chunk (token layout),
// else a cache slot; bits 24..30 = valid rows; bits 0..23 = the cache slot, or for a chunk
// block its first token (or, with CHUNK_IDS, its index in the chunk).
// Shared list (persistent mode): occupied P slots in slot order, then the chunk's blocks,
// then the routed blocks that A and B have in common (kept at the end of A's list area,
// last to first).  Private lists: the routed blocks of A only and of B only.
struct FwdLists {
  int cntA, cntB;  // entries of A's and B's private lists
  int nboth;       // routed blocks A and B share
  int nPq;         // persistent mode: P and chunk entries at the head of the shared list
  int nshared;     // shared entries (nPq + nboth)
  int offA, offB;  // first entries of A's and B's private lists in `lists`
};

// Builds the lists in LDS (`lists`: kAttnListCap entries, and one more word that is set to
// 0) for the query blocks rA and rB = rA + 1 of head h; rawA, rawB (sel_stride ints each)
// and pids (C ints) are LDS staging areas that no gather targets yet.  Every thread of the
// workgroup calls it.
template <bool PERSIST, bool CHUNK_IDS>
__device__ __forceinline__ FwdLists build_lists(const FwdArgs& a, int h, int rA, int rB,
                                                uint32_t* lists, int* wave_cnt,
                                                int (*part_cnt)[3], int& n_list, int32_t* rawA,
                                                int32_t* rawB, int32_t* pids) {
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  int cntA, cntB, nboth = 0;
  auto tok_entry = [&](int g) {
    const int f = g / a.nb, jj = g - f * a.nb;
    return 0x80000000u | (static_cast<uint32_t>(block_len(jj, a.n)) << 24) |
           static_cast<uint32_t>(CHUNK_IDS ? g : f * a.n + kBlock * jj);
  };
  auto slot_entry = [&](int slot, int len) {
    return (static_cast<uint32_t>(len) << 24) | static_cast<uint32_t>(slot);
  };
  uint32_t* shared_list = lists;
  uint32_t* listA = lists + (PERSIST ? a.C + a.nq : 0);
  uint32_t* listB = listA + a.sel_stride;
  int nshared = 0;
  // (union routing) the head's persistent block ids, staged in pids for the lookups of
  // routed persistent blocks below
  if (PERSIST) {
    if (t == 0) n_list = 0;
    const int32_t* bh = a.bid + static_cast<int64_t>(h) * a.slots;
    const int32_t* lh = a.blen + static_cast<int64_t>(h) * a.slots;
    if (a.route_union)
      for (int s = t; s < a.C; s += 256) pids[s] = bh[s];
    __syncthreads();
    // slots attended whole: every persistent slot, or only the sinks' (union routing)
    const int whole = a.route_union ? a.S : a.C;
    for (int s0 = 0; s0 < whole; s0 += 256) {
      const int s = s0 + t;
      const bool valid = s < whole && bh[s] >= 0;
      const unsigned long long m = __ballot(valid);
      if (l == 0) wave_cnt[w] = __popcll(m);
      __syncthreads();
      int off = n_list;
      for (int u = 0; u < w; ++u) off += wave_cnt[u];
      if (valid) shared_list[off + __popcll(m & ((1ull << l) - 1ull))] = slot_entry(s, lh[s]);
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
  auto entry = [&](int g) {
    // (two-level mode) an id outside the clip is an empty entry
    if (!PERSIST) return g >= 0 && g < a.nq ? tok_entry(g) : 0x80000000u;
    const int f = g / a.nb, jj = g - f * a.nb;
    int slot = a.C + (f % a.W) * a.nb + jj;
    if (a.route_union && a.bid[static_cast<int64_t>(h) * a.slots + slot] != g) {
      // not in the window: a persistent block (an id the cache does not hold becomes an
      // empty entry, which contributes nothing)
      int found = -1;
      for (int ps = a.S; ps < a.C; ++ps)
        if (pids[ps] == g) {
          found = ps;
          break;
        }
      if (found < 0) return slot_entry(0, 0);
      slot = found;
    }
    return slot_entry(slot, a.blen[static_cast<int64_t>(h) * a.slots + slot]);
  };
  const int32_t* sa = a.sel + (static_cast<int64_t>(h) * a.nq + rA) * a.sel_stride;
  const int32_t* sb = a.sel + (static_cast<int64_t>(h) * a.nq + rB) * a.sel_stride;
  {
    // Split A's and B's routed sets into A only, B only and both.  The ascending ids are
    // staged in rawA, rawB and looked up by binary search; each part is compacted in id order with ballots, so the lists (and the
    // summation order) do not depend on timing.
    const int na = PERSIST ? a.sel_stride : a.nsel[static_cast<int64_t>(h) * a.nq + rA];
    const int nbb = rB >= a.nq ? 0 : PERSIST ? a.sel_stride
                                             : a.nsel[static_cast<int64_t>(h) * a.nq + rB];
    for (int j = t; j < a.sel_stride; j += 256) {
      rawA[j] = j < na ? sa[j] : -1;
      rawB[j] = j < nbb ? sb[j] : -1;
    }
    __syncthreads();
    int ca = 0, cb = 0;
    for (int j = l; j < a.sel_stride; j += 64) {
      ca += rawA[j] >= 0;
      cb += rawB[j] >= 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      ca += __shfl_xor(ca, o, 64);
      cb += __shfl_xor(cb, o, 64);
    }
    const int nA = __builtin_amdgcn_readfirstlane(ca);
    const int nB = __builtin_amdgcn_readfirstlane(cb);
    auto contains = [](const int32_t* ids, int n_ids, int g) {
      int lo = 0, hi = n_ids;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ids[mid] < g) lo = mid + 1;
        else hi = mid;
      }
      return lo < n_ids && ids[lo] == g;
    };
    int oa = 0, ob = 0, oi = 0;
    const unsigned long long below = (1ull << l) - 1ull;
    for (int j0 = 0; j0 < a.sel_stride; j0 += 256) {
      const int j = j0 + t;
      const int ga = j < nA ? rawA[j] : -1;
      const int gb = j < nB ? rawB[j] : -1;
      const bool both = ga >= 0 && contains(rawB, nB, ga);
      const bool a_only = ga >= 0 && !both;
      const bool b_only = gb >= 0 && !contains(rawA, nA, gb);
      const unsigned long long ma = __ballot(a_only), mb = __ballot(b_only), mi = __ballot(both);
      if (l == 0) {
        part_cnt[w][0] = __popcll(ma);
        part_cnt[w][1] = __popcll(mb);
        part_cnt[w][2] = __popcll(mi);
      }
      __syncthreads();
      int pa = oa, pb = ob, pi = oi;
      for (int u = 0; u < 4; ++u) {
        if (u < w) {
          pa += part_cnt[u][0];
          pb += part_cnt[u][1];
          pi += part_cnt[u][2];
        }
        oa += part_cnt[u][0];
        ob += part_cnt[u][1];
        oi += part_cnt[u][2];
      }
      if (a_only) listA[pa + __popcll(ma & below)] = entry(ga);
      if (b_only) listB[pb + __popcll(mb & below)] = entry(gb);
      if (both) listA[a.sel_stride - 1 - (pi + __popcll(mi & below))] = entry(ga);
      __syncthreads();
    }
    cntA = __builtin_amdgcn_readfirstlane(oa);
    cntB = __builtin_amdgcn_readfirstlane(ob);
    nboth = __builtin_amdgcn_readfirstlane(oi);
  }
  // (the word past the lists holds 0: reads for steps without an entry point at it)
  if (t == 0) lists[kAttnListCap] = 0u;
  __syncthreads();
  FwdLists r;
  r.cntA = cntA;
  r.cntB = cntB;
  r.nboth = nboth;
  r.nPq = nshared;
  r.nshared = nshared + nboth;
  r.offA = static_cast<int>(listA - lists);
  r.offB = r.offA + a.sel_stride;
  return r;
}

}  // namespace pbsa
