// Backward of attention over selected blocks (trainable path), deterministic.
//
// Sparse Forcing (gist.science) 2.D / 3: the same sparse attention is used while training,
// so the kernel family must also give gradients.  With the selection held constant, the
// gradient of softmax attention is the textbook one: with P = exp(scale*S - LSE),
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// gfx950 design (atomics only build integer lists and hand out work; every floating-point
// sum runs in a fixed order, so results are bit-reproducible):
//   dq pass   -- one workgroup per pair of query blocks of a head (four waves of 32 rows);
//                like the forward it walks each query block's selected KV blocks in 32-key
//                half tiles, recomputes S^T = K Q^T and dP^T = V dO^T on MFMA (Q, dO in
//                registers) and accumulates dQ^T = K^T dS^T, reading K channel-major with
//                the transposing LDS read.  It also writes D for its rows.
//   inverse   -- the query blocks that selected each KV block, in ascending order: every
//                query block sets its bit in a bitmap row per selected KV block and the rows'
//                bits are counted; after the plan pass one workgroup per (KV block, head)
//                writes its row's list at its offset (the lists are stored back to back).
//   plan      -- one workgroup: cuts every inverse list into work items of at most
//                kSplitQ query blocks (a few KV blocks are selected by every query block,
//                most by a few dozen), numbering items, partial-sum slots and list offsets
//                by prefix sums.
//   dkdv pass -- work items taken largest first from a counter (the plan pass orders them
//                by size; each item writes only its own outputs, so results do not depend on
//                which workgroup takes it), two waves of 32 keys each; each lane keeps
//                its key's K and V rows in registers (the MFMA B operands) for the whole
//                item, which walks its part of the list in 32-query half tiles:
//                S = Q K^T and dP = dO V^T with keys as MFMA columns, then dV^T += dO^T P
//                and dK^T += Q^T dS (dO, Q read channel-major with the transposing read).
//                A block with one item writes dK, dV; otherwise each item writes an fp32
//                partial and
//   reduce    -- sums a split block's partials in item order and writes dK, dV.
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
  int32_t* inv_cnt;     // workspace [H][nkv]: query blocks that selected each KV block
  int32_t* inv_off;     // workspace [H][nkv]: start of each KV block's list in inv
  int32_t* inv;         // workspace: the inverse lists back to back (at most H*nq*max_sel)
  uint32_t* bits;       // workspace [H][nkv][ceil(nq / 32)]: bit r = query block r selected
  int2* items;          // workspace: work item -> (h*nq + g, split)
  int2* sorted;         // workspace: the same items by decreasing number of query blocks
  int32_t* nsplit;      // workspace [H*nq]
  int32_t* part_base;   // workspace [H*nq]: first partial slot of a split block
  int32_t* long_list;   // workspace: split blocks
  int32_t* counts;      // workspace: [0] items, [1] split blocks
  float* part;          // workspace: partial slots of 2 * 64 * D floats (dK^T, dV^T)
  int64_t T;
  int nq, nb, n, F, max_sel, H, pairs;
  float scale;
  // KV blocks per head: the clip's blocks (two-level mode, nkv = nq), or, in persistent
  // mode, the cache's slots 0..slots-1 followed by the chunk's nq blocks (k, v above are
  // then the chunk's tokens)
  int nkv;
  int persist;
  const uint16_t *ck, *cv;     // persistent: cache K/V [H][slots][64][D]
  const int32_t *cbid, *clen;  // persistent: cache block ids and lengths [H][slots]
  int slots, C, W, K;
  int S, route_union;          // persistent: sinks; top-K over P_t and the window together
  const int32_t* rsel;         // persistent: routed ids [H][nq][K]
  uint16_t *dkc, *dvc;         // persistent: gradients of the cache slots [H][slots][64][D]
};

// A half tile (32 rows) of a KV block, rows [32*half, +32): its first row, the row stride
// of K and V in bytes, and the valid rows.
struct Half {
  const uint16_t* p;
  int len;      // valid rows (0 = none)
  uint32_t sb;  // row stride (bytes)
};

// KV block list entries (32 bits): bit 31 set = a cache slot (bits 0..23 the slot), else
// a token block (bits 0..23 its first token); bits 24..30 the valid rows.
__device__ __forceinline__ uint32_t kv_entry(const BwdArgs& a, int h, int g) {
  if (g < 0 || g >= a.nkv) return 0u;  // not a block of this head: an empty entry
  if (a.persist && g < a.slots)
    return 0x80000000u | (static_cast<uint32_t>(a.clen[static_cast<int64_t>(h) * a.slots + g]) << 24) |
           static_cast<uint32_t>(g);
  const int b = a.persist ? g - a.slots : g;
  return static_cast<uint32_t>(block_token0(b, a.nb, a.n)) |
         (static_cast<uint32_t>(block_len(b % a.nb, a.n)) << 24);
}
__device__ __forceinline__ int entry_len(uint32_t e) { return static_cast<int>((e >> 24) & 0x7f); }


// 16 bytes per lane from a buffer straight into LDS (lane l writes lds + 1024 i + 16 l):
// piece i (0..3) of a run that shares one LDS base; the instruction's immediate offset
// 1024 i is added to both the global and the LDS address, so voff must already be lowered
// by it.
__device__ __forceinline__ void dma_piece(int i, __amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                          char* lds) {
  switch (i) {
    case 0: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 0, 0); break;
    case 1: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 1024, 0); break;
    case 2: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 2048, 0); break;
    default: __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voff, 0, 3072, 0); break;
  }
}

// Element t of an fp32 row of n valid values from p (p wave-uniform); 0 past n.
__device__ __forceinline__ float load_row_f32(const float* p, int n, int t) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p), 0, static_cast<uint32_t>(n) * 4u, 0x00020000);
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * t, 0, 0));
}

// A wave-uniform 64-bit value kept in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

}  // namespace

// ------------------------------------------------------------------ dQ pass (+ D)
// 1-D grid, 8 * ceil(H * pairs / 8) workgroups of 256 threads (XCD-aware numbering as in the
// forward).  Wave w: query block 2*pair + w/2, rows 32*(w%2) + [0, 32).
template <int D>
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int HT = 32 * Lds<D>::RS;
  // K and V half tiles of X and Y; head_dim 128 has a second set, gathered a step ahead
  // (two arrays rather than one indexed at run time, so that the compiler sees that the
  // reads of one set never touch the gathers in flight into the other)
  __shared__ __attribute__((aligned(1024))) uint16_t tiles0[4 * HT];
  __shared__ __attribute__((aligned(1024))) uint16_t tiles1[D == 128 ? 4 * HT : 8];
  uint16_t* KsX = tiles0;
  uint16_t* VsX = tiles0 + HT;
  uint16_t* KsY = tiles0 + 2 * HT;
  uint16_t* VsY = tiles0 + 3 * HT;
  // A's and B's selected blocks as (first token | valid rows << 24), staged once
  constexpr int kHalfCap = kAttnListCap / 2;
  __shared__ uint32_t lst[kAttnListCap];
  uint32_t* lstA = lst;
  uint32_t* lstB = lst + kHalfCap;

  const int per = gridDim.x / 8;
  const int L = static_cast<int>(blockIdx.x % 8) * per + static_cast<int>(blockIdx.x / 8);
  if (L >= a.H * a.pairs) return;
  const int h = L / a.pairs, pr = L - h * a.pairs;
  const int t = threadIdx.x, l = t & 63, h2 = l >> 5, c32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int mine = w >> 1;
  const int rA = 2 * pr, rB = 2 * pr + 1;
  const int r = mine ? rB : rA;
  const int qlen = r < a.nq ? block_len(r % a.nb, a.n) : 0;
  const int qrow = 32 * (w & 1) + c32;
  const int64_t t0 = r < a.nq ? block_token0(r, a.nb, a.n) : 0;
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
  const float lse2 = qrow < qlen ? a.lse[h * a.T + t0 + qrow] * kLog2e : 0.f;
  if (qrow < qlen && h2 == 0) a.Dw[h * a.T + t0 + qrow] = dsum;

  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};

  const int32_t* selA = a.sel + (static_cast<int64_t>(h) * a.nq + rA) * a.max_sel;
  const int32_t* selB = a.sel + (static_cast<int64_t>(h) * a.nq + rB) * a.max_sel;
  // (counts clamped to the list capacity: other nsel values are not a selection)
  const int cntA = min(max(a.nsel[static_cast<int64_t>(h) * a.nq + rA], 0), a.max_sel);
  const int cntB = rB < a.nq ? min(max(a.nsel[static_cast<int64_t>(h) * a.nq + rB], 0), a.max_sel)
                             : 0;
  const int nsteps = 2 * (cntA > cntB ? cntA : cntB);
  const uint16_t* kh = a.k + h * a.khs;
  const uint16_t* vh = a.v + h * a.vhs;
  // (persistent mode) this head's cache slots
  const uint16_t* ckh = a.persist ? a.ck + static_cast<int64_t>(h) * a.slots * kBlock * D : nullptr;
  const uint16_t* cvh = a.persist ? a.cv + static_cast<int64_t>(h) * a.slots * kBlock * D : nullptr;
  for (int j = t; j < (cntA > cntB ? cntA : cntB); j += 256) {
    if (j < cntA) lstA[j] = kv_entry(a, h, selA[j]);
    if (j < cntB) lstB[j] = kv_entry(a, h, selB[j]);
  }
  __syncthreads();

  const uint32_t kstride_b = static_cast<uint32_t>(2 * a.kts);
  const uint32_t vstride_b = static_cast<uint32_t>(2 * a.vts);
  // step s: half (s & 1) of A's and B's (s >> 1)-th selected block
  auto half_ref = [&](uint32_t e_, int half, Half& k_, Half& v_) {
    const uint32_t e = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(e_)));
    const int len = entry_len(e) - 32 * half;
    const int hl = len < 0 ? 0 : (len < 32 ? len : 32);
    if (e >> 31) {
      const int64_t row0 = static_cast<int64_t>(e & 0xffffffu) * kBlock + 32 * half;
      k_ = Half{ckh + row0 * D, hl, 2u * D};
      v_ = Half{cvh + row0 * D, hl, 2u * D};
    } else {
      const int64_t tk = (e & 0xffffffu) + 32 * half;
      k_ = Half{kh + tk * a.kts, hl, kstride_b};
      v_ = Half{vh + tk * a.vts, hl, vstride_b};
    }
  };
  auto refs = [&](int s, Half& kx, Half& vx, Half& ky, Half& vy) {
    const int j = s >> 1, half = s & 1;
    kx.len = vx.len = ky.len = vy.len = 0;
    if (j < cntA) half_ref(lstA[j], half, kx, vx);
    if (j < cntB) half_ref(lstB[j], half, ky, vy);
  };

  // This lane's transposing-read offsets, opaque to the optimizer: it would otherwise split
  // each read's address into a chain of steps too long for the compiler to still see which
  // LDS array the read is from, and make the read wait for every gather in flight.
  int trlo[ND], trhi[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    tr_offsets<D>(dt, l, trlo[dt], trhi[dt]);
    asm("" : "+v"(trlo[dt]), "+v"(trhi[dt]));
  }
  // this wave's rows against one K/V half tile of len keys: K at set + kb, V at set + kb + HT
  // (offsets from the LDS array itself, so that the compiler can tell these reads from the
  // gathers in flight into the other set)
  auto half_step = [&](const uint16_t* set, int kb, int len) {
    const int vb = kb + HT;
    u32x4 op[NS];
    f32x16 sacc[1], pacc = {};
    sacc[0] = f32x16{};
#pragma unroll
    for (int st = 0; st < NS; ++st) op[st] = rd_rows<D>(set + kb, 0, st, c32, h2);
#pragma unroll
    for (int st = 0; st < NS; ++st) sacc[0] = mfma32(op[st], qreg[st], sacc[0]);
#pragma unroll
    for (int st = 0; st < NS; ++st) op[st] = rd_rows<D>(set + vb, 0, st, c32, h2);
#pragma unroll
    for (int st = 0; st < NS; ++st) pacc = mfma32(op[st], dreg[st], pacc);
    // dS^T = P^T * (dP^T - D); keys past the block length contribute nothing
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const float p = acc_row(rr, h2) < len
                          ? __builtin_amdgcn_exp2f(fmaf(sacc[0][rr], c, -lse2))
                          : 0.f;
      sacc[0][rr] = p * (pacc[rr] - dsum);
    }
    // dQ^T += K^T dS^T (K channel-major through the transposing read)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      u32x4 kop[ND];
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        kop[dt] = rd_tr(set, kb + trlo[dt] + 16 * t2 * Lds<D>::RS,
                        kb + trhi[dt] + 16 * t2 * Lds<D>::RS);
      const u32x4 sb = pack_step(sacc, t2);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt] = mfma32(kop[dt], sb, acc[dt]);
    }
  };

  if constexpr (D == 128) {
    // Gathers straight into LDS (buffer loads with an LDS destination), one step ahead into
    // the other set: wave w fills tile w of the step (K of X, V of X, K of Y, V of Y) as
    // eight 1 KB pieces of four rows.  Lane l of piece i writes LDS bytes 1024 i + 16 l of
    // the tile, i.e. row 4 i + l / 16 at chunk position l % 16, which holds logical chunk
    // (l % 16) ^ swz(row) of the swizzled row-major layout.  Rows past the valid length
    // re-read the last valid row (finite data that a zero probability removes); an empty
    // half tile is not gathered, and no wave reads it.
    // This wave's list entries (its own query block's): the entry of a block is read from
    // LDS a step before it is used (one list array indexed by mine, not a pointer chosen at
    // run time: the compiler then still sees that the read cannot touch a gather in flight).
    const int cnt = mine ? cntB : cntA;
    auto entry_raw = [&](int j) { return lst[mine * kHalfCap + (j < cnt ? j : 0)]; };
    auto half_len = [&](uint32_t e, int j, int half) {
      const int tl = entry_len(e) - 32 * half;
      return j >= cnt ? 0 : (tl < 0 ? 0 : (tl < 32 ? tl : 32));
    };
    auto gather = [&](uint32_t e, int len, int half, uint16_t* set) {
      if (len == 0) return;
      uint32_t sb;
      const char* p;
      if (e >> 31) {  // a cache slot (persistent mode)
        const int64_t row0 = static_cast<int64_t>(e & 0xffffffu) * kBlock + 32 * half;
        sb = 2u * D;
        p = reinterpret_cast<const char*>(((w & 1) ? cvh : ckh) + row0 * D);
      } else {
        const int64_t tk = (e & 0xffffffu) + 32 * half;
        sb = (w & 1) ? vstride_b : kstride_b;
        p = (w & 1) ? reinterpret_cast<const char*>(vh + tk * a.vts)
                    : reinterpret_cast<const char*>(kh + tk * a.kts);
      }
      // scalar base 3 KB below the half tile: lane offsets lowered by a piece's immediate
      // offset (up to 3 KB) stay non-negative
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(p - 3072), 0, 0x7fffffff, 0x00020000);
      char* dst = reinterpret_cast<char*>(set + w * HT);
      const uint32_t q = static_cast<uint32_t>(l >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t row = 4 * i + q;
        const uint32_t rc = row < static_cast<uint32_t>(len) ? row : len - 1;
        const uint32_t cch = static_cast<uint32_t>(l & 15) ^ (4 * q + (i & 3));
        const uint32_t voff = 3072 + rc * sb + 16 * cch - 1024 * (i & 3);
        dma_piece(i & 3, rs, voff, dst + 4096 * (i >> 2));
      }
    };
    // Step st's tiles are in one set (tiles0 for even st, tiles1 for odd; lenC valid rows of
    // this wave's half tile) while the next step's are gathered into the other.  Every wave
    // waits for its own gathers (vmcnt(0)) before the barrier, so that after it every tile
    // of step st has landed; the barrier's own release covers LDS instructions only, and the
    // compiler, left to itself, may let the last gathers of a step still be in flight at
    // the barrier.  After the barrier every wave is also done with the set step st - 1 read.
    uint32_t eC = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(entry_raw(0))));
    uint32_t eN = entry_raw(1);
    int lenC = half_len(eC, 0, 0);
    gather(eC, lenC, 0, tiles0);
    // nsteps is even (two halves per block): step st = 2 j is half 0 of block j, st + 1 half 1
    for (int st = 0; st < nsteps; st += 2) {
      const int j = st >> 1;
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt not waited
      __syncthreads();
      int lenN = half_len(eC, j, 1);
      gather(eC, lenN, 1, tiles1);
      if (qlen > 0 && lenC > 0) half_step(tiles0, 2 * mine * HT, lenC);
      lenC = lenN;
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
      eC = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(eN)));
      eN = entry_raw(j + 2);
      lenN = half_len(eC, j + 1, 0);
      gather(eC, lenN, 0, tiles0);
      if (qlen > 0 && lenC > 0) half_step(tiles1, 2 * mine * HT, lenC);
      lenC = lenN;
    }
  } else {
    Tile<D, 256, 32> tkx, tvx, tky, tvy;
    Half kx, vx, ky, vy;
    if (nsteps > 0) {
      refs(0, kx, vx, ky, vy);
      tkx.load(kx.p, kx.sb, kx.len, t);
      tvx.load(vx.p, vx.sb, vx.len, t);
      tky.load(ky.p, ky.sb, ky.len, t);
      tvy.load(vy.p, vy.sb, vy.len, t);
    }
    for (int st = 0; st < nsteps; ++st) {
      __syncthreads();
      tkx.store_rows(KsX, t);
      tvx.store_rows(VsX, t);
      tky.store_rows(KsY, t);
      tvy.store_rows(VsY, t);
      const int lenX = kx.len, lenY = ky.len;
      __syncthreads();
      if (st + 1 < nsteps) {
        refs(st + 1, kx, vx, ky, vy);
        tkx.load(kx.p, kx.sb, kx.len, t);
        tvx.load(vx.p, vx.sb, vx.len, t);
        tky.load(ky.p, ky.sb, ky.len, t);
        tvy.load(vy.p, vy.sb, vy.len, t);
      }
      const int len = mine ? lenY : lenX;
      if (qlen > 0 && len > 0) half_step(tiles0, 2 * mine * HT, len);
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
// inv holds, for every (head, KV block), the ascending query blocks whose list holds the KV
// block, back to back (offsets inv_off from the plan pass), so it grows with the number of
// selections, not with nq * nkv.  They go through bitmaps: bit r of row (h, g) is set when
// query block r of head h selected KV block g.
__global__ void __launch_bounds__(256) attn_bwd_bits_clear_kernel(BwdArgs a) {
  const int W = (a.nq + 31) >> 5;
  const int64_t n = static_cast<int64_t>(a.H) * a.nkv * W;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    a.bits[i] = 0u;
}

// one workgroup per (query block, head): sets the query block's bit in the row of every
// KV block it selected (two-level mode: a query block of chunk i sees frames < F*i only;
// other entries, like ids outside the clip, are not listed)
__global__ void __launch_bounds__(128) attn_bwd_bits_set_kernel(BwdArgs a) {
  const int r = blockIdx.x, h = blockIdx.y;
  const int W = (a.nq + 31) >> 5;
  const int64_t hr = static_cast<int64_t>(h) * a.nq + r;
  const int cnt = a.nsel[hr];
  const int32_t* s = a.sel + hr * a.max_sel;
  for (int j = threadIdx.x; j < cnt; j += 128) {
    const int g = s[j];
    if (g < 0 || g >= a.nkv) continue;
    if (!a.persist) {
      const int f = g / a.nb;
      if (r < (f / a.F) * a.F * a.nb) continue;
    }
    uint32_t* row = a.bits + (static_cast<int64_t>(h) * a.nkv + g) * W;
    atomicOr(row + (r >> 5), 1u << (r & 31));
  }
}

// one thread per (head, KV block): the number of query blocks that selected it
__global__ void __launch_bounds__(256) attn_bwd_bits_count_kernel(BwdArgs a) {
  const int W = (a.nq + 31) >> 5;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (row >= static_cast<int64_t>(a.H) * a.nkv) return;
  const uint32_t* b = a.bits + row * W;
  int n = 0;
  for (int j = 0; j < W; ++j) n += __popc(b[j]);
  a.inv_cnt[row] = n;
}

// one workgroup per (KV block, head), after the plan pass: the row's set bits in ascending
// order become its inverse list at inv + inv_off
constexpr int kMaxBitWords = 2048;  // nq <= 65536
__global__ void __launch_bounds__(256) attn_bwd_bits_list_kernel(BwdArgs a) {
  __shared__ uint32_t bits[kMaxBitWords];
  __shared__ int wsum[4];
  const int g = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int w = t >> 6, l = t & 63;
  const int W = (a.nq + 31) >> 5;
  const int64_t row = static_cast<int64_t>(h) * a.nkv + g;
  int32_t* out = a.inv + a.inv_off[row];
  for (int j = t; j < W; j += 256) bits[j] = a.bits[row * W + j];
  __syncthreads();
  int total = 0;
  for (int base = 0; base < W; base += 256) {
    const int j = base + t;
    uint32_t m = j < W ? bits[j] : 0u;
    const int pc = __popc(m);
    int x = pc;  // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (l >= o) x += y;
    }
    if (l == 63) wsum[w] = x;
    __syncthreads();
    int off = total + x - pc;
    for (int u = 0; u < w; ++u) off += wsum[u];
    while (m) {
      out[off++] = 32 * j + (__ffs(m) - 1);
      m &= m - 1;
    }
    total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
}

// ------------------------------------------------------------------ plan
constexpr int kSplitQ = 96;  // query blocks per dK/dV work item, at most

// one workgroup of 1024 threads; thread t plans entries [t*per, (t+1)*per) of the H*nq
// (head, KV block) pairs, in order, then three block-wide exclusive scans number the work
// items, the partial slots and the split blocks.
__global__ void __launch_bounds__(1024) attn_bwd_plan_kernel(BwdArgs a) {
  __shared__ int sc[4][1024];
  const int t = threadIdx.x;
  const int N = a.H * a.nkv;
  const int per = (N + 1023) / 1024;
  const int e0 = t * per, e1 = min(N, e0 + per);
  int my_items = 0, my_parts = 0, my_long = 0, my_cnt = 0;
  for (int e = e0; e < e1; ++e) {
    const int cnt = a.inv_cnt[e];
    my_cnt += cnt;
    const int ns = cnt <= kSplitQ ? 1 : (cnt + kSplitQ - 1) / kSplitQ;
    my_items += ns;
    if (ns > 1) {
      my_parts += ns;
      ++my_long;
    }
  }
  sc[0][t] = my_items;
  sc[1][t] = my_parts;
  sc[2][t] = my_long;
  sc[3][t] = my_cnt;
  __syncthreads();
  // Hillis-Steele inclusive scans
  for (int o = 1; o < 1024; o <<= 1) {
    int v0 = 0, v1 = 0, v2 = 0, v3 = 0;
    if (t >= o) {
      v0 = sc[0][t - o];
      v1 = sc[1][t - o];
      v2 = sc[2][t - o];
      v3 = sc[3][t - o];
    }
    __syncthreads();
    sc[0][t] += v0;
    sc[1][t] += v1;
    sc[2][t] += v2;
    sc[3][t] += v3;
    __syncthreads();
  }
  int it = sc[0][t] - my_items, pt = sc[1][t] - my_parts, lg = sc[2][t] - my_long;
  int io = sc[3][t] - my_cnt;
  for (int e = e0; e < e1; ++e) {
    const int cnt = a.inv_cnt[e];
    a.inv_off[e] = io;
    io += cnt;
    const int ns = cnt <= kSplitQ ? 1 : (cnt + kSplitQ - 1) / kSplitQ;
    a.nsplit[e] = ns;
    a.part_base[e] = ns > 1 ? pt : -1;
    for (int s = 0; s < ns; ++s) a.items[it + s] = int2{e, s};
    it += ns;
    if (ns > 1) {
      a.long_list[lg++] = e;
      pt += ns;
    }
  }
  if (t == 1023) {
    a.counts[0] = sc[0][1023];
    a.counts[1] = sc[2][1023];
  }
  // The same items by decreasing size (query blocks, at most kSplitQ) for the dK/dV pass,
  // which takes them largest first from a counter (cleared here): a counting sort.  Items of
  // equal size may land in any order; each item writes only its own outputs, so the
  // results do not depend on it.
  __shared__ int hist[kSplitQ + 1], fill[kSplitQ + 1];
  for (int b = t; b <= kSplitQ; b += 1024) {
    hist[b] = 0;
    fill[b] = 0;
  }
  if (t == 0) a.counts[2] = 0;
  __syncthreads();
  auto size_of = [&](int cnt, int sp) {
    const int q = cnt - sp * kSplitQ;
    return q < kSplitQ ? q : kSplitQ;
  };
  for (int e = e0; e < e1; ++e) {
    const int cnt = a.inv_cnt[e];
    for (int sp = 0; sp < a.nsplit[e]; ++sp) atomicAdd(&hist[kSplitQ - size_of(cnt, sp)], 1);
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int b = 0; b <= kSplitQ; ++b) {
      const int c = hist[b];
      hist[b] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int e = e0; e < e1; ++e) {
    const int cnt = a.inv_cnt[e];
    for (int sp = 0; sp < a.nsplit[e]; ++sp) {
      const int b = kSplitQ - size_of(cnt, sp);
      a.sorted[hist[b] + atomicAdd(&fill[b], 1)] = int2{e, sp};
    }
  }
}

// ------------------------------------------------------------------ dK/dV pass
// Work items from a counter, largest first; 256 threads, two workgroups (two waves per
// SIMD) per CU, so that one wave's softmax, LDS reads and staging run under the other's
// MFMAs.  Wave w owns keys 32*(w & 1) + [0, 32) of the item's KV block (MFMA columns) and
// rows 32*(w >> 1) + [0, 32) of each step's query block; at the end of the item the two
// waves that share keys add their dK^T/dV^T sums through LDS (wave w + 2 into wave w, a
// fixed order).
template <int D>
__global__ void __launch_bounds__(256, 2) attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int TB = Lds<D>::ROWS;                   // elements of one 64-row tile
  constexpr int kSlot = 8 * ND * 64;                 // f32x4 per wave of dK^T | dV^T sums
  constexpr int kSmem = 8 * TB > 2 * kSlot * 16 ? 8 * TB : 2 * kSlot * 16;
  // K, V of the item's block and Q, dO of the step's query block (row-major tiles); at
  // the end of an item the same bytes hold the sums of waves 2 and 3
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  uint16_t* Kb = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vb = Kb + TB;
  uint16_t* Qs = Vb + TB;
  uint16_t* Os = Qs + TB;
  __shared__ __attribute__((aligned(16))) float lse2_s[kBlock];
  __shared__ __attribute__((aligned(16))) float d_s[kBlock];
  // this item's query blocks: first token and valid rows, staged once per item so that a
  // step's loads do not wait on a global read of the list
  __shared__ int64_t qtok_s[kSplitQ];
  __shared__ int qlen_s[kSplitQ];
  const int t = threadIdx.x;
  const int l = t & 63, h2 = l >> 5, c32 = l & 31;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int kt = w & 1, qh = w >> 1;
  const int key = 32 * kt + c32;  // this lane's key (MFMA column) inside the block
  const float c = a.scale * kLog2e;
  const int n_items = a.counts[0];

  __shared__ int s_item;
  for (;;) {
    // the next item, largest first (the counter is cleared by the plan pass)
    if (t == 0) s_item = atomicAdd(&a.counts[2], 1);
    __syncthreads();
    const int item = s_item;
    if (item >= n_items) break;
    const int2 it = a.sorted[item];
    const int hg = __builtin_amdgcn_readfirstlane(it.x), sp = __builtin_amdgcn_readfirstlane(it.y);
    const int h = hg / a.nkv, g = hg - h * a.nkv;
    // the item's KV block: a cache slot (persistent mode, g < slots) or a token block
    const bool is_slot = a.persist && g < a.slots;
    const int b = a.persist && !is_slot ? g - a.slots : g;
    const int64_t k0 = is_slot ? 0 : block_token0(b, a.nb, a.n);
    const int klen = is_slot ? a.clen[static_cast<int64_t>(h) * a.slots + g] : block_len(b % a.nb, a.n);
    __syncthreads();  // s_item is read and the previous item's sums are consumed
    {
      Tile<D, 256> tk, tv;
      if (is_slot) {
        const int64_t so = (static_cast<int64_t>(h) * a.slots + g) * kBlock * D;
        tk.load(a.ck + so, 2u * D, klen, t);
        tv.load(a.cv + so, 2u * D, klen, t);
      } else {
        tk.load(a.k + h * a.khs + k0 * a.kts, static_cast<uint32_t>(2 * a.kts), klen, t);
        tv.load(a.v + h * a.vhs + k0 * a.vts, static_cast<uint32_t>(2 * a.vts), klen, t);
      }
      tk.store_rows(Kb, t);
      tv.store_rows(Vb, t);
    }
    f32x16 dk[ND], dv[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dk[i] = f32x16{};
      dv[i] = f32x16{};
    }
    const int cnt = a.inv_cnt[hg];
    const int q_lo = sp * kSplitQ;
    const int q_hi = min(cnt, q_lo + kSplitQ);
    const int32_t* lst = a.inv + a.inv_off[hg];
    const int nsteps = q_hi - q_lo;  // one query block per step
    for (int i = t; i < nsteps; i += 256) {
      const int rb = lst[q_lo + i];
      qtok_s[i] = block_token0(rb, a.nb, a.n);
      qlen_s[i] = block_len(rb % a.nb, a.n);
    }
    const uint16_t* qhp = a.q + h * a.qhs;
    const uint16_t* dhp = a.dout + h * a.dhs;
    // a step's Q and dO rows, lse and D are loaded into registers one step ahead
    Tile<D, 256> tq, td;
    float lse_r = INFINITY, d_r = 0.f;
    int len_next = 0;
    auto fetch = [&](int s) {
      const int64_t q0 = uniform64(qtok_s[s]);
      const int ql = __builtin_amdgcn_readfirstlane(qlen_s[s]);
      tq.load(qhp + q0 * a.qts, static_cast<uint32_t>(2 * a.qts), ql, t);
      td.load(dhp + q0 * a.dts, static_cast<uint32_t>(2 * a.dts), ql, t);
      if (t < kBlock) {
        // raw values: nothing may wait for these loads before the next step stores them
        lse_r = load_row_f32(a.lse + h * a.T + q0, ql, t);
        d_r = load_row_f32(a.Dw + h * a.T + q0, ql, t);
      }
      len_next = ql;
    };
    __syncthreads();  // the list is staged
    if (nsteps > 0) fetch(0);
    for (int s = 0; s < nsteps; ++s) {
      // K and V are stored; every wave is done with the previous step's tiles
      __syncthreads();
      tq.store_rows(Qs, t);
      td.store_rows(Os, t);
      const int qlen = len_next;
      if (t < kBlock) {
        // rows past the query block's length get lse = +inf, so their P is 0 (and D 0)
        lse2_s[t] = t < qlen ? lse_r * kLog2e : INFINITY;
        d_s[t] = d_r;
      }
      __syncthreads();
      if (s + 1 < nsteps) fetch(s + 1);
      if (32 * qh < qlen) {
        // S (queries x keys): A = Q rows of this wave's half, B = K rows of its keys; dP
        // likewise from dO and V
        f32x16 sacc[1], pacc[1];
        sacc[0] = f32x16{};
        pacc[0] = f32x16{};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          sacc[0] = mfma32(rd_rows<D>(Qs, qh, st, c32, h2), rd_rows<D>(Kb, kt, st, c32, h2), sacc[0]);
          pacc[0] = mfma32(rd_rows<D>(Os, qh, st, c32, h2), rd_rows<D>(Vb, kt, st, c32, h2), pacc[0]);
        }
        // lse and D of the lane's rows 8 j + 4 h2 + [0, 4), four at a time
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2_s + 32 * qh + 8 * j + 4 * h2);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(d_s + 32 * qh + 8 * j + 4 * h2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rr = 4 * j + e;
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[0][rr], c, -l4[e]));
            sacc[0][rr] = p;
            pacc[0][rr] = p * (pacc[0][rr] - d4[e]);
          }
        }
        // dV^T += dO^T P, dK^T += Q^T dS (dO, Q channel-major through the transposing read)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 pb = pack_step(sacc, t2);
          const u32x4 sb = pack_step(pacc, t2);
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            dv[dt] = mfma32(rd_rows_tr<D>(Os, dt, 2 * qh + t2, l), pb, dv[dt]);
            dk[dt] = mfma32(rd_rows_tr<D>(Qs, dt, 2 * qh + t2, l), sb, dk[dt]);
          }
        }
      }
    }
    // waves 2 and 3 hand their sums to waves 0 and 1: slot kt, f32x4 j of lane l at
    // [j][l] (dK^T registers first, then dV^T)
    __syncthreads();  // every wave is done with the tiles
    f32x4* slot = reinterpret_cast<f32x4*>(smem) + kt * kSlot;
    if (qh == 1) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          slot[(4 * dt + r) * 64 + l] =
              f32x4{dk[dt][4 * r], dk[dt][4 * r + 1], dk[dt][4 * r + 2], dk[dt][4 * r + 3]};
          slot[(4 * ND + 4 * dt + r) * 64 + l] =
              f32x4{dv[dt][4 * r], dv[dt][4 * r + 1], dv[dt][4 * r + 2], dv[dt][4 * r + 3]};
        }
    }
    __syncthreads();
    if (qh == 1) continue;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 ok = slot[(4 * dt + r) * 64 + l];
        const f32x4 ov = slot[(4 * ND + 4 * dt + r) * 64 + l];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[dt][4 * r + e] += ok[e];
          dv[dt][4 * r + e] += ov[e];
        }
      }
    if (a.nsplit[hg] == 1) {
      // a cache slot's gradient covers all 64 rows (zero past its length)
      if (key < klen || is_slot) {
        if (key >= klen) {
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            dk[dt] = f32x16{};
            dv[dt] = f32x16{};
          }
        }
        const int64_t so = (static_cast<int64_t>(h) * a.slots + g) * kBlock * D + key * D;
        uint16_t* ko = is_slot ? a.dkc + so : a.dk + h * a.dkhs + (k0 + key) * a.dkts;
        uint16_t* vo = is_slot ? a.dvc + so : a.dv + h * a.dvhs + (k0 + key) * a.dvts;
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
    } else {
      // partial slot: [thread][dK^T registers | dV^T registers] for threads 0..127 (waves
      // 0 and 1), each thread's values contiguous so the stores take immediate offsets
      // from one address
      f32x4* pp = reinterpret_cast<f32x4*>(
          a.part + static_cast<int64_t>(a.part_base[hg] + sp) * (2 * kBlock * D) +
          static_cast<int64_t>(t) * (32 * ND));
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pp[4 * dt + r] = f32x4{dk[dt][4 * r], dk[dt][4 * r + 1], dk[dt][4 * r + 2], dk[dt][4 * r + 3]};
          pp[4 * ND + 4 * dt + r] =
              f32x4{dv[dt][4 * r], dv[dt][4 * r + 1], dv[dt][4 * r + 2], dv[dt][4 * r + 3]};
        }
    }
  }
}

// ------------------------------------------------------------------ reduce
// one workgroup (128 threads) per split block: sums its partials in item order.
template <int D>
__global__ void __launch_bounds__(128) attn_bwd_reduce_kernel(BwdArgs a) {
  constexpr int ND = D / 32;
  const int j = blockIdx.x;
  if (j >= a.counts[1]) return;
  const int hg = a.long_list[j];
  const int h = hg / a.nkv, g = hg - h * a.nkv;
  const int t = threadIdx.x, l = t & 63, w = t >> 6, h2 = l >> 5, c32 = l & 31;
  const int key = 32 * w + c32;
  const bool is_slot = a.persist && g < a.slots;
  const int b = a.persist && !is_slot ? g - a.slots : g;
  const int64_t k0 = is_slot ? 0 : block_token0(b, a.nb, a.n);
  const int klen = is_slot ? a.clen[static_cast<int64_t>(h) * a.slots + g] : block_len(b % a.nb, a.n);
  const int ns = a.nsplit[hg];
  const float* p0 = a.part + static_cast<int64_t>(a.part_base[hg]) * (2 * kBlock * D);
  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  for (int sp = 0; sp < ns; ++sp) {
    const f32x4* pp = reinterpret_cast<const f32x4*>(
        p0 + static_cast<int64_t>(sp) * (2 * kBlock * D) + static_cast<int64_t>(t) * (32 * ND));
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 x = pp[4 * dt + r], y = pp[4 * ND + 4 * dt + r];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dk[dt][4 * r + e] += x[e];
          dv[dt][4 * r + e] += y[e];
        }
      }
  }
  if (key < klen || is_slot) {
    if (key >= klen) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        dk[dt] = f32x16{};
        dv[dt] = f32x16{};
      }
    }
    const int64_t so = (static_cast<int64_t>(h) * a.slots + g) * kBlock * D + key * D;
    uint16_t* ko = is_slot ? a.dkc + so : a.dk + h * a.dkhs + (k0 + key) * a.dkts;
    uint16_t* vo = is_slot ? a.dvc + so : a.dv + h * a.dvhs + (k0 + key) * a.dvts;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int ch = 32 * dt + 8 * jj + 4 * h2;
        u32x2 pk = {pack_bf16x2(dk[dt][4 * jj] * a.scale, dk[dt][4 * jj + 1] * a.scale),
                    pack_bf16x2(dk[dt][4 * jj + 2] * a.scale, dk[dt][4 * jj + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(ko + ch) = pk;
        u32x2 pv = {pack_bf16x2(dv[dt][4 * jj], dv[dt][4 * jj + 1]),
                    pack_bf16x2(dv[dt][4 * jj + 2], dv[dt][4 * jj + 3])};
        *reinterpret_cast<u32x2*>(vo + ch) = pv;
      }
  }
}

// ------------------------------------------------------------------ persistent lists
// grid (nq, H), one wave: query block r's KV list in persistent mode, as virtual block ids
// (cache slots, then the chunk's blocks at slots + b): the occupied persistent slots in
// slot order (union routing: the sink slots), the slots of its routed blocks in routed
// order, then every block of the chunk -- exactly the blocks pbsa_attn_fwd attends.
__global__ void __launch_bounds__(64) attn_bwd_lists_persist_kernel(BwdArgs a, int32_t* sel,
                                                                    int32_t* nsel) {
  const int r = blockIdx.x, h = blockIdx.y, l = threadIdx.x;
  const int64_t hr = static_cast<int64_t>(h) * a.nq + r;
  int32_t* out = sel + hr * a.max_sel;
  const int32_t* bid = a.cbid + static_cast<int64_t>(h) * a.slots;
  const unsigned long long below = (1ull << l) - 1ull;
  const int whole = a.route_union ? a.S : a.C;
  int n = 0;
  for (int s0 = 0; s0 < whole; s0 += 64) {
    const int s = s0 + l;
    const bool on = s < whole && bid[s] >= 0;
    const unsigned long long m = __ballot(on);
    if (on) out[n + __popcll(m & below)] = s;
    n += __popcll(m);
  }
  const int32_t* rs = a.rsel + hr * a.K;
  for (int j0 = 0; j0 < a.K; j0 += 64) {
    const int j = j0 + l;
    const int g = j < a.K ? rs[j] : -1;
    int slot = -1;
    if (g >= 0) {
      slot = a.C + ((g / a.nb) % a.W) * a.nb + g % a.nb;
      if (a.route_union && bid[slot] != g) {
        // a persistent block (an id the cache does not hold is left out)
        slot = -1;
        for (int ps = a.S; ps < a.C; ++ps)
          if (bid[ps] == g) {
            slot = ps;
            break;
          }
      }
    }
    const bool on = slot >= 0;
    const unsigned long long m = __ballot(on);
    if (on) out[n + __popcll(m & below)] = slot;
    n += __popcll(m);
  }
  for (int b = l; b < a.nq; b += 64) out[n + b] = a.slots + b;
  n += a.nq;
  if (l == 0) nsel[hr] = n;
}

namespace {
// Workspace layout of the backward (bytes, 256-aligned pieces).  Persistent mode adds the
// query blocks' KV lists and their lengths.
struct BwdWs {
  size_t D, inv_cnt, inv_off, inv, bits, items, sorted, nsplit, part_base, long_list, counts,
      part, lists, nlists, total;
};
BwdWs bwd_ws(int64_t H, int64_t nq, int64_t nkv, int64_t T, int64_t max_sel, int head_dim,
             bool persist) {
  const int64_t pairs_max = H * nq * max_sel;                  // selected (query, KV) pairs
  const int64_t items_max = H * nkv + pairs_max / kSplitQ + 1;  // work items
  const int64_t parts_max = 2 * (pairs_max / kSplitQ) + 2;      // partial slots
  auto up = [](size_t x) { return (x + 255) & ~size_t{255}; };
  BwdWs w{};
  size_t o = 0;
  w.D = o; o += up(H * T * 4);
  w.inv_cnt = o; o += up(H * nkv * 4);
  w.inv_off = o; o += up(H * nkv * 4);
  w.inv = o; o += up(pairs_max * 4);
  w.bits = o; o += up(H * nkv * ((nq + 31) / 32) * 4);
  w.items = o; o += up(items_max * 8);
  w.sorted = o; o += up(items_max * 8);
  w.nsplit = o; o += up(H * nkv * 4);
  w.part_base = o; o += up(H * nkv * 4);
  w.long_list = o; o += up(H * nkv * 4);
  w.counts = o; o += up(16);
  w.part = o; o += up(static_cast<size_t>(parts_max) * 2 * kBlock * head_dim * 4);
  w.lists = o; o += persist ? up(H * nq * max_sel * 4) : 0;
  w.nlists = o; o += persist ? up(H * nq * 4) : 0;
  w.total = o;
  return w;
}

int64_t persist_max_sel(const pbsa_dims& d) {
  return static_cast<int64_t>(d.capacity) + d.topk + static_cast<int64_t>(d.chunk_frames) * nb_of(d);
}

void bind_ws(BwdArgs& a, const BwdWs& L, void* ws) {
  char* p = static_cast<char*>(ws);
  a.Dw = reinterpret_cast<float*>(p + L.D);
  a.inv_cnt = reinterpret_cast<int32_t*>(p + L.inv_cnt);
  a.inv_off = reinterpret_cast<int32_t*>(p + L.inv_off);
  a.inv = reinterpret_cast<int32_t*>(p + L.inv);
  a.bits = reinterpret_cast<uint32_t*>(p + L.bits);
  a.items = reinterpret_cast<int2*>(p + L.items);
  a.sorted = reinterpret_cast<int2*>(p + L.sorted);
  a.nsplit = reinterpret_cast<int32_t*>(p + L.nsplit);
  a.part_base = reinterpret_cast<int32_t*>(p + L.part_base);
  a.long_list = reinterpret_cast<int32_t*>(p + L.long_list);
  a.counts = reinterpret_cast<int32_t*>(p + L.counts);
  a.part = reinterpret_cast<float*>(p + L.part);
}

void bind_tokens(BwdArgs& a, TokIn q, TokIn k, TokIn v, TokIn o, const float* lse, TokIn dout,
                 TokOut dq, TokOut dk, TokOut dv) {
  a.q = q.p; a.qts = q.ts; a.qhs = q.hs;
  a.k = k.p; a.kts = k.ts; a.khs = k.hs;
  a.v = v.p; a.vts = v.ts; a.vhs = v.hs;
  a.o = o.p; a.ots = o.ts; a.ohs = o.hs;
  a.dout = dout.p; a.dts = dout.ts; a.dhs = dout.hs;
  a.dq = dq.p; a.dqts = dq.ts; a.dqhs = dq.hs;
  a.dk = dk.p; a.dkts = dk.ts; a.dkhs = dk.hs;
  a.dv = dv.p; a.dvts = dv.ts; a.dvhs = dv.hs;
  a.lse = lse;
}

// dQ pass, inverse lists, plan, dK/dV pass, reduce (a fully set up).
hipError_t launch_bwd_passes(const BwdArgs& a, int head_dim, hipStream_t s) {
  const int gq = 8 * cdiv(a.H * a.pairs, 8);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, dim3(gq), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, dim3(gq), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nq > 32 * kMaxBitWords) return hipErrorInvalidValue;
  {
    const int64_t words = static_cast<int64_t>(a.H) * a.nkv * ((a.nq + 31) / 32);
    const int64_t blocks = (words + 255) / 256;
    const int gc = static_cast<int>(blocks < 2048 ? blocks : 2048);
    hipLaunchKernelGGL(attn_bwd_bits_clear_kernel, dim3(gc), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL(attn_bwd_bits_set_kernel, dim3(a.nq, a.H), dim3(128), 0, s, a);
  hipLaunchKernelGGL(attn_bwd_bits_count_kernel, dim3(cdiv(a.H * a.nkv, 256)), dim3(256), 0, s,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_plan_kernel, dim3(1), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(attn_bwd_bits_list_kernel, dim3(a.nkv, a.H), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items_max = static_cast<int64_t>(a.H) * a.nkv +
                            static_cast<int64_t>(a.H) * a.nq * a.max_sel / kSplitQ + 1;
  // enough workgroups to fill every CU; they take items from the counter until none is left
  const int gi = static_cast<int>(items_max < 1024 ? items_max : 1024);
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, dim3(gi), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, dim3(gi), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int gr = a.H * a.nkv;
  if (head_dim == 128)
    hipLaunchKernelGGL(attn_bwd_reduce_kernel<128>, dim3(gr), dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL(attn_bwd_reduce_kernel<64>, dim3(gr), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace(const pbsa_dims& d, int chunks, int max_sel) {
  const int64_t nq = static_cast<int64_t>(chunks) * d.chunk_frames * nb_of(d);
  const int64_t T = static_cast<int64_t>(chunks) * d.chunk_frames * d.frame_tokens;
  return bwd_ws(d.heads, nq, nq, T, max_sel, d.head_dim, false).total;
}

size_t attn_bwd_persistent_workspace(const pbsa_dims& d) {
  const int64_t nq = static_cast<int64_t>(d.chunk_frames) * nb_of(d);
  const int64_t T = static_cast<int64_t>(d.chunk_frames) * d.frame_tokens;
  return bwd_ws(d.heads, nq, slots_of(d) + nq, T, persist_max_sel(d), d.head_dim, true).total;
}

hipError_t launch_attn_bwd(const pbsa_dims& d, int chunks, TokIn q, TokIn k, TokIn v, TokIn o,
                           const float* lse, TokIn dout, const int32_t* sel,
                           const int32_t* nsel, int max_sel, TokOut dq, TokOut dk, TokOut dv,
                           void* ws, hipStream_t s) {
  const int nb = nb_of(d);
  const int nq = chunks * d.chunk_frames * nb;
  const int64_t T = static_cast<int64_t>(chunks) * d.chunk_frames * d.frame_tokens;
  BwdArgs a{};
  bind_tokens(a, q, k, v, o, lse, dout, dq, dk, dv);
  a.sel = sel;
  a.nsel = nsel;
  bind_ws(a, bwd_ws(d.heads, nq, nq, T, max_sel, d.head_dim, false), ws);
  a.T = T;
  a.nq = nq;
  a.nkv = nq;
  a.persist = 0;
  a.nb = nb;
  a.n = d.frame_tokens;
  a.F = d.chunk_frames;
  a.max_sel = max_sel;
  a.H = d.heads;
  a.pairs = cdiv(nq, 2);
  a.scale = d.scale;
  return launch_bwd_passes(a, d.head_dim, s);
}

hipError_t launch_attn_bwd_persistent(const pbsa_dims& d, TokIn q, const pbsa_cache& c,
                                      TokIn ck, TokIn cv, const int32_t* sel, TokIn o,
                                      const float* lse, TokIn dout, TokOut dq, TokOut dk,
                                      TokOut dv, uint16_t* dk_cache, uint16_t* dv_cache,
                                      void* ws, hipStream_t s) {
  const int nb = nb_of(d);
  const int nq = d.chunk_frames * nb;
  const int64_t T = static_cast<int64_t>(d.chunk_frames) * d.frame_tokens;
  const int slots = static_cast<int>(slots_of(d));
  const int max_sel = static_cast<int>(persist_max_sel(d));
  BwdArgs a{};
  bind_tokens(a, q, ck, cv, o, lse, dout, dq, dk, dv);
  const BwdWs L = bwd_ws(d.heads, nq, slots + nq, T, max_sel, d.head_dim, true);
  bind_ws(a, L, ws);
  char* p = static_cast<char*>(ws);
  int32_t* lists = reinterpret_cast<int32_t*>(p + L.lists);
  int32_t* nlists = reinterpret_cast<int32_t*>(p + L.nlists);
  a.sel = lists;
  a.nsel = nlists;
  a.T = T;
  a.nq = nq;
  a.nkv = slots + nq;
  a.persist = 1;
  a.ck = static_cast<const uint16_t*>(c.k);
  a.cv = static_cast<const uint16_t*>(c.v);
  a.cbid = c.block_id;
  a.clen = c.len;
  a.slots = slots;
  a.C = d.capacity;
  a.W = d.window_frames;
  a.K = d.topk;
  a.S = d.sinks;
  a.route_union = d.route_mode == PBSA_ROUTE_UNION;
  a.rsel = sel;
  a.dkc = dk_cache;
  a.dvc = dv_cache;
  a.nb = nb;
  a.n = d.frame_tokens;
  a.F = d.chunk_frames;
  a.max_sel = max_sel;
  a.H = d.heads;
  a.pairs = cdiv(nq, 2);
  a.scale = d.scale;
  hipLaunchKernelGGL(attn_bwd_lists_persist_kernel, dim3(nq, d.heads), dim3(64), 0, s, a, lists,
                     nlists);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_passes(a, d.head_dim, s);
}

}  // namespace pbsa
