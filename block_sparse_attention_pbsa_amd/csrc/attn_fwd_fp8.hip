// Attention over selected blocks with an FP8 KV cache (persistent mode).
//
// Light Forcing (papernotes.org), "Key findings": the sparse attention is deployed with FP8
// (after Sparse Forcing's own mechanism, gist.science 2.C: persistent blocks, routed window
// blocks and the chunk, online softmax).  The cache keeps every block's K and V as OCP E4M3
// codes with one power-of-two scale per block and tensor (written by the memory update),
// which halves the cache's bytes and the bytes each gather moves; the current chunk's own
// K and V stay bf16.  Decoded values (code x scale) are exact in bf16, so the attention is
// the same bf16-MFMA attention over the decoded blocks.
//
// gfx950 design (a register-staged variant of the attention, simpler than the bf16
// kernel's direct-to-LDS gathers): one workgroup = two 64-row query blocks A and B of one
// head, four waves of 32 query rows (Q in registers).  Each query block has its own list
// (the whole persistent slots -- or only the sinks with union routing --, its routed
// blocks, the chunk's blocks); step s takes half s % 2 of the (s / 2)-th block of A's list
// (X) and of B's list (Y).  All 256 threads load the next step's four half tiles (K and V
// of X and Y: 16 codes or 16 bf16 per thread and tile) into registers while the waves
// compute; after a barrier they decode and store them as bf16 into row-major LDS tiles.
// S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 (V channel-major through the
// transposing LDS read), base-2 online softmax with a running max.
#include "attn_common.h"

namespace pbsa {

struct Fp8Args {
  const uint16_t* q;
  int64_t qts, qhs;
  uint16_t* o;
  int64_t ots, ohs;
  float* lse;
  const uint8_t* ck;     // cache K codes [H][slots][64][D]
  const uint8_t* cv;
  const float* kv_scale; // [H][slots][2]: K scale, V scale
  const int32_t* bid;    // [H][slots]
  const int32_t* blen;
  const uint16_t* xk;    // the chunk's K, V (bf16 tokens)
  const uint16_t* xv;
  int64_t xts, xhs;
  const int32_t* sel;    // [H][nq][K] routed ids
  int slots, C, W, S, K, route_union;
  int nq, n, nb, H, pairs, T;
  float scale;
};

namespace {

// A half tile in flight: 32 rows starting at `row0` of either a cache slot (codes) or the
// chunk (bf16 tokens); this thread's 16 values of row `rr`.
struct Fp8Half {
  u32x4 raw0, raw1;  // codes in raw0 (slot), or 16 bf16 in raw0, raw1 (chunk)
  float scale;
  int len;           // valid rows of the half tile
  bool slot;
};

}  // namespace

template <int D>
__global__ void __launch_bounds__(256, 2) attn_fwd_fp8_kernel(Fp8Args a) {
  static_assert(D == 128, "the FP8 cache is built for head_dim 128");
  constexpr int NS = D / 16, ND = D / 32;
  constexpr int HT = 32 * Lds<D>::RS;  // elements of one 32-row half tile
  __shared__ __attribute__((aligned(16))) uint16_t tiles[4 * HT];  // K X, V X, K Y, V Y
  __shared__ uint32_t lst[2][kAttnListCap / 2];
  __shared__ int cnt_s[2];

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
  const int32_t* bh = a.bid + static_cast<int64_t>(h) * a.slots;
  const int32_t* lh = a.blen + static_cast<int64_t>(h) * a.slots;

  // Lists (entries: bit 31 = a cache slot, bits 0..23 the slot, else the chunk token block
  // starting at bits 0..23; bits 24..30 valid rows): wave 0 builds A's, wave 1 B's.
  if (w < 2) {
    const int rq = w == 0 ? rA : rB;
    uint32_t* out = lst[w];
    const unsigned long long below = (1ull << l) - 1ull;
    int n = 0;
    if (rq < a.nq) {
      const int whole = a.route_union ? a.S : a.C;
      for (int s0 = 0; s0 < whole; s0 += 64) {
        const int s = s0 + l;
        const bool on = s < whole && bh[s] >= 0;
        const unsigned long long m = __ballot(on);
        if (on) out[n + __popcll(m & below)] = 0x80000000u | (static_cast<uint32_t>(lh[s]) << 24) | s;
        n += __popcll(m);
      }
      const int32_t* rs = a.sel + (static_cast<int64_t>(h) * a.nq + rq) * a.K;
      for (int j0 = 0; j0 < a.K; j0 += 64) {
        const int j = j0 + l;
        const int g = j < a.K ? rs[j] : -1;
        int slot = -1;
        if (g >= 0) {
          slot = a.C + ((g / a.nb) % a.W) * a.nb + g % a.nb;
          if (slot >= a.slots || bh[slot] != g) {
            // a persistent block (union routing); an id the cache does not hold is left out
            slot = -1;
            for (int ps = a.S; a.route_union && ps < a.C; ++ps)
              if (bh[ps] == g) {
                slot = ps;
                break;
              }
          }
        }
        const bool on = slot >= 0;
        const unsigned long long m = __ballot(on);
        if (on) out[n + __popcll(m & below)] = 0x80000000u | (static_cast<uint32_t>(lh[slot]) << 24) | slot;
        n += __popcll(m);
      }
      for (int b = l; b < a.nq; b += 64)
        out[n + b] = (static_cast<uint32_t>(block_len(b % a.nb, a.n)) << 24) |
                     static_cast<uint32_t>(block_token0(b, a.nb, a.n));
      n += a.nq;
    }
    if (l == 0) cnt_s[w] = n;
  }

  u32x4 qreg[NS];
  load_row_operand<D>(qreg, a.q + h * a.qhs + t0 * a.qts, a.qts, qrow, qlen, h2);
  f32x16 acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = f32x16{};
  float m_run = -3.0e38f, l_run = 0.f;
  __syncthreads();
  const int cntA = cnt_s[0], cntB = cnt_s[1];
  const int nsteps = 2 * (cntA > cntB ? cntA : cntB);

  const uint8_t* ckh = a.ck + static_cast<int64_t>(h) * a.slots * kBlock * D;
  const uint8_t* cvh = a.cv + static_cast<int64_t>(h) * a.slots * kBlock * D;
  const float* sch = a.kv_scale + static_cast<int64_t>(h) * a.slots * 2;
  const uint16_t* xkh = a.xk + h * a.xhs;
  const uint16_t* xvh = a.xv + h * a.xhs;
  // this thread's row and 16-value piece of every half tile
  const int rr = t >> 3, pc = t & 7;

  // load tile `which` (0 K X, 1 V X, 2 K Y, 3 V Y) of step s into registers
  auto load = [&](int s, int which, Fp8Half& hf) {
    const int j = s >> 1, half = s & 1;
    const bool y = which >= 2, isv = which & 1;
    hf.len = 0;
    hf.slot = false;
    hf.scale = 1.f;
    if (j >= (y ? cntB : cntA)) return;
    const uint32_t e = lst[y][j];
    const int len = static_cast<int>((e >> 24) & 0x7f) - 32 * half;
    hf.len = len < 0 ? 0 : (len < 32 ? len : 32);
    hf.slot = (e >> 31) != 0;
    if (rr >= hf.len) return;
    if (hf.slot) {
      const int s_ = static_cast<int>(e & 0xffffffu);
      const int64_t off = (static_cast<int64_t>(s_) * kBlock + 32 * half + rr) * D + 16 * pc;
      hf.raw0 = *reinterpret_cast<const u32x4*>((isv ? cvh : ckh) + off);
      hf.scale = sch[2 * s_ + (isv ? 1 : 0)];
    } else {
      const int64_t tok = static_cast<int64_t>(e & 0xffffffu) + 32 * half + rr;
      const uint16_t* p = (isv ? xvh : xkh) + tok * a.xts + 16 * pc;
      hf.raw0 = *reinterpret_cast<const u32x4*>(p);
      hf.raw1 = *reinterpret_cast<const u32x4*>(p + 8);
    }
  };
  // decode (codes) and store this thread's piece of a tile; rows past the length are zero
  auto store = [&](const Fp8Half& hf, uint16_t* tile) {
    u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (rr < hf.len) {
      if (hf.slot) {
        decode_e4m3x16(hf.raw0, hf.scale, lo, hi);
      } else {
        lo = hf.raw0;
        hi = hf.raw1;
      }
    }
    *reinterpret_cast<u32x4*>(tile + Lds<D>::chunk(rr, 2 * pc)) = lo;
    *reinterpret_cast<u32x4*>(tile + Lds<D>::chunk(rr, 2 * pc + 1)) = hi;
  };

  int trlo[ND], trhi[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) tr_offsets<D>(dt, l, trlo[dt], trhi[dt]);

  Fp8Half hx[4];
  if (nsteps > 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) load(0, i, hx[i]);
  for (int s = 0; s < nsteps; ++s) {
    __syncthreads();  // every wave is done with the previous step's tiles
#pragma unroll
    for (int i = 0; i < 4; ++i) store(hx[i], tiles + i * HT);
    const int len = mine ? hx[2].len : hx[0].len;
    __syncthreads();
    if (s + 1 < nsteps)
#pragma unroll
      for (int i = 0; i < 4; ++i) load(s + 1, i, hx[i]);
    if (qlen == 0 || len == 0) continue;
    const uint16_t* kt = tiles + (2 * mine) * HT;
    const uint16_t* vt = tiles + (2 * mine + 1) * HT;
    // S^T: keys acc_row(r, h2) of the half tile, this lane's query row c32
    f32x16 sa = {};
#pragma unroll
    for (int st = 0; st < NS; ++st) sa = mfma32(rd_rows<D>(kt, 0, st, c32, h2), qreg[st], sa);
    float mx = -INFINITY;
#pragma unroll
    for (int rr2 = 0; rr2 < 16; ++rr2) {
      if (acc_row(rr2, h2) >= len) sa[rr2] = -INFINITY;
      mx = fmaxf(mx, sa[rr2]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.f;
#pragma unroll
    for (int rr2 = 0; rr2 < 16; ++rr2) {
      sa[rr2] = __builtin_amdgcn_exp2f(fmaf(sa[rr2], c, -m_new));
      ps += sa[rr2];
    }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
    // O^T += V^T P^T (V channel-major through the transposing read)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const u32x4 pb = pack_step(&sa, t2);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
        acc[dt] = mfma32(rd_tr(vt, trlo[dt] + 16 * t2 * Lds<D>::RS, trhi[dt] + 16 * t2 * Lds<D>::RS),
                         pb, acc[dt]);
    }
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qrow < qlen) {
    const float inv = 1.f / l_tot;
    uint16_t* orow = a.o + h * a.ohs + (t0 + qrow) * a.ots;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ch = 32 * dt + 8 * j + 4 * h2;
        u32x2 pk = {pack_bf16x2(acc[dt][4 * j] * inv, acc[dt][4 * j + 1] * inv),
                    pack_bf16x2(acc[dt][4 * j + 2] * inv, acc[dt][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + ch) = pk;
      }
    if (h2 == 0) a.lse[h * a.T + t0 + qrow] = m_run * kLn2 + logf(l_tot);
  }
}

hipError_t launch_attn_fwd_fp8(const pbsa_dims& d, TokIn q, const pbsa_cache& c, TokIn ck,
                               TokIn cv, const int32_t* sel, TokOut o, float* lse,
                               hipStream_t s) {
  Fp8Args a{};
  const int nb = nb_of(d);
  a.q = q.p; a.qts = q.ts; a.qhs = q.hs;
  a.o = o.p; a.ots = o.ts; a.ohs = o.hs;
  a.lse = lse;
  a.ck = static_cast<const uint8_t*>(c.k);
  a.cv = static_cast<const uint8_t*>(c.v);
  a.kv_scale = c.kv_scale;
  a.bid = c.block_id;
  a.blen = c.len;
  a.xk = ck.p; a.xv = cv.p; a.xts = ck.ts; a.xhs = ck.hs;
  a.sel = sel;
  a.slots = static_cast<int>(slots_of(d));
  a.C = d.capacity;
  a.W = d.window_frames;
  a.S = d.sinks;
  a.K = d.topk;
  a.route_union = d.route_mode == PBSA_ROUTE_UNION;
  a.nq = d.chunk_frames * nb;
  a.n = d.frame_tokens;
  a.nb = nb;
  a.H = d.heads;
  a.pairs = cdiv(a.nq, 2);
  a.T = d.chunk_frames * d.frame_tokens;
  a.scale = d.scale;
  const int G = a.H * a.pairs;
  hipLaunchKernelGGL(attn_fwd_fp8_kernel<128>, dim3(8 * cdiv(G, 8)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pbsa
