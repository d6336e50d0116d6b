"""Attention over KV blocks whose scores differ by hundreds of exp2 units, so that the online
softmax has to move its offset in the middle of a row: later blocks that overflow exp2
against the offset the first blocks set (head 0), and first blocks far below everything
after them (head 1).  Every query row against the fp64 definition (masked softmax over the
persistent blocks, the GPU's routed window blocks and the chunk).

Construction: every query has 4 in channel 0; a key block with bias b has b in channel 0,
so its scores are about 4 b * scale (other channels standard normal)."""
import numpy as np
import pytest
import torch

import oracle as orc
from block_sparse_attention_pbsa_amd import ops, synth
from parity import ATTN_MAX, ATTN_MEAN, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


N_TOK, NB, W, C, TOPK = 200, 4, 6, 8, 6   # 3 full blocks + an 8-token tail per frame
F_LAST = 20                                # window holds frames 15..20, the chunk is 21

# per head: bias of the persistent blocks, of the chunk, and the cycle of window biases
BIAS = [
    (0.0, 50.0, (0.0, 100.0, 300.0)),      # growth: chunk 2^25 above P, window overflows
    (-800.0, 0.0, (0.0, 20.0, -800.0)),    # first blocks hundreds of exp2 units below
]


@pytest.mark.parametrize("head_dim", [128, 64])
def test_attn_fwd_offset_moves_mid_row(head_dim):
    H, D = len(BIAS), head_dim
    shape = ops.Shape(H, D, N_TOK, 1, W, C, 1, TOPK)
    rng = np.random.default_rng(9100 + D)
    slots = shape.slots
    bid = np.full((H, slots), -1, np.int32)
    bias = np.zeros((H, slots))
    for h, (bp, _, cyc) in enumerate(BIAS):
        old = rng.choice(np.arange(1, (F_LAST - W + 1) * NB), C - 1, replace=False)
        bid[h, 0] = 0
        bid[h, 1:C] = np.sort(old)
        bias[h, :C] = bp
        for f in range(F_LAST - W + 1, F_LAST + 1):
            for j in range(NB):
                s = C + (f % W) * NB + j
                bid[h, s] = f * NB + j
                bias[h, s] = cyc[(f * NB + j) % len(cyc)]
    blen = np.where(bid >= 0, np.where(bid % NB == NB - 1, N_TOK - 64 * (NB - 1), 64), 0)
    kc = rng.standard_normal((H, slots, 64, D)).astype(np.float32)
    kc[..., 0] = bias[:, :, None]
    kc = synth.round_bf16(kc)
    vc = synth.round_bf16(rng.standard_normal((H, slots, 64, D)).astype(np.float32))
    for h in range(H):
        for s in range(slots):
            kc[h, s, blen[h, s]:] = 0
            vc[h, s, blen[h, s]:] = 0
    rep = kc.mean(axis=2).astype(np.float32)
    cache = ops.Cache(shape)
    cache.block_id.copy_(torch.from_numpy(bid))
    cache.len.copy_(torch.from_numpy(blen.astype(np.int32)))
    cache.k.copy_(torch.from_numpy(kc).to(torch.bfloat16))
    cache.v.copy_(torch.from_numpy(vc).to(torch.bfloat16))
    cache.rep.copy_(torch.from_numpy(rep))
    cache.chunk_index = F_LAST + 1
    q = rng.standard_normal((N_TOK, H, D)).astype(np.float32)
    q[:, :, 0] = 4.0
    k = rng.standard_normal((N_TOK, H, D)).astype(np.float32)
    for h, (_, bc, _) in enumerate(BIAS):
        k[:, h, 0] = bc
    q, k = synth.round_bf16(q), synth.round_bf16(k)
    v = synth.round_bf16(rng.standard_normal((N_TOK, H, D)).astype(np.float32))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    scores = torch.empty(H, shape.nq, slots, dtype=torch.float32, device="cuda")
    sel = torch.empty(H, shape.nq, TOPK, dtype=torch.int32, device="cuda")
    o = torch.empty(N_TOK, H, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(H, N_TOK, dtype=torch.float32, device="cuda")
    say(f"[softmax range] D={D}")
    ops.pbsa_route(shape, dev(q), cache, None, scores, sel)
    ops.pbsa_attn_fwd(shape, dev(q), cache, dev(k), dev(v), sel, o, lse)
    torch.cuda.synchronize()
    sl = sel.cpu().numpy()
    og = o.float().cpu().numpy()
    lg = lse.cpu().numpy()
    scale = shape.c().scale
    for h in range(H):
        slot_of = {int(g): s for s, g in enumerate(bid[h])}
        P = [s for s in range(C) if bid[h, s] >= 0]
        err = []
        spread = 0.0
        for r in range(shape.nq):
            picked = [slot_of[int(g)] for g in sl[h, r] if g >= 0]
            assert len(picked) == TOPK
            K = np.concatenate([kc[h, s, :blen[h, s]] for s in P + picked] + [k[:, h]])
            V = np.concatenate([vc[h, s, :blen[h, s]] for s in P + picked] + [v[:, h]])
            rows = slice(64 * r, min(64 * r + 64, N_TOK))
            qq = q[rows, h].astype(np.float64)
            o_ref, lse_ref = orc.masked_attention(qq, K, V, np.ones((len(qq), len(K)), bool),
                                                  scale)
            s_all = scale * qq @ K.astype(np.float64).T
            spread = max(spread, float((s_all.max(1) - s_all.min(1)).max()))
            err.append(np.abs(og[rows, h] - o_ref))
            assert np.abs(lg[h, rows] - lse_ref).max() < 1e-3, f"lse head {h} block {r}"
        err = np.concatenate(err)
        say(f"  head {h}: score spread {spread:.0f} nats, max err {err.max():.2e}, "
            f"mean {err.mean():.2e}")
        assert spread > 100.0  # the construction really spans the range it is meant to
        assert err.max() < ATTN_MAX and err.mean() < ATTN_MEAN
