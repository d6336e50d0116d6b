"""The allocation-free memory update (library-held scratch) against the workspace version.

Two rollouts of the same seeded chunks, one updated through pbsa_memory_update with a
caller workspace and one through pbsa_memory_update_noalloc; after every update both
caches must hold the same bytes.  The second workload is smaller than the first, so the
scratch is reused with a smaller layout right after a larger one.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_pbsa_amd import ops, runtime, synth
from parity import say


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)


def _shape(wl):
    return ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                     wl.capacity, wl.sinks, wl.topk, wl.scale)


@pytest.mark.gpu
@pytest.mark.parametrize("name,chunks", [("wan_5s", 8), ("tiny", 5)])
def test_memory_update_noalloc_matches_workspace_version(name, chunks):
    wl, seed = synth.WORKLOADS[name], synth.SEEDS[name]
    shape = _shape(wl)
    say(f"noalloc update vs workspace update: {name}, {chunks} chunks")
    a = runtime.PersistentLayer(shape)
    a.reset()
    b = ops.Cache(shape)
    ops.pbsa_cache_reset(shape, b)
    for c in range(chunks):
        q, k, v = (_dev(x) for x in synth.chunk_qkv(wl, seed, c))
        # both caches are routed from cache a (their contents must be equal anyway)
        a.route(q)
        ops.pbsa_memory_update_noalloc(shape, a.scores, b, k, v, None)
        a.update(k, v)
        torch.cuda.synchronize()
        for nm in ("k", "v", "rep", "block_id", "len"):
            assert torch.equal(getattr(a.cache, nm), getattr(b, nm)), (name, c, nm)
        assert a.cache.chunk_index == b.chunk_index == c + 1


@pytest.mark.gpu
def test_memory_update_noalloc_rejects_oversized_dims():
    # 128 heads x capacity 1025: the persistent tables alone exceed the 1 MiB scratch
    big = ops.Shape(heads=128, head_dim=64, frame_tokens=64, chunk_frames=1, window_frames=1,
                    capacity=1025, sinks=1, topk=1)
    assert ops.pbsa_workspace_bytes(big, ops.PBSA_OP_MEMORY_UPDATE) > (1 << 20)
    cache = ops.Cache(big)
    scores = torch.zeros(big.heads, big.nq, big.slots, dtype=torch.float32, device="cuda")
    k = torch.zeros(big.chunk_tokens, big.heads, big.head_dim, dtype=torch.bfloat16,
                    device="cuda")
    with pytest.raises(ops.PbsaError) as e:
        ops.pbsa_memory_update_noalloc(big, scores, cache, k, k, None)
    assert e.value.status == 3 and "scratch" in str(e.value)
    assert cache.chunk_index == 0
