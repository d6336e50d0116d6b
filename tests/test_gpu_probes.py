"""The measurement probes (pbsa_probe.h) run through the C ABI and leave the attention's
outputs alone; their timings are reported by bench.py, not checked here."""
import numpy as np
import pytest
import torch

from block_sparse_attention_pbsa_amd import ops, runtime, synth
from parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()
    yield
    torch.cuda.synchronize()


def test_probe_mfma_counts_and_finishes():
    say("[probe] mfma")
    out = torch.zeros(131072, dtype=torch.float32, device="cuda")
    flop = ops.pbsa_probe_mfma(8, out)
    torch.cuda.synchronize()
    assert flop == 8 * 512 * 4 * 4 * 2 * 32 * 32 * 16
    o = out.cpu().numpy()
    assert np.isfinite(o).all() and (o != 0).all()


def test_probe_gather_leaves_outputs_alone():
    wl = synth.WORKLOADS["tiny"]
    shape = ops.Shape(wl.heads, wl.head_dim, wl.frame_tokens, wl.chunk_frames, wl.window_frames,
                      wl.capacity, wl.sinks, wl.topk, wl.scale)
    layer = runtime.PersistentLayer(shape)
    layer.reset()
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    for c in range(wl.measured_chunk):
        q, k, v = synth.chunk_qkv(wl, 5, c)
        layer.step(dev(q), dev(k), dev(v), attend=False)
    q, k, v = (dev(x) for x in synth.chunk_qkv(wl, 5, wl.measured_chunk))
    layer.route(q)
    layer.attend(q, k, v)
    torch.cuda.synchronize()
    o0, l0 = layer.o.clone(), layer.lse.clone()
    say("[probe] gather")
    ops.pbsa_probe_gather(shape, q, layer.cache, k, v, layer.sel)
    torch.cuda.synchronize()
    assert torch.equal(layer.o, o0) and torch.equal(layer.lse, l0)
