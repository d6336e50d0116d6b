"""CPU checks of the C ABI: the library loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_pbsa_amd import ops, runtime

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pbsa.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

pytestmark = pytest.mark.skipif(not os.path.exists(ops._LIB_PATH),
                                reason="libpbsa.so not built (run __graft_entry__.build())")


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pbsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("pbsa_pool", "pbsa_score_topk", "pbsa_attn_fwd", "pbsa_attn_bwd",
              "pbsa_memory_update"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(ops._LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    assert set(declared_functions()) == set(ops.exported_symbols())


def test_abi_version_and_status_strings():
    L = ops.lib()
    assert L.pbsa_abi_version() == 2
    assert L.pbsa_status_str(0) == b"ok"
    assert L.pbsa_status_str(5) == b"workspace too small"
    assert L.pbsa_status_str(99) == b"unknown status"


WAN = ops.Shape(heads=12, head_dim=128, frame_tokens=1560, chunk_frames=3, window_frames=6,
                capacity=64, sinks=1, topk=32)


def _dims(**kw):
    base = dict(heads=12, head_dim=128, block=64, frame_tokens=1560, chunk_frames=3,
                window_frames=6, capacity=64, sinks=1, topk=32, scale=128 ** -0.5)
    base.update(kw)
    return ops.Dims(**base)


@pytest.mark.parametrize("kw,mode,status", [
    (dict(), 0, 0),
    (dict(), 1, 0),
    (dict(head_dim=96), 0, 3),
    (dict(head_dim=0), 0, 2),
    (dict(block=32), 0, 3),
    (dict(heads=0), 0, 2),
    (dict(window_frames=2), 0, 2),       # W < F
    (dict(window_frames=2), 1, 0),       # two-level calls ignore W
    (dict(sinks=65), 0, 2),              # S > C
    (dict(sinks=26), 0, 2),              # S > blocks per frame
    (dict(topk=0), 0, 2),
    (dict(scale=0.0), 0, 2),
    (dict(scale=float("nan")), 1, 2),
    (dict(capacity=5000), 0, 3),
    (dict(topk=1025), 0, 3),             # topk above the supported maximum
])
def test_check_dims(kw, mode, status):
    L = ops.lib()
    st = L.pbsa_check_dims(ctypes.byref(_dims(**kw)), mode)
    assert st == status, L.pbsa_last_error()
    if status:
        assert L.pbsa_last_error()


def test_null_dims_and_sizes():
    L = ops.lib()
    assert L.pbsa_check_dims(None, 0) == 1
    assert L.pbsa_cache_slots(ctypes.byref(_dims())) == 64 + 6 * 25
    assert L.pbsa_cache_slots(ctypes.byref(_dims(head_dim=3))) == 0
    # copy list [H][F*nb], the new persistent table [H][C] twice, the chunk index used,
    # 256-byte pieces
    up = lambda x: (x + 255) // 256 * 256
    assert ops.pbsa_workspace_bytes(WAN, ops.PBSA_OP_MEMORY_UPDATE) == (
        up(4 * 12 * 75) + 2 * up(4 * 12 * 64) + up(8))
    assert ops.pbsa_workspace_bytes(WAN, ops.PBSA_OP_ATTN_BWD, 8, 75) > 12 * 600 * 600 * 4
    assert ops.pbsa_workspace_bytes(WAN, 77) == 0


def _tensor(ptr, ts=12 * 128, hs=128):
    return ops.Tensor(ptr, ts, hs)


def test_calls_reject_bad_arguments_before_launching():
    L = ops.lib()
    d = ctypes.byref(_dims())
    # NULL token pointer
    assert L.pbsa_pool(d, _tensor(None), 3, ctypes.c_void_p(16), None, None) == 1
    # misaligned token pointer and stride
    assert L.pbsa_pool(d, _tensor(8), 3, ctypes.c_void_p(16), None, None) == 4
    assert L.pbsa_pool(d, _tensor(16, ts=12 * 128 + 4), 3, ctypes.c_void_p(16), None, None) == 4
    # negative frame count
    assert L.pbsa_pool(d, _tensor(16), -1, ctypes.c_void_p(16), None, None) == 2
    # cache with a NULL buffer
    cache = ops.CacheC(16, 16, 16, None, 16, 0)
    assert L.pbsa_score_topk(d, ctypes.c_void_p(16), ctypes.byref(cache), ctypes.c_void_p(16),
                             ctypes.c_void_p(16), None) == 1
    # negative chunk index
    cache = ops.CacheC(16, 16, 16, 16, 16, -3)
    assert L.pbsa_score_topk(d, ctypes.c_void_p(16), ctypes.byref(cache), ctypes.c_void_p(16),
                             ctypes.c_void_p(16), None) == 6
    # workspace too small for the memory update
    cache = ops.CacheC(16, 16, 16, 16, 16, 0)
    st = L.pbsa_memory_update(d, ctypes.c_void_p(16), ctypes.byref(cache), _tensor(16),
                              _tensor(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 8, None)
    assert st == 5 and b"10240" in L.pbsa_last_error()
    assert cache.chunk_index == 0
    # its two halves check the same workspace; a failed apply leaves chunk_index alone
    assert L.pbsa_memory_select(d, ctypes.c_void_p(16), ctypes.byref(cache), ctypes.c_void_p(16),
                                8, None) == 5
    assert L.pbsa_memory_apply(d, ctypes.byref(cache), _tensor(16), _tensor(16),
                               ctypes.c_void_p(16), ctypes.c_void_p(16), 8, None) == 5
    assert cache.chunk_index == 0
    # two-level: budget above max_sel, too many chunks
    ks = (ctypes.c_int32 * 8)(0, 8, 12, 16, 20, 24, 28, 80)
    assert L.pbsa_score_topk_2lvl(d, 8, 8, ks, *(ctypes.c_void_p(16),) * 3, 75,
                                  ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 2
    assert L.pbsa_score_topk_2lvl(d, 300, 8, ks, *(ctypes.c_void_p(16),) * 3, 75,
                                  ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 2
    # max_sel below one chunk's blocks
    ks = (ctypes.c_int32 * 8)(0, 8, 12, 16, 20, 24, 28, 32)
    assert L.pbsa_score_topk_2lvl(d, 8, 8, ks, *(ctypes.c_void_p(16),) * 3, 70,
                                  ctypes.c_void_p(16), ctypes.c_void_p(16), None) == 2
    # attention lists beyond the per-workgroup cap: C + chunk blocks + 2*topk > 3072
    big = _dims(capacity=1000, sinks=1, topk=1000, window_frames=40)
    t = _tensor(16)
    assert L.pbsa_attn_fwd(big, t, ctypes.byref(ops.CacheC(16, 16, 16, 16, 16, 0)), t, t,
                           ctypes.c_void_p(16), t, ctypes.c_void_p(16), None) == 3
    assert b"3072" in L.pbsa_last_error()
    # two-level attention: max_sel above 1536
    assert L.pbsa_attn_fwd_2lvl(d, 8, t, t, t, ctypes.c_void_p(16), ctypes.c_void_p(16), 1537,
                                t, ctypes.c_void_p(16), None) == 3
    # backward without workspace
    t = _tensor(16)
    assert L.pbsa_attn_bwd(d, 8, t, t, t, t, ctypes.c_void_p(16), t, ctypes.c_void_p(16),
                           ctypes.c_void_p(16), 75, t, t, t, None, 0, None) == 5
    # backward: max_sel above 1536
    assert L.pbsa_attn_bwd(d, 8, t, t, t, t, ctypes.c_void_p(16), t, ctypes.c_void_p(16),
                           ctypes.c_void_p(16), 1537, t, t, t, None, 0, None) == 3
    assert b"1536" in L.pbsa_last_error()
    # backward: a token stride above 2^24 elements (32-bit row offsets inside a block)
    wide = _tensor(16, ts=(1 << 24) + 8)
    short = ctypes.byref(_dims(frame_tokens=16, chunk_frames=1))  # 16 tokens: span < 2 GiB
    assert L.pbsa_attn_bwd(short, 1, wide, t, t, t, ctypes.c_void_p(16), t,
                           ctypes.c_void_p(16), ctypes.c_void_p(16), 1, t, t, t, None, 0,
                           None) == 3
    assert b"stride" in L.pbsa_last_error()


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(3 * 1560, 12, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ops.pbsa_pool(WAN, x, 3, torch.zeros(12, 75, 128))
    with pytest.raises(TypeError):
        ops.pbsa_pool(WAN, x.float(), 3, torch.zeros(12, 75, 128))


def test_host_budget_matches_oracle_budget():
    import numpy as np
    import oracle
    rs = np.random.default_rng(4)
    for _ in range(50):
        a = rs.uniform(0, 1, size=8)
        assert runtime.cag_budgets(a, 32, 8)[1:] == oracle.cag_budgets(a, 32, 8)[1:]


def test_chunk_step_checks_before_launching():
    L = ops.lib()
    d = ctypes.byref(_dims())
    cache = ops.CacheC(16, 16, 16, 16, 16, 0, None)
    a = ops.ChunkArgs()
    for p in range(ops.MAX_PASSES):
        a.q[p] = a.k[p] = a.v[p] = a.o[p] = _tensor(16)
        a.lse[p] = 16
    a.scores, a.sel, a.workspace = 16, 16, 16
    a.workspace_bytes = ops.pbsa_workspace_bytes(WAN, ops.PBSA_OP_MEMORY_UPDATE)
    for bad in (0, ops.MAX_PASSES + 1):
        a.passes = bad
        assert L.pbsa_chunk_step(d, ctypes.byref(a), ctypes.byref(cache), None) == 2
    a.passes = 2
    a.lse[1] = None
    assert L.pbsa_chunk_step(d, ctypes.byref(a), ctypes.byref(cache), None) == 1
    a.lse[1] = 16
    a.workspace_bytes = 8
    assert L.pbsa_chunk_step(d, ctypes.byref(a), ctypes.byref(cache), None) == 5
    a.workspace_bytes = 1 << 20
    # a captured step needs the device chunk counter; a misaligned one is refused
    h = ctypes.c_void_p()
    assert L.pbsa_chunk_graph_create(d, ctypes.byref(a), ctypes.byref(cache), ctypes.byref(h)) == 6
    assert not h.value
    cache = ops.CacheC(16, 16, 16, 16, 16, 0, 12)
    assert L.pbsa_chunk_graph_create(d, ctypes.byref(a), ctypes.byref(cache), ctypes.byref(h)) == 4
    assert L.pbsa_chunk_graph_launch(None, ctypes.byref(cache), None) == 1
