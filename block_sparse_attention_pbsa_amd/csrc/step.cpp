// The per-chunk step of the persistent mode as one call, and as one captured HIP graph.
//
// Sparse Forcing (gist.science), 2.B: the persistent memory and the window are kept across
// the denoising passes of a chunk and updated once per chunk (the Chinese page's 2.1: the
// memory is shared between diffusion steps).  A chunk of T passes is therefore
//   for each pass p:  route(q_p)  ->  attention(q_p, k_p, v_p)
//   then:             memory update with the last pass's scores, its K/V entering the cache.
// The graph form overlaps the update's selection (which only reads the cache and the last
// pass's scores) with the last pass's attention on a second captured stream, and takes the
// chunk index from the cache's device counter, so that one capture serves every later
// chunk whose inputs are written into the same buffers.
#include <hip/hip_runtime.h>

#include <new>

#include "../../include/pbsa.h"
#include "launch.h"
#include "step_internal.h"

namespace pbsa {

hipError_t enqueue_chunk_step(const pbsa_dims& d, const pbsa_chunk_args& a, const pbsa_cache& c,
                              hipStream_t s, hipStream_t side, hipEvent_t fork, hipEvent_t join) {
  hipError_t e = hipSuccess;
  const int T = a.passes;
  for (int p = 0; p < T; ++p) {
    e = launch_route(d, tok_in(a.q[p]), a.q_rep, c, a.scores, a.sel, s);
    if (e != hipSuccess) return e;
    if (p == T - 1 && side) {
      // the selection reads the last pass's scores and the cache, beside the attention
      if ((e = hipEventRecord(fork, s)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess) return e;
      if ((e = launch_memory_select(d, a.scores, c, a.workspace, true, side)) != hipSuccess)
        return e;
      if ((e = hipEventRecord(join, side)) != hipSuccess) return e;
    }
    e = a.fp8_arithmetic
            ? launch_attn_fwd_f8(d, tok_in(a.q[p]), c, tok_in(a.k[p]), tok_in(a.v[p]), a.sel,
                                 tok_out(a.o[p]), a.lse[p], a.attn_workspace, s)
        : d.kv_format == PBSA_KV_FP8
            ? launch_attn_fwd_fp8(d, tok_in(a.q[p]), c, tok_in(a.k[p]), tok_in(a.v[p]), a.sel,
                                  tok_out(a.o[p]), a.lse[p], s)
            : launch_attn_fwd_persistent(d, tok_in(a.q[p]), c, tok_in(a.k[p]), tok_in(a.v[p]),
                                         a.sel, tok_out(a.o[p]), a.lse[p], s);
    if (e != hipSuccess) return e;
  }
  if (side) {
    if ((e = hipStreamWaitEvent(s, join, 0)) != hipSuccess) return e;
  } else {
    e = launch_memory_select(d, a.scores, c, a.workspace, false, s);
    if (e != hipSuccess) return e;
  }
  return launch_memory_apply(d, c, tok_in(a.k[T - 1]), tok_in(a.v[T - 1]), nullptr, a.workspace,
                             s);
}

}  // namespace pbsa

struct pbsa_chunk_graph {
  pbsa_dims dims;
  pbsa_cache cache;  // the buffers the graph was captured on
  hipStream_t cap = nullptr, side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

void release(pbsa_chunk_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->fork) (void)hipEventDestroy(g->fork);
  if (g->join) (void)hipEventDestroy(g->join);
  if (g->side) (void)hipStreamDestroy(g->side);
  if (g->cap) (void)hipStreamDestroy(g->cap);
  delete g;
}

}  // namespace

extern "C" {

pbsa_status pbsa_chunk_step(const pbsa_dims* dims, const pbsa_chunk_args* args,
                            pbsa_cache* cache, void* stream) {
  PBSA_TRY(pbsa::api::check_chunk_args(dims, args, cache));
  const pbsa_status st = pbsa::api::hip_status(
      pbsa::enqueue_chunk_step(*dims, *args, *cache, static_cast<hipStream_t>(stream), nullptr,
                               nullptr, nullptr),
      "chunk_step");
  if (st == PBSA_OK) cache->chunk_index += 1;
  return st;
}

pbsa_status pbsa_chunk_graph_create(const pbsa_dims* dims, const pbsa_chunk_args* args,
                                    const pbsa_cache* cache, pbsa_chunk_graph** out) {
  if (!out) return pbsa::api::fail(PBSA_ERR_NULL, "out is NULL");
  *out = nullptr;
  PBSA_TRY(pbsa::api::check_chunk_args(dims, args, cache));
  if (!cache->chunk_index_dev)
    return pbsa::api::fail(PBSA_ERR_STATE,
                           "a captured chunk step needs the cache's device chunk counter "
                           "(chunk_index_dev)");
  pbsa_chunk_graph* g = new (std::nothrow) pbsa_chunk_graph;
  if (!g) return pbsa::api::fail(PBSA_ERR_HIP, "chunk_graph_create: out of host memory");
  g->dims = *dims;
  g->cache = *cache;
  hipError_t e = hipStreamCreateWithFlags(&g->cap, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&g->side, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&g->fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&g->join, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamBeginCapture(g->cap, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    const hipError_t le =
        pbsa::enqueue_chunk_step(*dims, *args, *cache, g->cap, g->side, g->fork, g->join);
    e = hipStreamEndCapture(g->cap, &g->graph);
    if (le != hipSuccess) e = le;
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    release(g);
    return pbsa::api::hip_status(e, "chunk_graph_create");
  }
  *out = g;
  return PBSA_OK;
}

pbsa_status pbsa_chunk_graph_launch(pbsa_chunk_graph* graph, pbsa_cache* cache, void* stream) {
  if (!graph || !cache) return pbsa::api::fail(PBSA_ERR_NULL, "graph and cache are required");
  const pbsa_cache& c = graph->cache;
  if (cache->k != c.k || cache->v != c.v || cache->rep != c.rep ||
      cache->block_id != c.block_id || cache->len != c.len ||
      cache->chunk_index_dev != c.chunk_index_dev)
    return pbsa::api::fail(PBSA_ERR_STATE, "the graph was captured on another cache");
  const pbsa_status st = pbsa::api::hip_status(
      hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream)), "chunk_graph_launch");
  if (st == PBSA_OK) cache->chunk_index += 1;
  return st;
}

void pbsa_chunk_graph_destroy(pbsa_chunk_graph* graph) { release(graph); }

}  // extern "C"
