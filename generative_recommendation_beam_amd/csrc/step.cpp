// Multi-layer decode step captured into one HIP graph: the optional beam
// selection, then per layer the Non-Shared append and the fused decode,
// exactly as the eager entry points enqueue them (they are called on a
// capture stream). Nothing in either path
// records a memset, so the graph replays cleanly; the split-merge counters in
// each layer's workspace return to zero at the end of every launch.
#include <hip/hip_runtime.h>

#include <new>

#include "xattn.h"

struct xattn_step_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

xattn_status capture_step(const xattn_beam_select* sel, const xattn_layer_step* layers, int n,
                          hipStream_t cs) {
  if (sel) {
    const xattn_status e = xattn_beam_topk(sel->num_requests, sel->beam_width, sel->top_k, sel->n_out,
                                           sel->beam_score, sel->logprob, sel->token, sel->parent,
                                           sel->token_out, sel->score_out, cs);
    if (e != XATTN_OK) return e;
  }
  for (int i = 0; i < n; ++i) {
    const xattn_layer_step& l = layers[i];
    xattn_status e;
    if (l.k_new != nullptr && l.table_in != l.table_out && l.decode_begin == nullptr) {
      // Ping-pong tables: the append folds into the decode launch when the plan allows.
      e = xattn_append_decode(&l.dims, l.q, l.k_shared, l.v_shared, l.prefix_off, l.prefix_len, l.k_new,
                              l.v_new, l.parent, l.slot_base, l.active, l.k_pool, l.v_pool, l.table_in,
                              l.table_out, l.unshared_len, l.o, l.lse, l.workspace, l.workspace_bytes, cs);
      if (e != XATTN_OK) return e;
    } else {
      if (l.k_new != nullptr) {
        e = xattn_cache_append(&l.dims, l.k_new, l.v_new, l.parent, l.slot_base, l.active, l.k_pool,
                               l.v_pool, l.table_in, l.table_out, l.unshared_len, cs);
        if (e != XATTN_OK) return e;
      }
      if (l.decode_begin && hipEventRecordWithFlags(static_cast<hipEvent_t>(l.decode_begin), cs,
                                                    hipEventRecordExternal) != hipSuccess)
        return XATTN_ERR_HIP;
      e = xattn_decode(&l.dims, l.q, l.k_shared, l.v_shared, l.prefix_off, l.prefix_len, l.k_pool,
                       l.v_pool, l.table_out, l.unshared_len, l.o, l.lse, l.workspace,
                       l.workspace_bytes, cs);
      if (e != XATTN_OK) return e;
    }
    if (l.decode_end && hipEventRecordWithFlags(static_cast<hipEvent_t>(l.decode_end), cs,
                                                hipEventRecordExternal) != hipSuccess)
      return XATTN_ERR_HIP;
  }
  return XATTN_OK;
}

}  // namespace

extern "C" {

xattn_status xattn_step_graph_create(const xattn_beam_select* select,
                                     const xattn_layer_step* layers, int32_t n_layers,
                                     xattn_step_graph** out) {
  if (!out) return XATTN_ERR_INVALID_ARG;
  *out = nullptr;
  if (n_layers < 0 || (n_layers > 0 && !layers) || (n_layers == 0 && !select))
    return XATTN_ERR_INVALID_ARG;
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return XATTN_ERR_HIP;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    hipStreamDestroy(cs);
    return XATTN_ERR_HIP;
  }
  const xattn_status e = capture_step(select, layers, n_layers, cs);
  hipGraph_t graph = nullptr;
  const hipError_t ce = hipStreamEndCapture(cs, &graph);
  hipStreamDestroy(cs);
  if (e != XATTN_OK || ce != hipSuccess || graph == nullptr) {
    if (graph) hipGraphDestroy(graph);
    return e != XATTN_OK ? e : XATTN_ERR_HIP;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    hipGraphDestroy(graph);
    return XATTN_ERR_HIP;
  }
  xattn_step_graph* g = new (std::nothrow) xattn_step_graph{graph, exec};
  if (!g) {
    hipGraphExecDestroy(exec);
    hipGraphDestroy(graph);
    return XATTN_ERR_HIP;
  }
  *out = g;
  return XATTN_OK;
}

xattn_status xattn_step_graph_launch(xattn_step_graph* g, void* stream) {
  if (!g) return XATTN_ERR_INVALID_ARG;
  return hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) == hipSuccess ? XATTN_OK
                                                                                   : XATTN_ERR_HIP;
}

xattn_status xattn_step_graph_destroy(xattn_step_graph* g) {
  if (!g) return XATTN_OK;
  const hipError_t a = hipGraphExecDestroy(g->exec);
  const hipError_t b = hipGraphDestroy(g->graph);
  delete g;
  return (a == hipSuccess && b == hipSuccess) ? XATTN_OK : XATTN_ERR_HIP;
}

}  // extern "C"
