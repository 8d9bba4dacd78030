// Graph-captured decode steps (MinivLLM guide "vLLM 技术路线", Step 4 §4.7:
// decode runs are captured once per batch-size bucket [1, 2, 4, 8] + multiples
// of 16 up to the largest batch, into static input tensors; a step copies its
// inputs into the first rows, pads the remaining rows with sentinel values and
// replays the smallest bucket that fits; §4.5: the per-step index tensors are
// built on the host in pinned memory and uploaded with non-blocking copies).
//
// One object captures the fused store + decode call (pa_paged_decode_append,
// or its FP8 form) for every bucket.  The object owns the static device
// buffers the graphs read (q, the new K/V rows, slot mapping, context lengths,
// block tables, output, split-K workspace) and a ring of pinned host staging
// areas for the index tensors; before a staging area is refilled the host
// waits for the event recorded after its last upload, so a step never
// overwrites index data the GPU has not copied yet.  The graph of bucket b
// reads its index tensors packed as [slots b | lengths b | tables b x MBS], so
// a step uploads them with one copy.  Padded rows get slot -1 (nothing
// stored) and context length 0 (output row zero, no K/V read).
#include <hip/hip_runtime.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/pagedattn.h"

struct pa_decode_graph {
  int device = 0;
  int max_batch = 0, num_q_heads = 0, num_kv_heads = 0, head_dim = 0, block_size = 0;
  int num_blocks = 0, max_blocks_per_seq = 0, kv_fp8 = 0, out_dtype = 0;
  float scale = 0.f, k_scale = 1.f, v_scale = 1.f;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  // static device buffers read by the graphs
  void* q = nullptr;
  void* k_new = nullptr;
  void* v_new = nullptr;
  void* out = nullptr;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  int32_t* meta = nullptr;  // bucket b: [slots b | lens b | tables b * MBS]
  // pinned staging, same packing, used in turn
  static constexpr int kStaging = 4;
  int32_t* staging[kStaging] = {};
  hipEvent_t uploaded[kStaging] = {};
  int next = 0;
  std::vector<int> buckets;
  std::vector<hipGraph_t> graphs;
  std::vector<hipGraphExec_t> execs;
};

namespace {

size_t meta_ints(const pa_decode_graph* g) {
  return (size_t)g->max_batch * (2 + (size_t)g->max_blocks_per_seq);
}

void release(pa_decode_graph* g) {
  if (!g) return;
  for (hipGraphExec_t e : g->execs)
    if (e) (void)hipGraphExecDestroy(e);
  for (hipGraph_t gr : g->graphs)
    if (gr) (void)hipGraphDestroy(gr);
  for (int i = 0; i < pa_decode_graph::kStaging; ++i) {
    if (g->uploaded[i]) (void)hipEventDestroy(g->uploaded[i]);
    if (g->staging[i]) (void)hipHostFree(g->staging[i]);
  }
  void* bufs[] = {g->q, g->k_new, g->v_new, g->out, g->workspace, g->meta};
  for (void* p : bufs)
    if (p) (void)hipFree(p);
  delete g;
}

// Pack B rows of caller data, padded to `rows`, as [slots | lens | tables].
void stage(const pa_decode_graph* g, int32_t* h, int B, int rows, const int32_t* slots,
           const int32_t* tables, int tables_stride, const int32_t* lens) {
  const int M = g->max_blocks_per_seq;
  int32_t* hs = h;
  int32_t* hl = h + rows;
  int32_t* ht = h + 2 * (size_t)rows;
  for (int i = 0; i < rows; ++i) {
    hs[i] = i < B ? slots[i] : -1;
    hl[i] = i < B ? lens[i] : 0;
    int32_t* row = ht + (size_t)i * M;
    if (i < B) {
      memcpy(row, tables + (size_t)i * tables_stride, sizeof(int32_t) * (size_t)tables_stride);
      for (int j = tables_stride; j < M; ++j) row[j] = -1;
    } else {
      for (int j = 0; j < M; ++j) row[j] = -1;
    }
  }
}

size_t packed_ints(const pa_decode_graph* g, int rows) {
  return (size_t)rows * (2 + (size_t)g->max_blocks_per_seq);
}

// One fused store + decode call over the first `rows` static rows.
int launch_step(pa_decode_graph* g, int rows, hipStream_t stream) {
  int32_t* slots = g->meta;
  int32_t* lens = g->meta + rows;
  int32_t* tables = g->meta + 2 * (size_t)rows;
  if (g->kv_fp8)
    return pa_paged_decode_append_fp8(
        g->q, g->k_new, g->v_new, slots, g->k_cache, g->v_cache, tables, g->max_blocks_per_seq,
        lens, rows, g->num_q_heads, g->num_kv_heads, g->head_dim, g->block_size, g->num_blocks,
        g->scale, g->k_scale, g->v_scale, g->out, g->out_dtype, g->workspace,
        g->workspace_bytes, stream);
  return pa_paged_decode_append(g->q, g->k_new, g->v_new, slots, g->k_cache, g->v_cache, tables,
                                g->max_blocks_per_seq, lens, rows, g->num_q_heads,
                                g->num_kv_heads, g->head_dim, g->block_size, g->num_blocks,
                                g->scale, g->out, g->out_dtype, g->workspace, g->workspace_bytes,
                                stream);
}

}  // namespace

extern "C" {

int pa_decode_graph_create(int max_batch, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_blocks_per_seq, int kv_fp8,
                           float scale, float k_scale, float v_scale, void* k_cache,
                           void* v_cache, int out_dtype, pa_decode_graph** out_graph) {
  if (!out_graph) return PA_ERR_NULL;
  *out_graph = nullptr;
  if (max_batch <= 0 || max_batch > 65536 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (!k_cache || !v_cache) return PA_ERR_NULL;
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  const size_t ws = kv_fp8 ? pa_paged_decode_fp8_workspace_bytes(max_batch, num_q_heads,
                                                                  num_kv_heads, head_dim,
                                                                  block_size, max_blocks_per_seq)
                           : pa_paged_decode_workspace_bytes(max_batch, num_q_heads,
                                                             num_kv_heads, head_dim, block_size,
                                                             max_blocks_per_seq);
  if (ws == 0) return PA_ERR_SHAPE;

  pa_decode_graph* g = new (std::nothrow) pa_decode_graph();
  if (!g) return PA_ERR_HIP;
  g->max_batch = max_batch;
  g->num_q_heads = num_q_heads;
  g->num_kv_heads = num_kv_heads;
  g->head_dim = head_dim;
  g->block_size = block_size;
  g->num_blocks = num_blocks;
  g->max_blocks_per_seq = max_blocks_per_seq;
  g->kv_fp8 = kv_fp8 ? 1 : 0;
  g->out_dtype = out_dtype;
  g->scale = scale;
  g->k_scale = k_scale;
  g->v_scale = v_scale;
  g->k_cache = k_cache;
  g->v_cache = v_cache;
  g->workspace_bytes = ws;

  const size_t qb = (size_t)max_batch * num_q_heads * head_dim * 2;
  const size_t kvb = (size_t)max_batch * num_kv_heads * head_dim * 2;
  const size_t ob = (size_t)max_batch * num_q_heads * head_dim * (out_dtype == PA_F32 ? 4 : 2);
  const size_t metab = sizeof(int32_t) * meta_ints(g);
  hipStream_t cap = nullptr;
  int rc = PA_ERR_HIP;
  bool ok = hipGetDevice(&g->device) == hipSuccess && hipMalloc(&g->q, qb) == hipSuccess &&
            hipMalloc(&g->k_new, kvb) == hipSuccess && hipMalloc(&g->v_new, kvb) == hipSuccess &&
            hipMalloc(&g->out, ob) == hipSuccess && hipMalloc(&g->workspace, ws) == hipSuccess &&
            hipMalloc((void**)&g->meta, metab) == hipSuccess;
  for (int i = 0; ok && i < pa_decode_graph::kStaging; ++i)
    ok = hipHostMalloc((void**)&g->staging[i], metab, hipHostMallocDefault) == hipSuccess &&
         // the host only needs the copy out of this staging area to have run, not
         // device memory made visible to it: no system-scope fence at the record
         // (which would write back and invalidate L2 and stall the stream ~5 us)
         hipEventCreateWithFlags(&g->uploaded[i],
                                 hipEventDisableTiming | hipEventDisableSystemFence) == hipSuccess;
  // Zero inputs and sentinel index rows (for the largest packing; a smaller
  // bucket's packing is rewritten by every step that uses it).
  if (ok) {
    stage(g, g->staging[0], 0, max_batch, nullptr, nullptr, 0, nullptr);
    ok = hipMemcpy(g->meta, g->staging[0], metab, hipMemcpyHostToDevice) == hipSuccess &&
         hipMemset(g->q, 0, qb) == hipSuccess && hipMemset(g->k_new, 0, kvb) == hipSuccess &&
         hipMemset(g->v_new, 0, kvb) == hipSuccess && hipMemset(g->workspace, 0, ws) == hipSuccess &&
         hipDeviceSynchronize() == hipSuccess;
  }
  if (ok) {
    for (int b : {1, 2, 4, 8})
      if (b < max_batch) g->buckets.push_back(b);
    for (int b = 16; b < max_batch; b += 16) g->buckets.push_back(b);
    g->buckets.push_back(max_batch);
    ok = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) == hipSuccess;
  }
  for (size_t i = 0; ok && i < g->buckets.size(); ++i) {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    ok = hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal) == hipSuccess;
    if (!ok) break;
    const int lrc = launch_step(g, g->buckets[i], cap);
    const hipError_t ee = hipStreamEndCapture(cap, &graph);
    if (lrc != PA_OK) {
      rc = lrc;
      ok = false;
    } else {
      ok = ee == hipSuccess && graph &&
           hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess;
    }
    g->graphs.push_back(graph);
    g->execs.push_back(exec);
  }
  if (cap) (void)hipStreamDestroy(cap);
  if (!ok) {
    release(g);
    return rc;
  }
  *out_graph = g;
  return PA_OK;
}

int pa_decode_graph_buffers(const pa_decode_graph* g, void** q, void** k_new, void** v_new,
                            void** out) {
  if (!g) return PA_ERR_NULL;
  if (q) *q = g->q;
  if (k_new) *k_new = g->k_new;
  if (v_new) *v_new = g->v_new;
  if (out) *out = g->out;
  return PA_OK;
}

int pa_decode_graph_bucket(const pa_decode_graph* g, int batch) {
  if (!g || batch <= 0 || batch > g->max_batch) return 0;
  for (int b : g->buckets)
    if (b >= batch) return b;
  return 0;
}

int pa_decode_graph_run(pa_decode_graph* g, int batch, const void* q, const void* k_new,
                        const void* v_new, const int32_t* slot_mapping,
                        const int32_t* block_tables, int tables_stride,
                        const int32_t* context_lens, void* out, void* stream) {
  if (!g) return PA_ERR_NULL;
  if (batch < 0 || batch > g->max_batch) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!slot_mapping || !block_tables || !context_lens) return PA_ERR_NULL;
  if (tables_stride <= 0 || tables_stride > g->max_blocks_per_seq) return PA_ERR_SHAPE;
  const int rows = pa_decode_graph_bucket(g, batch);
  size_t k = 0;
  while (g->buckets[k] != rows) ++k;
  hipStream_t s = (hipStream_t)stream;
  int cur_dev = 0;
  if (hipGetDevice(&cur_dev) != hipSuccess || cur_dev != g->device) return PA_ERR_UNSUPPORTED;

  const int slot = g->next;
  if (hipEventSynchronize(g->uploaded[slot]) != hipSuccess) return PA_ERR_HIP;
  stage(g, g->staging[slot], batch, rows, slot_mapping, block_tables, tables_stride,
        context_lens);
  if (hipMemcpyAsync(g->meta, g->staging[slot], sizeof(int32_t) * packed_ints(g, rows),
                     hipMemcpyHostToDevice, s) != hipSuccess)
    return PA_ERR_HIP;
  if (hipEventRecord(g->uploaded[slot], s) != hipSuccess) return PA_ERR_HIP;
  g->next = (slot + 1) % pa_decode_graph::kStaging;

  const size_t qb = (size_t)batch * g->num_q_heads * g->head_dim * 2;
  const size_t kvb = (size_t)batch * g->num_kv_heads * g->head_dim * 2;
  if (q && q != g->q && hipMemcpyAsync(g->q, q, qb, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return PA_ERR_HIP;
  if (k_new && k_new != g->k_new &&
      hipMemcpyAsync(g->k_new, k_new, kvb, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return PA_ERR_HIP;
  if (v_new && v_new != g->v_new &&
      hipMemcpyAsync(g->v_new, v_new, kvb, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return PA_ERR_HIP;
  if (hipGraphLaunch(g->execs[k], s) != hipSuccess) return PA_ERR_HIP;
  if (out && out != g->out) {
    const size_t ob = (size_t)batch * g->num_q_heads * g->head_dim *
                      (g->out_dtype == PA_F32 ? 4 : 2);
    if (hipMemcpyAsync(out, g->out, ob, hipMemcpyDeviceToDevice, s) != hipSuccess)
      return PA_ERR_HIP;
  }
  return PA_OK;
}

int pa_decode_graph_destroy(pa_decode_graph* g) {
  if (!g) return PA_OK;
  int cur_dev = 0;
  const bool same = hipGetDevice(&cur_dev) == hipSuccess && cur_dev == g->device;
  if (same) {
    for (int i = 0; i < pa_decode_graph::kStaging; ++i) (void)hipEventSynchronize(g->uploaded[i]);
    (void)hipDeviceSynchronize();
  }
  release(g);
  return PA_OK;
}

}  // extern "C"
