// C ABI of libpagedattn: argument checks, launch geometry, status codes.
// The operations and their conventions are documented in include/pagedattn.h.
#include "../../include/pagedattn.h"

#include <math.h>

#include <mutex>

#include "kernels.h"

namespace {

bool pow2_log2(int x, int* lg) {
  if (x <= 0 || (x & (x - 1)) != 0) return false;
  int l = 0;
  while ((1 << l) < x) ++l;
  *lg = l;
  return true;
}

// Head dim and block size support shared by every call.
int check_geometry(int num_kv_heads, int head_dim, int block_size, int num_blocks, int* bs_log2) {
  if (num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!pow2_log2(block_size, bs_log2) || block_size > 1024) return PA_ERR_UNSUPPORTED;
  // Every flat slot index and every element offset inside one pool must fit.
  const int64_t slots = (int64_t)num_blocks * block_size;
  if (slots > INT32_MAX) return PA_ERR_SHAPE;
  return PA_OK;
}

float resolve_scale(float scale, int head_dim) {
  return (scale > 0.f && isfinite(scale)) ? scale : (float)(1.0 / sqrt((double)head_dim));
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: invalid or inconsistent size";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim, block_size or dtype not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: decode workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: kernel launch or HIP call failed";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS: not enough free KV blocks";
    case PA_ERR_SEQUENCE: return "PA_ERR_SEQUENCE: unknown or already allocated sequence";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the decode needs more than the library's fixed scratch buffer "
             "(PA_DECODE_SCRATCH_BYTES); pass a workspace to pa_paged_decode_append instead";
    default: return "unknown pa_status";
  }
}

int pa_kvcache_store(const void* k, const void* v, const int32_t* slot_mapping, int T,
                     void* k_cache, void* v_cache, int num_blocks, int block_size,
                     int num_kv_heads, int head_dim, void* stream) {
  if (T < 0) return PA_ERR_SHAPE;
  int bs_log2 = 0;
  const int g = check_geometry(num_kv_heads, head_dim, block_size, num_blocks, &bs_log2);
  if (g != PA_OK) return g;
  if (T == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  if ((int64_t)T * num_kv_heads * head_dim / 8 > INT32_MAX) return PA_ERR_SHAPE;
  return pa::launch_kvcache_store(k, v, slot_mapping, T, k_cache, v_cache, num_blocks, block_size,
                                  num_kv_heads, head_dim, (hipStream_t)stream) == 0
             ? PA_OK
             : PA_ERR_HIP;
}

}  // extern "C"

namespace {

// Workspace of a decode call with num_seqs sequences: the most any batch of
// 1 .. num_seqs sequences needs, so one workspace serves every smaller batch.
// A plan's own size grows with the batch except where longer splits switch
// on (VALU long splits: half the partial slots per sequence; MFMA long
// splits: an eighth); that happens once, at a threshold batch, so the maximum
// is the larger of the plan at num_seqs and the plan just below the
// threshold.
size_t decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int block_size, int max_blocks_per_seq, bool kv8) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const pa::DecodePlan p = pa::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           block_size, max_blocks_per_seq, kv8);
  if (p.units > pa::kDecodeMaxUnits || p.nsplit_short > pa::kDecodeMaxSplits) return 0;
  size_t bytes = p.workspace_bytes();
  if (p.coarse()) {
    // largest batch below num_seqs whose plan keeps short splits
    int lo = 1, hi = num_seqs - 1, below = 0;
    while (lo <= hi) {
      const int mid = lo + (hi - lo) / 2;
      if (pa::plan_decode(mid, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, kv8).coarse()) {
        hi = mid - 1;
      } else {
        below = mid;
        lo = mid + 1;
      }
    }
    if (below > 0) {
      const size_t b = pa::plan_decode(below, num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_blocks_per_seq, kv8).workspace_bytes();
      if (b > bytes) bytes = b;
    }
  }
  return bytes;
}



// The new tokens of a fused store + decode call (all NULL for plain decode).
struct NewTokens {
  const void* k;
  const void* v;
  const int32_t* slot_mapping;
};

// Shared body of the decode entry points (bf16 or FP8 pools, with or without
// the fused store).  For FP8 the K scale is folded into the score scale and
// the V scale multiplies the outputs.
int decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
           int max_blocks_per_seq, const int32_t* context_lens, int num_seqs, int num_q_heads,
           int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
           bool kv8, float k_scale, float v_scale, void* out, int out_dtype, void* workspace,
           size_t workspace_bytes, void* stream, const NewTokens* append = nullptr) {
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  int bs_log2 = 0;
  const int g = check_geometry(num_kv_heads, head_dim, block_size, num_blocks, &bs_log2);
  if (g != PA_OK) return g;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if (kv8 && !(k_scale > 0.f && isfinite(k_scale) && v_scale > 0.f && isfinite(v_scale)))
    return PA_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_ERR_NULL;
  if (append && (!append->k || !append->v || !append->slot_mapping)) return PA_ERR_NULL;
  const pa::DecodePlan p = pa::plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           block_size, max_blocks_per_seq, kv8);
  if (!workspace || ((uintptr_t)workspace & 7) != 0) return PA_ERR_WORKSPACE;
  if (workspace_bytes < p.workspace_bytes()) return PA_ERR_WORKSPACE;
  const int64_t hg = (int64_t)num_kv_heads * p.nsub;
  if ((int64_t)num_seqs * hg * p.nsplit_max > INT32_MAX) return PA_ERR_SHAPE;
  if (p.units > pa::kDecodeMaxUnits) return PA_ERR_SHAPE;
  if (p.nsplit_short > pa::kDecodeMaxSplits) return PA_ERR_UNSUPPORTED;

  pa::DecodeArgs a{};
  a.q = (const uint16_t*)q;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  char* ws = (char*)workspace;
  a.ws_ml = (float*)ws;
  a.ws_o = (float*)(ws + p.ml_bytes);
  a.mbs = max_blocks_per_seq;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.group = p.group;
  a.nsub = p.nsub;
  a.hg = (int)hg;
  a.bs_log2 = bs_log2;
  a.split_log2 = p.split_log2;
  a.nsplit_max = p.nsplit_max;
  a.long_splits = p.long_splits;
  a.long_above = p.long_above;
  a.batch = num_seqs;
  a.compact = p.compact;
  a.num_blocks = num_blocks;
  a.out_f32 = out_dtype == PA_F32;
  const float sc = resolve_scale(scale, head_dim);
  a.scale_log2e = (kv8 ? sc * k_scale : sc) * pa::kLog2eHost;
  a.v_scale = kv8 ? v_scale : 1.f;
  if (append) {
    a.k_new = (const uint16_t*)append->k;
    a.v_new = (const uint16_t*)append->v;
    a.slot_mapping = append->slot_mapping;
    a.k_cache_w = (void*)k_cache;
    a.v_cache_w = (void*)v_cache;
    a.num_slots = (int64_t)num_blocks * block_size;
    a.qscale_k = k_scale;
    a.qscale_v = v_scale;
  }
  return pa::launch_paged_decode(a, num_seqs, head_dim, p.gt, kv8, append != nullptr, p.mfma,
                                 (hipStream_t)stream) == 0
             ? PA_OK
             : PA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t pa_paged_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int max_blocks_per_seq) {
  return decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, false);
}

size_t pa_paged_decode_fp8_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                           int head_dim, int block_size,
                                           int max_blocks_per_seq) {
  return decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                max_blocks_per_seq, true);
}

int pa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, int num_seqs, int num_q_heads,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                    void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, false, 1.f,
                1.f, out, out_dtype, workspace, workspace_bytes, stream);
}

int pa_paged_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int block_size, int num_blocks,
                        float scale, float k_scale, float v_scale, void* out, int out_dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, true, k_scale,
                v_scale, out, out_dtype, workspace, workspace_bytes, stream);
}

int pa_paged_decode_append(const void* q, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, void* k_cache, void* v_cache,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           float scale, void* out, int out_dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  return decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, false, 1.f,
                1.f, out, out_dtype, workspace, workspace_bytes, stream, &nt);
}

}  // extern "C"

namespace {

// Split-K scratch of pa_paged_decode_append_noalloc: one array per GPU the
// library runs on (a device variable has one instance per device), held until
// the process ends.  Host code never uses the name `scratch` as an address:
// each device's address comes from hipGetSymbolAddress, taken once with that
// device current.
constexpr int kMaxScratchDevices = 64;
__device__ __align__(256) char scratch[PA_DECODE_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxScratchDevices] = {};
std::mutex g_scratch_mutex;

// The current device's scratch address, or NULL if it cannot be found.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int pa_paged_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                   const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int num_blocks, float scale, void* out, int out_dtype,
                                   void* stream) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  if (num_seqs > 0) {
    const size_t need = pa_paged_decode_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq);
    if (need > PA_DECODE_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  }
  // Argument errors first, with no device call: without a workspace the
  // checks report PA_ERR_WORKSPACE exactly when everything else is valid.
  const int rc = decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                        scale, false, 1.f, 1.f, out, out_dtype, nullptr, 0, stream, &nt);
  if (rc != PA_ERR_WORKSPACE) return rc;
  void* ws = device_scratch();
  if (!ws) return PA_ERR_HIP;
  return decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, false, 1.f,
                1.f, out, out_dtype, ws, PA_DECODE_SCRATCH_BYTES, stream, &nt);
}

int pa_paged_decode_append_fp8(const void* q, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, void* k_cache, void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               float scale, float k_scale, float v_scale, void* out,
                               int out_dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  const NewTokens nt{k_new, v_new, slot_mapping};
  return decode(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, true, k_scale,
                v_scale, out, out_dtype, workspace, workspace_bytes, stream, &nt);
}

int pa_kvcache_store_fp8(const void* k, const void* v, const int32_t* slot_mapping, int T,
                         void* k_cache, void* v_cache, int num_blocks, int block_size,
                         int num_kv_heads, int head_dim, float k_scale, float v_scale,
                         void* stream) {
  if (T < 0) return PA_ERR_SHAPE;
  int bs_log2 = 0;
  const int g = check_geometry(num_kv_heads, head_dim, block_size, num_blocks, &bs_log2);
  if (g != PA_OK) return g;
  if (!(k_scale > 0.f && isfinite(k_scale) && v_scale > 0.f && isfinite(v_scale)))
    return PA_ERR_SHAPE;
  if (T == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
  if ((int64_t)T * num_kv_heads * head_dim / 16 > INT32_MAX) return PA_ERR_SHAPE;
  return pa::launch_kvcache_store_fp8(k, v, slot_mapping, T, k_cache, v_cache, num_blocks,
                                      block_size, num_kv_heads, head_dim, k_scale, v_scale,
                                      (hipStream_t)stream) == 0
             ? PA_OK
             : PA_ERR_HIP;
}

}  // extern "C"

namespace {

// The fork and join events of two-stream mixed calls: two per thread and
// device, created by the first such call and kept until the process ends (an
// event's record and the waits on it are consumed at the call, so a thread
// reuses its pair).  Device scope: both streams are on the current device.
int fork_join_events(hipEvent_t* fork, hipEvent_t* join) {
  constexpr int kMaxDevices = 64;
  thread_local hipEvent_t events[kMaxDevices][2] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  for (int i = 0; i < 2; ++i) {
    if (!events[dev][i] &&
        hipEventCreateWithFlags(&events[dev][i], hipEventDisableTiming |
                                                     hipEventReleaseToDevice) != hipSuccess) {
      events[dev][i] = nullptr;
      return -1;
    }
  }
  *fork = events[dev][0];
  *join = events[dev][1];
  return 0;
}

// Shared argument checks and launch of both prefill forms (kv8: FP8 pools,
// every key from the cache; otherwise bf16 pools, the chunk's keys from k_new / v_new).
int prefill(const void* q, const void* k_new, const void* v_new, const int32_t* cu_seqlens_q,
            int num_seqs, int total_q, int max_q_len, const void* k_cache, const void* v_cache,
            const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
            int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
            float scale, bool kv8, float k_scale, float v_scale, void* out, int out_dtype,
            void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_q_heads <= 0 ||
      max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (kv8 && !(k_scale > 0.f && isfinite(k_scale) && v_scale > 0.f && isfinite(v_scale)))
    return PA_ERR_SHAPE;
  int bs_log2 = 0;
  const int g = check_geometry(num_kv_heads, head_dim, block_size, num_blocks, &bs_log2);
  if (g != PA_OK) return g;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX / 2) return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PA_OK;
  if (!q || (!kv8 && (!k_new || !v_new)) || !cu_seqlens_q || !k_cache || !v_cache ||
      !block_tables || !context_lens || !out)
    return PA_ERR_NULL;
  if (max_q_len > total_q) return PA_ERR_SHAPE;

  pa::PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.cu_seqlens_q = cu_seqlens_q;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.B = num_seqs;
  a.mbs = max_blocks_per_seq;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.bs_log2 = bs_log2;
  a.num_blocks = num_blocks;
  a.out_f32 = out_dtype == PA_F32;
  a.max_q_len = max_q_len;
  a.scale_log2e = resolve_scale(scale, head_dim) * (kv8 ? k_scale : 1.f) * pa::kLog2eHost;
  a.v_scale = kv8 ? v_scale : 1.f;
  const int rc = pa::launch_paged_prefill(a, head_dim, kv8, (hipStream_t)stream);
  if (rc == -3) return PA_ERR_UNSUPPORTED;
  return rc == 0 ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int pa_paged_prefill(const void* q, const void* k_new, const void* v_new,
                     const int32_t* cu_seqlens_q, int num_seqs, int total_q, int max_q_len,
                     const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     int max_blocks_per_seq, const int32_t* context_lens, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                     void* out, int out_dtype, void* stream) {
  return prefill(q, k_new, v_new, cu_seqlens_q, num_seqs, total_q, max_q_len, k_cache, v_cache,
                 block_tables, max_blocks_per_seq, context_lens, num_q_heads, num_kv_heads,
                 head_dim, block_size, num_blocks, scale, false, 1.f, 1.f, out, out_dtype, stream);
}

int pa_paged_prefill_fp8(const void* q, const int32_t* cu_seqlens_q, int num_seqs, int total_q,
                         int max_q_len, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, float scale, float k_scale,
                         float v_scale, void* out, int out_dtype, void* stream) {
  return prefill(q, nullptr, nullptr, cu_seqlens_q, num_seqs, total_q, max_q_len, k_cache, v_cache,
                 block_tables, max_blocks_per_seq, context_lens, num_q_heads, num_kv_heads,
                 head_dim, block_size, num_blocks, scale, true, k_scale, v_scale, out, out_dtype,
                 stream);
}

int pa_paged_attention_mixed(const void* q, const void* k_new, const void* v_new,
                             const int32_t* slot_mapping, const int32_t* cu_seqlens_q,
                             int num_prefill_seqs, int num_decode_seqs, int prefill_tokens,
                             int max_prefill_q_len, void* k_cache, void* v_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int num_q_heads, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, float scale, void* out,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream,
                             void* decode_stream) {
  if (num_prefill_seqs < 0 || num_decode_seqs < 0 || prefill_tokens < 0 || max_prefill_q_len < 0)
    return PA_ERR_SHAPE;
  if (num_prefill_seqs == 0 && prefill_tokens != 0) return PA_ERR_SHAPE;
  if (max_prefill_q_len > prefill_tokens) return PA_ERR_SHAPE;
  if (num_prefill_seqs + num_decode_seqs == 0) return PA_OK;
  int bs_log2 = 0;
  const int g = check_geometry(num_kv_heads, head_dim, block_size, num_blocks, &bs_log2);
  if (g != PA_OK) return g;
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 || max_blocks_per_seq <= 0)
    return PA_ERR_SHAPE;
  if (out_dtype != PA_BF16 && out_dtype != PA_F32) return PA_ERR_UNSUPPORTED;
  if (!q || !k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !block_tables ||
      !context_lens || !out || (num_prefill_seqs > 0 && !cu_seqlens_q))
    return PA_ERR_NULL;
  if (num_decode_seqs > 0) {
    const size_t need = pa_paged_decode_workspace_bytes(num_decode_seqs, num_q_heads, num_kv_heads,
                                                        head_dim, block_size, max_blocks_per_seq);
    if (need == 0) return PA_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
  }
  hipStream_t s = (hipStream_t)stream;
  hipStream_t ds = decode_stream ? (hipStream_t)decode_stream : s;
  const bool two_streams = num_decode_seqs > 0 && ds != s;
  // 1. new K/V into the cache before anything attends: a sequence of this
  //    step may reuse a block another one fills in this step, and reads it
  //    from the cache.  On one stream the decode rows store theirs in their
  //    fused call, which runs before the chunks; with a second stream every
  //    row is stored here, before the fork.
  const int stored = two_streams ? prefill_tokens + num_decode_seqs : prefill_tokens;
  int rc = pa_kvcache_store(k_new, v_new, slot_mapping, stored, k_cache, v_cache, num_blocks,
                            block_size, num_kv_heads, head_dim, stream);
  if (rc != PA_OK) return rc;
  // 2. the decode rows, optionally on a second stream that joins back afterwards
  hipEvent_t fork = nullptr, join = nullptr;
  if (two_streams) {
    if (fork_join_events(&fork, &join) != 0 || hipEventRecord(fork, s) != hipSuccess ||
        hipStreamWaitEvent(ds, fork, 0) != hipSuccess)
      return PA_ERR_HIP;
  }
  if (num_decode_seqs > 0) {
    const size_t qrow = (size_t)num_q_heads * head_dim;
    const size_t kvrow = (size_t)num_kv_heads * head_dim;
    const size_t orow = qrow * (out_dtype == PA_F32 ? 4 : 2);
    const void* qd = (const uint16_t*)q + (size_t)prefill_tokens * qrow;
    const int32_t* td = block_tables + (size_t)num_prefill_seqs * max_blocks_per_seq;
    const int32_t* cd = context_lens + num_prefill_seqs;
    void* od = (char*)out + (size_t)prefill_tokens * orow;
    if (two_streams)
      rc = pa_paged_decode(qd, k_cache, v_cache, td, max_blocks_per_seq, cd, num_decode_seqs,
                           num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale, od,
                           out_dtype, workspace, workspace_bytes, ds);
    else
      rc = pa_paged_decode_append(
          qd, (const uint16_t*)k_new + (size_t)prefill_tokens * kvrow,
          (const uint16_t*)v_new + (size_t)prefill_tokens * kvrow, slot_mapping + prefill_tokens,
          k_cache, v_cache, td, max_blocks_per_seq, cd, num_decode_seqs, num_q_heads,
          num_kv_heads, head_dim, block_size, num_blocks, scale, od, out_dtype, workspace,
          workspace_bytes, s);
  }
  // 3. the chunks
  if (rc == PA_OK && num_prefill_seqs > 0 && prefill_tokens > 0)
    rc = pa_paged_prefill(q, k_new, v_new, cu_seqlens_q, num_prefill_seqs, prefill_tokens,
                          max_prefill_q_len > 0 ? max_prefill_q_len : prefill_tokens, k_cache,
                          v_cache, block_tables, max_blocks_per_seq, context_lens, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, scale, out, out_dtype,
                          stream);
  if (two_streams) {
    // join even after an error, so the caller's stream never runs ahead of the decode work
    const bool ok = hipEventRecord(join, ds) == hipSuccess &&
                    hipStreamWaitEvent(s, join, 0) == hipSuccess;
    if (!ok && rc == PA_OK) rc = PA_ERR_HIP;
  }
  return rc;
}

int pa_paged_gather(const void* cache, const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, const int32_t* cu_seqlens_k, int num_seqs,
                    int max_context_len, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, void* out, void* stream) {
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  int bs_log2 = 0;
  const int g = check_geometry(num_kv_heads, head_dim, block_size, num_blocks, &bs_log2);
  if (g != PA_OK) return g;
  if (num_seqs > 65535) return PA_ERR_SHAPE;
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (!cache || !block_tables || !context_lens || !cu_seqlens_k || !out) return PA_ERR_NULL;
  return pa::launch_paged_gather(cache, block_tables, max_blocks_per_seq, context_lens,
                                 cu_seqlens_k, num_seqs, max_context_len, num_kv_heads, head_dim,
                                 bs_log2, num_blocks, out, (hipStream_t)stream) == 0
             ? PA_OK
             : PA_ERR_HIP;
}

int pa_decode_time_next_launch(void* start_event, void* end_event) {
  pa::set_decode_timing((hipEvent_t)start_event, (hipEvent_t)end_event);
  return PA_OK;
}

int pa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return PA_ERR_NULL;
  if (bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || ((uintptr_t)sink & 3) != 0)
    return PA_ERR_SHAPE;
  return pa::launch_stream_read(src, bytes, sink, (hipStream_t)stream) == 0 ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
