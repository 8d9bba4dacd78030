// Internal launch interface between the C ABI (pagedattn.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr float kLog2eHost = 1.4426950408889634f;
// Upper bound of (sequence, KV-head group) pairs in one decode call (one
// combine workgroup each).
constexpr int64_t kDecodeMaxUnits = 1 << 24;
// Most short splits one decode context may span (bounds the longest context;
// the merge stages up to this many partials in LDS).
constexpr int kDecodeMaxSplits = 256;
// Long splits (twice the short length) are used when the longest context
// spans at least this many short splits ...
constexpr int kLongSplitMinShort = 8;
// ... and the grid with half the slots per sequence still has this many
// workgroups (32 per compute unit of a 256-CU device; 4 on FP8 pools, whose
// workgroups carry more vector work per byte, so halving their number pays
// from smaller grids).
constexpr int64_t kLongSplitMinGrid = 8192;
constexpr int64_t kLongSplitMinGridFp8 = 1024;
// Decode grids of up to this many sequences take their (sequence, split)
// items from a compacted list (4 sequences per lane of one wave in the
// lookup); larger batches take their slots split-major from the last slot
// down, where the lookup's extra round trip costs more than the empty
// workgroups it removes (measured at 512).
constexpr int kCompactPerLane = 4;
constexpr int kCompactMaxSeqs = 64 * kCompactPerLane;
// Query heads per KV head from which decode runs on MFMA (bf16 and FP8
// pools), the most heads one MFMA workgroup serves, and its split lengths:
// long splits when the grid with them still has kMfmaLongMinGrid workgroups
// (8 per compute unit), short ones otherwise (small batches keep enough
// workgroups to fill the device).
constexpr int kMfmaMinGroup = 3;
constexpr int kMfmaMinGroupFp8 = 3;
constexpr int kMfmaMaxGt = 16;
constexpr int kMfmaSplitTokens = 256;
constexpr int kMfmaLongSplitTokens = 2048;
constexpr int64_t kMfmaLongMinGrid = 2048;

int launch_kvcache_store(const void* k, const void* v, const int32_t* slot_mapping, int T,
                         void* k_cache, void* v_cache, int num_blocks, int block_size,
                         int num_kv_heads, int head_dim, hipStream_t stream);

int launch_paged_gather(const void* cache, const int32_t* block_tables, int mbs,
                        const int32_t* context_lens, const int32_t* cu_seqlens_k, int B,
                        int max_context_len, int num_kv_heads, int head_dim, int bs_log2,
                        int num_blocks, void* out, hipStream_t stream);

// Split-K geometry of a decode call; a function of host-known sizes only.
struct DecodePlan {
  int group;       // query heads per KV head
  int nsub;        // workgroups sharing one KV head's query heads
  int gt;          // query heads handled by one workgroup (<= 8)
  int split_log2;    // tokens per short split = 1 << split_log2
  int nsplit_short;  // short splits of the longest possible context
  bool long_splits;  // contexts above long_above short splits use splits of twice the length
  int long_above;    // nsplit_max on bf16 pools, 1 on FP8 pools (with long_splits)
  int nsplit_max;    // workgroups (and partial slots) per (sequence, head group)
  bool mfma;         // the MFMA kernel (bf16 pools, large query-head groups)
  bool compact;      // workgroups take compacted (sequence, split) items
  int64_t units;   // (sequence, head group) pairs
  size_t ml_bytes, o_bytes;  // workspace regions: (max, sum) pairs, then unnormalised outputs
  // Splits longer than the kernel's short split (VALU long splits, or the
  // MFMA kernel's long split length): chosen from some batch size up.
  bool coarse() const {
    return long_splits || (mfma && (1 << split_log2) == kMfmaLongSplitTokens);
  }
  size_t workspace_bytes() const { return ml_bytes + o_bytes; }
};

DecodePlan plan_decode(int B, int Hq, int Hkv, int head_dim, int block_size, int mbs,
                       bool kv8 = false);

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_ml;
  float* ws_o;
  int mbs, Hq, Hkv, group, nsub, hg, bs_log2, split_log2, nsplit_max, num_blocks, out_f32;
  int long_splits;    // see DecodePlan
  int long_above;     // see DecodePlan
  int batch;          // sequences (B)
  int compact;        // see DecodePlan
  float scale_log2e;  // softmax scale (times the K scale of an FP8 cache) times log2(e)
  float v_scale;      // V scale of an FP8 cache (1 for bf16)
  // Fused store of the new token (append variants only; unused otherwise).
  const uint16_t* k_new;  // [B, Hkv, D] bf16
  const uint16_t* v_new;
  const int32_t* slot_mapping;  // [B]
  void* k_cache_w;  // the caches again, written
  void* v_cache_w;
  int64_t num_slots;
  float qscale_k, qscale_v;  // FP8 quantization divisors
};

int launch_paged_decode(const DecodeArgs& args, int B, int head_dim, int gt, bool kv8,
                        bool append, bool mfma, hipStream_t stream);

// Measurement aid: events the next decode launch of the calling thread records
// on its stream right before and right after its main (split) kernel.
void set_decode_timing(hipEvent_t start, hipEvent_t end);
// The calling thread's pending events (cleared by the call); null when none.
void take_decode_timing(hipEvent_t* start, hipEvent_t* end);
int launch_paged_decode_mfma(const DecodeArgs& args, int B, int head_dim, bool kv8, bool append,
                             hipStream_t stream);
// Merge kernel of both decode kernels: split partials -> outputs.
int launch_decode_combine(const DecodeArgs& args, int B, int head_dim, int gt,
                          hipStream_t stream);

int launch_kvcache_store_fp8(const void* k, const void* v, const int32_t* slot_mapping, int T,
                             void* k_cache, void* v_cache, int num_blocks, int block_size,
                             int num_kv_heads, int head_dim, float k_scale, float v_scale,
                             hipStream_t stream);

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* cu_seqlens_q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  int B, mbs, Hq, Hkv, group, bs_log2, num_blocks, out_f32, max_q_len;
  float scale_log2e;  // softmax scale (times the K scale of an FP8 cache) times log2(e)
  float v_scale;      // V scale of an FP8 cache (1 for bf16)
};

int launch_paged_prefill(const PrefillArgs& args, int head_dim, bool kv8, hipStream_t stream);

int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace pa
