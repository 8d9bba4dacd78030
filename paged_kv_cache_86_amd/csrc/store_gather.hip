// KV store (slot_mapping scatter) and the block-table un-page used by tests.
//
// Store: MinivLLM guide "vLLM 技术路线", Step 4 §4.4 (slot_mapping tracks
// which token of which sequence goes where) and §4.5 (only uncached tokens get
// a slot; slot = block_id * block_size + offset).  With the [num_blocks,
// block_size, Hkv, D] layout, slot s is simply row s of a [num_blocks *
// block_size, Hkv * D] matrix, so the scatter needs no division.
#include "common.h"
#include "kernels.h"

namespace pa {

// Each thread moves kStoreItems 16-byte vectors (8 bf16 each) of K and the
// same vectors of V: all loads are issued before the first store.  Vector e
// of token t is element (t * row_vecs + e) of the flat [T * row_vecs] view;
// its destination is row slot_mapping[t] of the [NB * BS, row_vecs] cache.
constexpr int kStoreItems = 4;

__global__ __launch_bounds__(256) void kvcache_store_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int32_t* __restrict__ slot_mapping, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int T, int row_vecs, int64_t num_slots) {
  const int64_t total = (int64_t)T * row_vecs;
  const int64_t first = (int64_t)blockIdx.x * 256 * kStoreItems + threadIdx.x;
  u32x4 kv[kStoreItems], vv[kStoreItems];
  int64_t dst[kStoreItems];
#pragma unroll
  for (int i = 0; i < kStoreItems; ++i) {
    const int64_t idx = first + (int64_t)i * 256;
    dst[i] = -1;
    if (idx < total) {
      const int t = (int)(idx / row_vecs);
      const int e = (int)(idx - (int64_t)t * row_vecs);
      const int32_t s = slot_mapping[t];
      kv[i] = k[idx];
      vv[i] = v[idx];
      if (s >= 0 && (int64_t)s < num_slots) dst[i] = (int64_t)s * row_vecs + e;
    }
  }
#pragma unroll
  for (int i = 0; i < kStoreItems; ++i) {
    if (dst[i] >= 0) {
      k_cache[dst[i]] = kv[i];
      v_cache[dst[i]] = vv[i];
    }
  }
}

int launch_kvcache_store(const void* k, const void* v, const int32_t* slot_mapping, int T,
                         void* k_cache, void* v_cache, int num_blocks, int block_size,
                         int num_kv_heads, int head_dim, hipStream_t stream) {
  if (T == 0) return 0;
  const int row_vecs = num_kv_heads * head_dim / 8;
  const int64_t total = (int64_t)T * row_vecs;
  const int64_t per_wg = 256 * kStoreItems;
  dim3 grid((unsigned)((total + per_wg - 1) / per_wg));
  hipLaunchKernelGGL(kvcache_store_kernel, grid, dim3(256), 0, stream,
                     (const u32x4*)k, (const u32x4*)v, slot_mapping, (u32x4*)k_cache,
                     (u32x4*)v_cache, T, row_vecs, (int64_t)num_blocks * block_size);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// FP8 store: each thread turns 16 bf16 values of K (and of V) into 16 E4M3
// codes (quantize8 twice).  Vector e of token t covers elements 16e .. 16e+15
// of its row.
__device__ __forceinline__ u32x4 quantize16(const u32x4& a, const u32x4& b, float s) {
  const u32x2 lo = quantize8(a, s), hi = quantize8(b, s);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

__global__ __launch_bounds__(256) void kvcache_store_fp8_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v,
    const int32_t* __restrict__ slot_mapping, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, int T, int row_vecs8, int64_t num_slots, float k_scale,
    float v_scale) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)T * row_vecs8) return;
  const int t = (int)(idx / row_vecs8);
  const int e = (int)(idx - (int64_t)t * row_vecs8);
  const int32_t s = slot_mapping[t];
  if (s < 0 || (int64_t)s >= num_slots) return;
  const u32x4 k0 = k[2 * idx], k1 = k[2 * idx + 1];
  const u32x4 v0 = v[2 * idx], v1 = v[2 * idx + 1];
  k_cache[(int64_t)s * row_vecs8 + e] = quantize16(k0, k1, k_scale);
  v_cache[(int64_t)s * row_vecs8 + e] = quantize16(v0, v1, v_scale);
}

int launch_kvcache_store_fp8(const void* k, const void* v, const int32_t* slot_mapping, int T,
                             void* k_cache, void* v_cache, int num_blocks, int block_size,
                             int num_kv_heads, int head_dim, float k_scale, float v_scale,
                             hipStream_t stream) {
  if (T == 0) return 0;
  const int row_vecs8 = num_kv_heads * head_dim / 16;
  const int64_t total = (int64_t)T * row_vecs8;
  hipLaunchKernelGGL(kvcache_store_fp8_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, stream, (const u32x4*)k, (const u32x4*)v, slot_mapping, (u32x4*)k_cache,
                     (u32x4*)v_cache, T, row_vecs8, (int64_t)num_blocks * block_size, k_scale,
                     v_scale);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Un-page: grid (token tiles of 64, sequences).  Thread layout: 64 tokens x
// `row_vecs` 16-byte vectors, strided by the block size of 256 threads.
__global__ __launch_bounds__(256) void paged_gather_kernel(
    const u32x4* __restrict__ cache, const int32_t* __restrict__ block_tables, int mbs,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_seqlens_k,
    u32x4* __restrict__ out, int row_vecs, int bs_log2, int num_blocks) {
  const int seq = blockIdx.y;
  int ctx = context_lens[seq];
  ctx = ctx < 0 ? 0 : ctx;
  const int cap = mbs << bs_log2;
  ctx = ctx > cap ? cap : ctx;
  const int tok0 = blockIdx.x * 64;
  if (tok0 >= ctx) return;
  const int64_t base = cu_seqlens_k[seq];
  const int work = 64 * row_vecs;
  for (int i = threadIdx.x; i < work; i += blockDim.x) {
    const int j = tok0 + i / row_vecs;
    const int e = i % row_vecs;
    if (j >= ctx) continue;
    const int32_t blk = block_tables[(int64_t)seq * mbs + (j >> bs_log2)];
    if (blk < 0 || blk >= num_blocks) continue;
    const int64_t row = ((int64_t)blk << bs_log2) + (j & ((1 << bs_log2) - 1));
    out[(base + j) * row_vecs + e] = cache[row * row_vecs + e];
  }
}

int launch_paged_gather(const void* cache, const int32_t* block_tables, int mbs,
                        const int32_t* context_lens, const int32_t* cu_seqlens_k, int B,
                        int max_context_len, int num_kv_heads, int head_dim, int bs_log2,
                        int num_blocks, void* out, hipStream_t stream) {
  if (B == 0 || max_context_len == 0) return 0;
  const int row_vecs = num_kv_heads * head_dim / 8;
  dim3 grid((unsigned)((max_context_len + 63) / 64), (unsigned)B);
  hipLaunchKernelGGL(paged_gather_kernel, grid, dim3(256), 0, stream, (const u32x4*)cache,
                     block_tables, mbs, context_lens, cu_seqlens_k, (u32x4*)out, row_vecs,
                     bs_log2, num_blocks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace pa
