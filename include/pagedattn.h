/*
 * libpagedattn — attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * The three operations are the ones a minimal vLLM engine runs inside every
 * attention layer, as described in the MinivLLM guide "vLLM 技术路线"
 * (Step 4 §4.4 allocate_kv_cache, §4.5 prepare_prefill / prepare_decode,
 * §4.6 run_model) and in "Nano-vLLM源码学习(2)" §2 Config (decode and
 * prefix-hit prefill both read paged KV through a block table):
 *
 *   pa_kvcache_store   write the new tokens' K/V rows into cache slots (slot_mapping)
 *   pa_paged_decode    one query token per sequence over its paged context
 *   pa_paged_prefill   a chunk of new tokens over a cached prefix plus itself, causal
 *
 * plus pa_paged_gather, a test aid that un-pages a cache through the block tables,
 * and the FP8 cache variants pa_kvcache_store_fp8 / pa_paged_decode_fp8 /
 * pa_paged_prefill_fp8 (VLLM
 * 0.7.3 source article §5.3: the KV cache may be kept in FP8 while the
 * attention output stays in high precision).
 *
 * Common conventions
 * ------------------
 * - Every tensor pointer is a DEVICE pointer to a dense row-major buffer that
 *   the caller owns.  No call allocates device memory, frees or synchronizes
 *   (except pa_decode_graph_create / _destroy, and the two events a
 *   two-stream pa_paged_attention_mixed creates once per thread and device);
 *   every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream).
 * - bf16 = IEEE bfloat16 bit patterns; indices are int32.
 * - KV cache layout: K and V are separate pools [num_blocks, block_size,
 *   num_kv_heads, head_dim]; the flat slot s = block_id * block_size + offset
 *   addresses row [s / block_size, s % block_size, :, :] (MinivLLM guide
 *   §4.5: a block is kv_cache[..., b*bs:(b+1)*bs, ...], and the decode slot is
 *   block_table[-1] * block_size + last_block_num_tokens - 1).
 * - block_tables [B, max_blocks_per_seq]: logical block j of sequence i lives
 *   in physical block block_tables[i][j] (VLLM 0.7.3 source article §3.1).
 *   Entries past ceil(context_len / block_size) are never read (pad with -1).
 * - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 * - Supported: head_dim in {64, 128}; block_size a power of two in [1, 1024];
 *   num_q_heads a multiple of num_kv_heads.  Decode additionally needs
 *   max_blocks_per_seq * block_size <= 65536 tokens (256 splits of 256
 *   tokens), or 131072 tokens at head_dim 64 with fewer than 3 query heads
 *   per KV head (that kernel's splits are 512 tokens); otherwise the decode
 *   calls return PA_ERR_UNSUPPORTED.
 * - Return value: PA_OK, or a negative pa_status.  Argument errors are found
 *   on the host before anything is launched.  PA_ERR_HIP reports a failed
 *   launch (the HIP error is left for the caller's next HIP call to see).
 * - Device-data preconditions (not checked on the host): slots unique within
 *   a call; table entries for read blocks in [0, num_blocks); context_len <=
 *   max_blocks_per_seq * block_size.  The kernels never touch memory outside
 *   the buffers when these are violated: out-of-range slots are skipped,
 *   out-of-range block ids drop their tokens from the softmax, and context
 *   lengths are clamped to the table width.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = -2,       /* a size is negative/zero where it may not be, or inconsistent */
  PA_ERR_UNSUPPORTED = -3, /* head_dim / block_size / dtype outside the supported set */
  PA_ERR_WORKSPACE = -4,   /* decode workspace missing or too small */
  PA_ERR_HIP = -5,         /* a kernel launch (or another HIP call) failed */
  PA_ERR_OUT_OF_BLOCKS = -6, /* block manager: not enough free blocks */
  PA_ERR_SEQUENCE = -7,    /* block manager: unknown (or already allocated) sequence id */
  PA_ERR_SCRATCH = -8      /* the call needs more than the library's fixed scratch buffer */
} pa_status;

typedef enum { PA_BF16 = 0, PA_F32 = 1 } pa_dtype; /* output element type */

/* Human-readable name of a status code (static storage, never NULL). */
const char* pa_status_string(int status);

/*
 * KV store (MinivLLM guide §4.4-4.5: slot_mapping records where each new
 * token's K/V is written; only uncached tokens get a slot; §4.6: padded rows
 * carry a sentinel).
 *   k, v          [T, num_kv_heads, head_dim] bf16, read
 *   slot_mapping  [T] int32; slot < 0 (padding) or >= num_blocks*block_size writes nothing
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim] bf16, updated in place
 * A bit-exact copy of each row.  T == 0 is a no-op.
 */
int pa_kvcache_store(const void* k, const void* v, const int32_t* slot_mapping, int T,
                     void* k_cache, void* v_cache, int num_blocks, int block_size,
                     int num_kv_heads, int head_dim, void* stream);

/*
 * Bytes of scratch pa_paged_decode needs for these sizes (0 if the sizes are
 * invalid): the most that any batch of 1 .. num_seqs sequences with the other
 * sizes equal needs, so one workspace sized for the largest batch serves
 * every smaller one (the size never decreases as num_seqs grows).  The
 * workspace holds split-K partial results (a running max and sum per query
 * head and split, then the unnormalised outputs); it needs no initialisation
 * and keeps nothing between calls.  It must be 8-byte aligned.  Calls that
 * may run concurrently need separate workspaces.
 */
size_t pa_paged_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int max_blocks_per_seq);

/*
 * Paged decode (MinivLLM guide §4.5 prepare_decode, §4.6 run_model;
 * "Nano-vLLM源码学习(2)" §2: the decode path reads paged KV via block_table).
 *   q             [B, num_q_heads, head_dim] bf16
 *   k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_dim] bf16
 *   block_tables  [B, max_blocks_per_seq] int32
 *   context_lens  [B] int32: keys of sequence i are its logical tokens 0..ctx-1
 *                 (the token being decoded included); ctx <= 0 marks a padded
 *                 row whose output is all zeros
 *   scale         multiplies q.k (fp32); scale <= 0 selects 1/sqrt(head_dim)
 *   out           [B, num_q_heads, head_dim], bf16 (round to nearest even) or fp32
 *   workspace     see pa_paged_decode_workspace_bytes
 * out[i,h] = softmax(scale * q[i,h] . K_i^T) V_i, fp32 accumulation.  With
 * three or more query heads per KV head (the matrix-core path) the attention
 * weights enter the V product rounded to bf16 (relative error at most 2^-9
 * each, the softmax denominator summing the same rounded weights).
 * Deterministic: the same inputs give bit-identical outputs.  Runs as one or
 * two kernels on `stream` (partials, then a merge when a context spans
 * more than one split).
 */
int pa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, int num_seqs, int num_q_heads,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                    void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Fused store + decode: the effect of pa_kvcache_store(k_new, v_new,
 * slot_mapping, T = num_seqs) followed by pa_paged_decode, in one call that
 * launches the decode kernels only (MinivLLM guide §4.5 prepare_decode: each
 * decode step appends one token per sequence at slot_mapping[i] and then
 * attends over its context_lens[i] tokens).
 *   k_new, v_new  [num_seqs, num_kv_heads, head_dim] bf16: the new token of each sequence
 *   slot_mapping  [num_seqs] int32; < 0 or >= num_blocks*block_size stores nothing
 *   k_cache, v_cache  updated in place at those slots; everything else as pa_paged_decode
 * Position context_lens[i]-1 (the new token) is taken from k_new/v_new rather
 * than read back from the cache, so the result equals store-then-decode when
 * slot_mapping[i] is that position's slot under block_tables[i], which is
 * what a decode step passes.  Workspace: pa_paged_decode_workspace_bytes.
 */
int pa_paged_decode_append(const void* q, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, void* k_cache, void* v_cache,
                           const int32_t* block_tables, int max_blocks_per_seq,
                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int num_blocks,
                           float scale, void* out, int out_dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Fused store + decode without a caller workspace, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same operation, arguments and kernels as
 * pa_paged_decode_append, with the split-K partials in a scratch array the
 * library holds in device memory (PA_DECODE_SCRATCH_BYTES per GPU, from the
 * first such call on that GPU until the process ends).  The call allocates and
 * frees nothing.  Sizes whose pa_paged_decode_workspace_bytes exceeds
 * PA_DECODE_SCRATCH_BYTES return PA_ERR_SCRATCH (before anything is launched).
 * Every call on one GPU uses that GPU's one array, so calls that may overlap
 * in time on one GPU (other streams, other threads) race and give wrong
 * results; calls ordered on one stream are safe.  The scratch needs no
 * clearing between calls.
 */
#define PA_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
int pa_paged_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                   const int32_t* slot_mapping, void* k_cache, void* v_cache,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* context_lens, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int num_blocks, float scale, void* out, int out_dtype,
                                   void* stream);

/*
 * FP8 KV cache (VLLM 0.7.3 source article §5.3, KV cache precision: the cache
 * is stored in FP8 while attention outputs stay in high precision).  The page
 * fixes neither format nor scaling; this library uses OCP FP8 E4M3 codes
 * (4 exponent bits, bias 7, 3 mantissa bits, subnormals, no infinities,
 * NaN = S.1111.111, largest magnitude 448) with one fp32 scale per tensor:
 * a value x is stored as E4M3(x / scale) and read back as decode(code) * scale.
 * The pools have the bf16 layout with one byte per element:
 * [num_blocks, block_size, num_kv_heads, head_dim] uint8.
 *
 * pa_kvcache_store_fp8: as pa_kvcache_store, but each bf16 element x of k (v)
 * becomes the code nearest to x / k_scale (x / v_scale), the division in fp32
 * (correctly rounded), the rounding to E4M3 to nearest with ties to the even
 * code, magnitudes above 448 saturating to 448, NaN stored as NaN with its
 * sign.  k_scale and v_scale must be finite and > 0 (else PA_ERR_SHAPE).
 */
int pa_kvcache_store_fp8(const void* k, const void* v, const int32_t* slot_mapping, int T,
                         void* k_cache, void* v_cache, int num_blocks, int block_size,
                         int num_kv_heads, int head_dim, float k_scale, float v_scale,
                         void* stream);

/* Workspace bytes for pa_paged_decode_fp8 (0 if the sizes are invalid). */
size_t pa_paged_decode_fp8_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                           int head_dim, int block_size,
                                           int max_blocks_per_seq);

/*
 * pa_paged_decode on FP8 pools (layout above): attention over the
 * dequantized keys decode(code) * k_scale and values decode(code) * v_scale;
 * q and out as for pa_paged_decode.  The codes are widened exactly to bf16
 * (every E4M3 value is a bf16 value); k_scale is folded into the score scale
 * and v_scale multiplies the merged outputs.  The attention weights enter the
 * V product rounded to bf16 (relative error at most 2^-9 each, the softmax
 * denominator summing the same rounded weights), for every head-group size.
 * k_scale and v_scale must be finite and > 0.
 * Limits, workspace rules and determinism as for pa_paged_decode.
 */
int pa_paged_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int block_size, int num_blocks,
                        float scale, float k_scale, float v_scale, void* out, int out_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused store + decode on FP8 pools: pa_kvcache_store_fp8 followed by
 * pa_paged_decode_fp8 (same scales for both), in one call.  The new token is
 * quantized exactly as the store does and attended from those codes.
 * Workspace: pa_paged_decode_fp8_workspace_bytes.
 */
int pa_paged_decode_append_fp8(const void* q, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, void* k_cache, void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               float scale, float k_scale, float v_scale, void* out,
                               int out_dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Prefix-hit prefill on FP8 pools (layout above).  The chunk's own tokens must
 * already be in the cache (stored by pa_kvcache_store_fp8 with the same
 * scales: a step stores before it attends, MinivLLM guide §4.6), so every key
 * 0 .. context_lens[i]-1 of sequence i is read through its block table: chunk
 * token t (absolute position P + t, P = context_lens[i] - q_len) attends to
 * keys 0 .. P + t with K = decode(code) * k_scale, V = decode(code) * v_scale.
 * Codes are widened exactly to bf16, k_scale is folded into the score scale
 * and v_scale multiplies the outputs; the MFMA arithmetic is that of
 * pa_paged_prefill.  q, cu_seqlens_q, out, limits and errors as for
 * pa_paged_prefill; k_scale and v_scale must be finite and > 0 (else
 * PA_ERR_SHAPE).
 */
int pa_paged_prefill_fp8(const void* q, const int32_t* cu_seqlens_q, int num_seqs, int total_q,
                         int max_q_len, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int max_blocks_per_seq,
                         const int32_t* context_lens, int num_q_heads, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, float scale, float k_scale,
                         float v_scale, void* out, int out_dtype, void* stream);

/*
 * Graph-captured decode steps (MinivLLM guide §4.7: decode steps are captured
 * once per batch-size bucket 1, 2, 4, 8, 16, 32, ... into static input
 * buffers, a step fills the first rows, pads the rest with sentinels and
 * replays the smallest bucket that fits; §4.5: the index tensors are built in
 * pinned host memory and uploaded with non-blocking copies).
 *
 * An opaque object that owns static device buffers (q, new K/V rows, output,
 * index arrays, split-K workspace), four pinned host staging areas, and one
 * instantiated HIP graph per bucket of the fused store + decode call
 * (pa_paged_decode_append, or pa_paged_decode_append_fp8 when kv_fp8 != 0)
 * over the caller's caches.  Unlike the other calls, create allocates (device
 * memory, pinned host memory, graphs) and synchronizes the device; run
 * allocates nothing.
 *
 * pa_decode_graph_create: buckets are 1, 2, 4, 8 and the multiples of 16 below
 *   max_batch (<= 65536), plus max_batch.  k_cache/v_cache must stay valid for
 *   the object's life.  Other arguments as for the decode calls.
 * pa_decode_graph_buffers: the static q [max_batch, Hq, D], k_new/v_new
 *   [max_batch, Hkv, D] (bf16) and out [max_batch, Hq, D] device buffers;
 *   writing q/k_new/v_new there in place saves run's copies.
 * pa_decode_graph_bucket: the bucket a batch of `batch` rows replays (0 if
 *   batch is out of range).
 * pa_decode_graph_run: one decode step for `batch` sequences on `stream`.
 *   q, k_new, v_new: device pointers to the batch's rows (copied into the
 *   static buffers unless they are those buffers; NULL = already there).
 *   slot_mapping [batch], context_lens [batch] and block_tables
 *   [batch, tables_stride] (tables_stride <= max_blocks_per_seq) are HOST
 *   arrays: they are copied into pinned staging (rows batch..bucket-1 get
 *   slot -1, length 0 and table -1) and uploaded asynchronously with one copy;
 *   the host blocks only if the staging area it is about to refill (the one
 *   used four steps earlier) is still being uploaded.  out: device pointer
 *   that receives the
 *   batch's rows (NULL = leave them in the static output).  Must be called on
 *   the device the object was created on; consecutive runs of one object
 *   must use the same stream (or be ordered by the caller).
 * pa_decode_graph_destroy: waits for the device, frees everything.  NULL is a no-op.
 */
typedef struct pa_decode_graph pa_decode_graph;

int pa_decode_graph_create(int max_batch, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_blocks_per_seq, int kv_fp8,
                           float scale, float k_scale, float v_scale, void* k_cache,
                           void* v_cache, int out_dtype, pa_decode_graph** out_graph);
int pa_decode_graph_buffers(const pa_decode_graph* graph, void** q, void** k_new, void** v_new,
                            void** out);
int pa_decode_graph_bucket(const pa_decode_graph* graph, int batch);
int pa_decode_graph_run(pa_decode_graph* graph, int batch, const void* q, const void* k_new,
                        const void* v_new, const int32_t* slot_mapping,
                        const int32_t* block_tables, int tables_stride,
                        const int32_t* context_lens, void* out, void* stream);
int pa_decode_graph_destroy(pa_decode_graph* graph);

/*
 * Prefix-hit prefill ("Nano-vLLM源码学习(2)" §2: the prefix-hit prefill path
 * reads the cached prefix through block_table; MinivLLM guide §4.5: the batch
 * is flattened and delimited by cu_seqlens_q, e.g. [0, 3, 5, 9]).
 *   q             [total_q, num_q_heads, head_dim] bf16
 *   k_new, v_new  [total_q, num_kv_heads, head_dim] bf16: K/V of the new tokens
 *   cu_seqlens_q  [B+1] int32 (device), cu_seqlens_q[0] = 0, cu_seqlens_q[B] = total_q
 *   max_q_len     host-known upper bound of any q_len (sizes the grid)
 *   k_cache, v_cache, block_tables: the cached prefix, as for decode
 *   context_lens  [B] int32 = prefix_len + q_len per sequence
 * Chunk token t of sequence i sits at absolute position P_i + t, P_i =
 * context_lens[i] - q_len_i, and attends to keys 0..P_i+t: keys below P_i are
 * read from the cache, the rest from k_new/v_new.  The new tokens need not
 * have been stored yet.  out is [total_q, num_q_heads, head_dim], bf16 or fp32.
 */
int pa_paged_prefill(const void* q, const void* k_new, const void* v_new,
                     const int32_t* cu_seqlens_q, int num_seqs, int total_q, int max_q_len,
                     const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     int max_blocks_per_seq, const int32_t* context_lens, int num_q_heads,
                     int num_kv_heads, int head_dim, int block_size, int num_blocks, float scale,
                     void* out, int out_dtype, void* stream);

/*
 * Mixed prefill + decode step in one call: chunks and single decode tokens
 * under one cu_seqlens_q ("Nano-vLLM源码学习(2)" §2: prefill and decode both
 * read paged KV through block_table; the VLLM 0.7.3 source article §3.2: one
 * iteration batches new requests' prefill with running requests' decode).
 * Sequences 0 .. num_prefill_seqs-1 are chunks over rows 0 .. prefill_tokens-1
 * (cu_seqlens_q [num_prefill_seqs+1], device, as for pa_paged_prefill; any
 * q_len >= 0); sequences num_prefill_seqs .. +num_decode_seqs-1 have one row
 * each, rows prefill_tokens + i (a decode row is a chunk of one token).
 *   q [prefill_tokens + num_decode_seqs, Hq, D]; k_new, v_new and
 *   slot_mapping [prefill_tokens + num_decode_seqs] rows: every new token's
 *   K/V and slot; block_tables [num_prefill_seqs + num_decode_seqs, MBS] and
 *   context_lens (prefix + q_len) in the same sequence order; out like q.
 *   workspace: pa_paged_decode_workspace_bytes(num_decode_seqs, ...).
 * Effect: every new token is stored (slot < 0 skips), then each row attends
 * to its sequence's keys 0 .. its position, as pa_paged_prefill would for a
 * q_len-1 chunk and as pa_paged_decode does.  Every token of the call is
 * stored before any row that could read it attends, so a chunk may read a
 * block that another chunk or a decode row of the same call fills (prefix
 * caching registers a block as soon as its last token arrives).  On one
 * stream: the chunks' tokens are stored, then the decode rows run as
 * pa_paged_decode_append (storing their own tokens), then the chunks attend.
 * With decode_stream != NULL and != stream: every token is stored on
 * `stream`, then the decode rows run as pa_paged_decode on decode_stream
 * while the chunks attend on `stream`; decode_stream is forked from and
 * joined back into `stream` with two events (the call then returns with all
 * of its work ordered before later work on `stream`).  The events are
 * created by the first such call on a thread and device and kept until the
 * process ends (the only objects this call creates).  decode_stream must
 * have default priority and be on the current device.
 */
int pa_paged_attention_mixed(const void* q, const void* k_new, const void* v_new,
                             const int32_t* slot_mapping, const int32_t* cu_seqlens_q,
                             int num_prefill_seqs, int num_decode_seqs, int prefill_tokens,
                             int max_prefill_q_len, void* k_cache, void* v_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int num_q_heads, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, float scale, void* out,
                             int out_dtype, void* workspace, size_t workspace_bytes, void* stream,
                             void* decode_stream);

/*
 * Test aid: un-page one cache (MinivLLM guide §4.5 block_tables).
 *   cache         [num_blocks, block_size, num_kv_heads, head_dim] bf16
 *   cu_seqlens_k  [B+1] int32 (device): prefix sums of context_lens
 *   out           [cu_seqlens_k[B], num_kv_heads, head_dim] bf16:
 *                 out[cu_seqlens_k[i] + j] = cache row of logical token j of sequence i
 *   max_context_len  host-known upper bound of any context_len (sizes the grid)
 * Bit-exact copy; rows of tokens whose block id is out of range are left untouched.
 */
int pa_paged_gather(const void* cache, const int32_t* block_tables, int max_blocks_per_seq,
                    const int32_t* context_lens, const int32_t* cu_seqlens_k, int num_seqs,
                    int max_context_len, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, void* out, void* stream);

/*
 * Measurement aid: reads `bytes` bytes at `src` (device) once, in contiguous
 * 32 KiB runs per workgroup with non-temporal 16-byte loads; a timed call
 * gives the device's streaming-read rate, the practical ceiling of the
 * bandwidth-bound decode next to the HBM spec peak.  Not part of the
 * attention path.
 *   src    16-byte aligned, bytes a multiple of 16 (else PA_ERR_SHAPE)
 *   sink   4 bytes of device memory, 4-byte aligned, that the kernel may
 *          overwrite (it keeps the loads live; the value means nothing)
 * Asynchronous on `stream`; bytes == 0 is a no-op.
 */
int pa_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Measurement aid: the next decode call made by the calling thread
 * (pa_paged_decode*, including the fused and FP8 forms and the decode rows of
 * pa_paged_attention_mixed) attaches start_event and end_event to the launch
 * of its main split kernel (hipExtLaunchKernel), so the two events carry that
 * kernel's own start and end times: no separate event packets, and neither
 * the store nor the split merge.  Events are hipEvent_t handles the caller
 * created with timing enabled (either may be NULL).  The request is consumed
 * by that call.  Always returns PA_OK.
 */
int pa_decode_time_next_launch(void* start_event, void* end_event);

/*
 * Host block manager with prefix caching (MinivLLM guide Step 3 §3.2 Block,
 * §3.3 BlockManager; Step 4 §4.5 prepare_prefill / prepare_decode).  Host
 * memory only, no GPU calls; not thread-safe (one caller at a time per
 * object).  It hands out the physical block ids of one KV pool and produces
 * the slot_mapping / block_tables / context_lens / cu_seqlens_q arrays the
 * kernels above consume.
 *
 * Readings where the pages leave a step open:
 * - A full block's hash is 64-bit FNV-1a over the previous block's hash (8
 *   bytes, little endian; omitted for the first block) then the block's token
 *   ids (4 bytes each, little endian), masked to hash_bits bits (64 = all;
 *   fewer only to provoke collisions in tests).  A cached block is reused only
 *   if its hash is registered and it holds exactly the same tokens.
 * - Free blocks form a FIFO list, initially 0..num_blocks-1: allocation takes
 *   the head, a freed block joins the tail and keeps its contents and hash
 *   (still reusable) until it is handed out for other contents.
 * - allocate: the prompt's blocks in order; the first miss makes every later
 *   block a miss; a hit on a block in use adds a reference, a hit on a free
 *   block takes it back (reference count 1); a missed full block gets a fresh
 *   block and registers its hash; the partial last block is never shared.
 *   can_allocate counts all the prompt's blocks (hits not subtracted).
 * - append adds one token: it takes a new block when the token opens one and
 *   registers the last block's hash when the token fills it (a 256-token
 *   sequence's 257th token opens block 2 at offset 0).
 * - deallocate drops one reference per table entry, last block first; blocks
 *   reaching zero join the free list in that order.
 *
 * pa_bm_create: num_blocks * block_size <= INT32_MAX, 1 <= hash_bits <= 64.
 * pa_bm_can_allocate / pa_bm_can_append return 1 or 0 (or an error < 0).
 * pa_bm_allocate: *num_cached_tokens = tokens covered by reused blocks.
 *   PA_ERR_OUT_OF_BLOCKS if can_allocate is false (nothing changes);
 *   PA_ERR_SEQUENCE if seq_id is live.
 * pa_bm_append: PA_ERR_OUT_OF_BLOCKS (nothing changes) if the token needs a
 *   block and none is free.
 * pa_bm_block_table / pa_bm_free_list: write up to `capacity` entries, return
 *   the full count.  pa_bm_ref_count: a block's reference count.
 * pa_bm_prepare_decode: per sequence, context_lens = its length, slot_mapping =
 *   slot of its last token, block_tables row padded with -1 to
 *   max_blocks_per_seq (PA_ERR_SHAPE if a table is longer).
 * pa_bm_prepare_prefill: per sequence, its uncached tokens (positions
 *   num_cached .. len-1): cu_seqlens_q [num_seqs+1] over those counts,
 *   slot_mapping [total_q] (at most slot_capacity), context_lens = lengths,
 *   padded block_tables; *total_q and *max_q_len for the prefill call.
 */
typedef struct pa_block_manager pa_block_manager;

int pa_bm_create(int num_blocks, int block_size, int hash_bits, pa_block_manager** out);
int pa_bm_destroy(pa_block_manager* bm);
int pa_bm_num_free(const pa_block_manager* bm);
int pa_bm_can_allocate(const pa_block_manager* bm, int num_tokens);
int pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens, int num_tokens,
                   int* num_cached_tokens);
int pa_bm_can_append(const pa_block_manager* bm, int64_t seq_id);
int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t token);
int pa_bm_deallocate(pa_block_manager* bm, int64_t seq_id);
int pa_bm_seq_info(const pa_block_manager* bm, int64_t seq_id, int* num_tokens,
                   int* num_cached_tokens, int* num_blocks);
int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out, int capacity);
int pa_bm_free_list(const pa_block_manager* bm, int32_t* out, int capacity);
int pa_bm_ref_count(const pa_block_manager* bm, int block_id);
int pa_bm_prepare_decode(const pa_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                         int max_blocks_per_seq, int32_t* slot_mapping, int32_t* context_lens,
                         int32_t* block_tables);
int pa_bm_prepare_prefill(const pa_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                          int max_blocks_per_seq, int32_t* cu_seqlens_q, int32_t* context_lens,
                          int32_t* block_tables, int32_t* slot_mapping, int slot_capacity,
                          int* total_q, int* max_q_len);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
