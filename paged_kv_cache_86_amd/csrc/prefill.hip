// Prefix-hit paged prefill for gfx950 on bf16 MFMA ("Nano-vLLM源码学习(2)" §2:
// the prefix-hit prefill path reads the cached prefix through block_table;
// MinivLLM guide "vLLM 技术路线", Step 4 §4.5: one launch over the flattened
// batch, sequences delimited by cu_seqlens_q).
//
// Chunk token t of a sequence sits at position P + t (P = cached prefix) and
// attends to keys 0 .. P + t; keys < P come from the paged cache, the rest from
// k_new / v_new.  Both contractions are dense, so they run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation and an online softmax in
// fp32 (flash-attention style):
//
//   * a workgroup (4 waves) owns 128 query rows = TT tokens x G heads of one
//     KV head (GQA rows share every K/V tile) and walks 64-key tiles;
//   * S^T = K Q^T and O^T = V^T P^T: the accumulator layout gives each lane one
//     query row, so the softmax is per lane (plus one exchange with the lane
//     holding the row's other 32 keys, v_permlane32_swap) and P feeds the
//     second MFMA from registers; the softmax denominator sums exactly the
//     bf16 weights the PV product uses (v_dot2_f32_bf16 against ones, each
//     lane over its half of the keys, the halves added at the end);
//   * K and V tiles go straight from global memory to LDS
//     (global_load_lds_dwordx4), double-buffered, one barrier per tile; rows are
//     stored with their 16-byte chunks XOR-swizzled so that both the K operand
//     reads (ds_read_b128) and the V^T operand reads (ds_read_b64_tr_b16, a
//     transposing read) spread over the LDS banks;
//   * O is rescaled only when a row's running max grows by more than 2^8
//     (exp2 units), otherwise the stale max is kept;
//   * workgroups take their (token tile, sequence) items longest first (see
//     ranked_item), which keeps the grid's tail short when cached prefixes
//     differ in length.
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kRows = 128;     // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kMaxBt = 1024;   // prefix block ids staged in LDS
constexpr float kRescaleLog2 = 8.f;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Chunk swizzle of a K/V row inside a tile: 16-byte chunk c of row r is stored
// at chunk position c ^ swz(r).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}

// Max and sum of a value over lanes l and l ^ 32 (v_permlane32_swap exchanges
// the two halves of the wave).
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Exclusive prefix sum of one int per thread over a 256-thread workgroup
// (`tmp`: 4 ints of LDS used by this call only); `total` gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) base += i < w ? tmp[i] : 0;
  total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  return base + x - v;
}

// Work order of the prefill grid.  Workgroups are handed out roughly in
// index order and the work per (token tile, sequence) item varies with the
// sequence's cached prefix, so index order leaves a long tail; ranking the
// items by the keys they walk, most first, and giving rank r to workgroups
// r * Hkv .. r * Hkv + Hkv - 1 is the longest-processing-time-first list
// schedule.  Every workgroup computes the ranking itself from the lengths in
// device memory (a 256-bin histogram of tile counts, then two workgroup
// scans), which costs O(items / 256) per thread, so it is used up to
// kOrderMaxItems items and index order beyond.
constexpr int kOrderBins = 256;
constexpr int kOrderMaxItems = 4096;

// Priority bin of item i = seq * ntt + tt (0 = most keys to walk).
__device__ __forceinline__ int order_bin(const PrefillArgs& a, int i, int ntt, int tt_tokens,
                                         int cap, int shift) {
  const int seq = i / ntt;
  const int tt = i - seq * ntt;
  const int qa = a.cu_seqlens_q[seq];
  const int n = a.cu_seqlens_q[seq + 1] - qa;
  const int t0 = tt * tt_tokens;
  if (n <= 0 || t0 >= n) return kOrderBins - 1;
  int P = a.context_lens[seq] - n;
  P = P < 0 ? 0 : (P > cap ? cap : P);
  const int tiles = (P + min(t0 + tt_tokens, n) + 63) >> 6;
  return kOrderBins - 1 - min(tiles >> shift, kOrderBins - 1);
}

// The (token tile, sequence) item of rank r when items are ordered by the
// keys they walk, most first, ties by index.  s: 256 + 16 ints of LDS.
__device__ void ranked_item(const PrefillArgs& a, int ntt, int tt_tokens, int r, int* s,
                            int& tt_out, int& seq_out) {
  const int tid = threadIdx.x;
  const int M = a.B * ntt;
  const int per = (M + 255) >> 8;
  const int i0 = min(tid * per, M), i1 = min(i0 + per, M);
  const int cap = a.mbs << a.bs_log2;
  const int64_t maxtiles = ((int64_t)cap + a.max_q_len + 63) >> 6;
  int shift = 0;
  while ((maxtiles >> shift) >= kOrderBins) ++shift;
  int* hist = s;
  int* sel = s + kOrderBins;  // [0..3] scan 1, [4..7] scan 2, [8] bin, [9] offset, [10] item
  hist[tid] = 0;
  if (tid == 0) sel[10] = 0;  // a valid item whatever happens below
  __syncthreads();
  for (int i = i0; i < i1; ++i) atomicAdd(&hist[order_bin(a, i, ntt, tt_tokens, cap, shift)], 1);
  __syncthreads();
  const int h = hist[tid];
  int total;
  const int start = block_excl_scan(h, sel, total);
  if (r >= start && r < start + h) {
    sel[8] = tid;
    sel[9] = r - start;
  }
  __syncthreads();
  const int bin = sel[8];
  const int off = sel[9];
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += order_bin(a, i, ntt, tt_tokens, cap, shift) == bin;
  const int before = block_excl_scan(cnt, sel + 4, total);
  if (off >= before && off < before + cnt) {
    int k = off - before;
    for (int i = i0; i < i1; ++i) {
      if (order_bin(a, i, ntt, tt_tokens, cap, shift) == bin) {
        if (k == 0) { sel[10] = i; break; }
        --k;
      }
    }
  }
  __syncthreads();
  const int item = sel[10];
  seq_out = item / ntt;
  tt_out = item - seq_out * ntt;
}

// KV8 reads an FP8 (OCP E4M3) cache: the chunk's own tokens have been stored
// into it already, so every key 0 .. ctx-1 comes through the block table; a
// tile's codes are loaded into registers, widened exactly to bf16 (scale 1)
// and written into the same swizzled LDS layout (so the MFMA part is
// unchanged), one tile ahead of the compute; the K scale is folded into the
// score scale and the V scale multiplies the outputs.
template <int D, bool KV8>
__global__ __launch_bounds__(256, 2) void paged_prefill_kernel(PrefillArgs a, int tt_tokens,
                                                            int ntt, int ranked) {
  constexpr int KS = D / 16;                    // 16-wide K steps over head_dim
  constexpr int DT = D / 32;                    // 32-row tiles of O^T
  constexpr int CPR = D / 8;                    // 16-byte chunks per K/V row
  constexpr int RPI = 64 / CPR;                 // rows per 1 KiB direct-to-LDS load
  constexpr int IPW = kBN / RPI / 4;            // such loads per wave per tile and tensor
  constexpr int TILE = kBN * D;                 // elements of one K or V tile

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* tiles = smem;                                   // [2 buffers][K, V][TILE]
  int* s_bt = (int*)(smem + 4 * TILE);                      // prefix block ids
  int* s_flags = s_bt + kMaxBt;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;  // this lane's query row within the wave
  const int hi = lane >> 5;  // which half of a 16-wide K step

  // Items in rank order (see ranked_item), else the last token tiles first
  // (later tiles attend to more keys).  Either way the workgroups of one
  // (sequence, KV head) are a multiple of Hkv apart, so they land on one XCD
  // when Hkv is a multiple of 8 and share its L2.
  int tt, seq, kvh;
  if (ranked) {
    kvh = (int)(blockIdx.x % a.Hkv);
    ranked_item(a, ntt, tt_tokens, (int)(blockIdx.x / a.Hkv), (int*)smem, tt, seq);
  } else {
    const int per_tt = a.B * a.Hkv;
    tt = ntt - 1 - (int)(blockIdx.x / per_tt);
    const int rem = blockIdx.x % per_tt;
    seq = rem / a.Hkv;
    kvh = rem - seq * a.Hkv;
  }

  const int qa = a.cu_seqlens_q[seq];
  const int n = a.cu_seqlens_q[seq + 1] - qa;
  const int t0 = tt * tt_tokens;
  if (n <= 0 || t0 >= n) return;
  const int cap = a.mbs << a.bs_log2;
  int P = a.context_lens[seq] - n;
  P = P < 0 ? 0 : (P > cap ? cap : P);
  const int t_hi = min(t0 + tt_tokens, n);
  const int kend = P + t_hi;  // keys this workgroup needs: 0 .. kend-1
  const int ntiles = (kend + kBN - 1) / kBN;
  const int G = a.group;

  // This lane's query row.
  const int row = w * 32 + lr;
  const int t_loc = row / G;
  const int hq = row - t_loc * G;
  const bool row_ok = (t_loc < tt_tokens) && (t0 + t_loc < n);
  const int tok = row_ok ? t0 + t_loc : t0;
  const int pos = P + tok;  // sees keys 0 .. pos
  const int64_t qrow = ((int64_t)(qa + tok) * a.Hq + kvh * G + hq) * D;

  u32x4 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qb[ks] = row_ok ? *(const u32x4*)(a.q + qrow + ks * 16 + hi * 8) : u32x4{0u, 0u, 0u, 0u};

  // Keys below `cached` come from the cache: the prefix, or (KV8) every key
  // (never past the table's width; keys beyond it are masked out).
  const int cached = KV8 ? min(kend, cap) : P;
  const bool clipped = KV8 && kend > cached;
  // Stage their block ids (invalid ids become -1).
  const int nblk = (cached + (1 << a.bs_log2) - 1) >> a.bs_log2;
  const bool bt_in_lds = nblk <= kMaxBt;
  if (tid == 0) s_flags[0] = 0;
  __syncthreads();
  if (bt_in_lds) {
    bool bad = false;
    for (int i = tid; i < nblk; i += blockDim.x) {
      const int b = a.block_tables[(int64_t)seq * a.mbs + i];
      const bool ok = b >= 0 && b < a.num_blocks;
      s_bt[i] = ok ? b : -1;
      bad |= !ok;
    }
    if (bad) s_flags[0] = 1;
  }
  __syncthreads();
  const bool has_bad = bt_in_lds ? s_flags[0] != 0 : true;

  const int bs_mask = (1 << a.bs_log2) - 1;
  const int64_t kv_stride = (int64_t)a.Hkv * D;
  const int64_t head_off = (int64_t)kvh * D;
  auto block_of = [&](int kk) -> int {
    if (bt_in_lds) return s_bt[kk >> a.bs_log2];
    const int b = a.block_tables[(int64_t)seq * a.mbs + (kk >> a.bs_log2)];
    return (b >= 0 && b < a.num_blocks) ? b : -1;
  };

  // Byte offsets inside the tile area.  A buffer holds the K tile then the V
  // tile (TILE elements each); buffer 1 follows buffer 0.
  constexpr int TB = TILE * 2;         // bytes of one K or V tile
  constexpr int BUFB = 2 * TB;         // bytes of one buffer
  const char* lds = (const char*)tiles;

  // Loader: lane L of load `i` of this wave fills LDS chunk L of row
  // r_i = inst * RPI + L / CPR with global chunk (L % CPR) ^ swz(r_i).  The
  // lane's element offset inside a source row run is loop-invariant.
  int lrow[IPW];
  int lpart[IPW];  // (r_i * kv_stride + chunk * 8) in elements
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int inst = w * IPW + i;
    lrow[i] = inst * RPI + lane / CPR;
    lpart[i] = lrow[i] * (int)kv_stride + (((lane % CPR) ^ swz<D>(lrow[i])) * 8);
  }
  const int bsz = 1 << a.bs_log2;

  // Issue the direct-to-LDS loads of tile j.  Uniform fast paths: a tile that
  // lies inside one cache block, or wholly among the new tokens, has one base
  // address plus the lane's fixed offset.  Otherwise each lane resolves its
  // own key; keys past kend or in an invalid block fetch the first new token's
  // row (valid, finite) and the softmax masks them.
  auto issue_tile = [&](int j, int buf) {
    char* kdst = (char*)tiles + buf * BUFB;
    char* vdst = kdst + TB;
    const int k0 = j * kBN;
    const uint16_t* kbase = nullptr;
    const uint16_t* vbase = nullptr;
    if (k0 + kBN <= P && bsz >= kBN) {
      const int b = block_of(k0);
      if (b >= 0) {
        const int64_t o = (((int64_t)b << a.bs_log2) + (k0 & bs_mask)) * kv_stride + head_off;
        kbase = a.k_cache + o;
        vbase = a.v_cache + o;
      }
    } else if (k0 >= P && k0 + kBN <= kend) {
      const int64_t o = (int64_t)(qa + k0 - P) * kv_stride + head_off;
      kbase = a.k_new + o;
      vbase = a.v_new + o;
    }
    if (kbase != nullptr) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int inst = w * IPW + i;
        // (named pointers: an arithmetic expression as the builtin's argument
        // makes the host pass silently drop the kernel's launch stub)
        const uint16_t* kp = kbase + lpart[i];
        const uint16_t* vp = vbase + lpart[i];
        __builtin_amdgcn_global_load_lds(kp, (__attribute__((address_space(3))) void*)(kdst + inst * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp, (__attribute__((address_space(3))) void*)(vdst + inst * 1024), 16, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int inst = w * IPW + i;
      const int r = lrow[i];
      const int kk = k0 + r;
      int64_t off = (int64_t)qa * kv_stride + head_off;
      bool fresh = true;
      if (kk < P) {
        const int b = block_of(kk);
        if (b >= 0) {
          off = (((int64_t)b << a.bs_log2) + (kk & bs_mask)) * kv_stride + head_off;
          fresh = false;
        }
      } else if (kk < kend) {
        off = (int64_t)(qa + kk - P) * kv_stride + head_off;
      }
      off += lpart[i] - r * (int)kv_stride;  // the lane's chunk within the row
      const uint16_t* ks = (fresh ? a.k_new : a.k_cache) + off;
      const uint16_t* vs = (fresh ? a.v_new : a.v_cache) + off;
      __builtin_amdgcn_global_load_lds(ks, (__attribute__((address_space(3))) void*)(kdst + inst * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vs, (__attribute__((address_space(3))) void*)(vdst + inst * 1024), 16, 0, 0);
    }
  };

  // KV8 tile loader: thread tid holds 16 codes (one 16-byte load) of rows
  // tid / CPR8 + R8 i of the K and of the V tile, columns 16 (tid % CPR8) .. + 15;
  // keys past `cached` or in an unmapped block get zero codes.
  constexpr int CPR8 = D / 16;                 // 16-byte code chunks per row
  constexpr int R8 = 256 / CPR8;               // rows per pass
  constexpr int NP8 = KV8 ? kBN / R8 : 1;      // passes per tile
  u32x4 k8r[NP8], v8r[NP8];
  auto load_tile8 = [&](int j) {
#pragma unroll
    for (int i = 0; i < NP8; ++i) {
      const int kk = j * kBN + tid / CPR8 + R8 * i;
      const int b = kk < cached ? block_of(kk) : -1;
      const int64_t off = b < 0 ? 0
          : (((int64_t)b << a.bs_log2) + (kk & bs_mask)) * kv_stride + head_off + (tid % CPR8) * 16;
      const u32x4 kv = *(const u32x4*)((const char*)a.k_cache + off);
      const u32x4 vv = *(const u32x4*)((const char*)a.v_cache + off);
      k8r[i] = b < 0 ? u32x4{0u, 0u, 0u, 0u} : kv;
      v8r[i] = b < 0 ? u32x4{0u, 0u, 0u, 0u} : vv;
    }
  };
  auto store_tile8 = [&](int buf) {
    char* kdst = (char*)tiles + buf * (4 * TILE);
    char* vdst = kdst + TILE * 2;
#pragma unroll
    for (int i = 0; i < NP8; ++i) {
      const int r = tid / CPR8 + R8 * i;
      const int c0 = 2 * (tid % CPR8);
      const u32x4 src[2] = {k8r[i], v8r[i]};
      char* dst[2] = {kdst, vdst};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t w[4] = {src[t].x, src[t].y, src[t].z, src[t].w};
        uint32_t bf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf[2 * e] = fp8x2_to_bf16x2<false>(w[e]);
          bf[2 * e + 1] = fp8x2_to_bf16x2<true>(w[e]);
        }
        *(u32x4*)(dst[t] + r * D * 2 + ((c0 ^ swz<D>(r)) * 16)) = u32x4{bf[0], bf[1], bf[2], bf[3]};
        *(u32x4*)(dst[t] + r * D * 2 + (((c0 + 1) ^ swz<D>(r)) * 16)) =
            u32x4{bf[4], bf[5], bf[6], bf[7]};
      }
    }
  };

  // Operand read offsets.  K operand of (kt, ks): row 32 kt + lr, chunk
  // 2 ks + hi; V^T operand of (s, dt, rd): row 16 s + 4 hi + 8 rd + i16 / 4,
  // element 32 dt + 16 ((lane >> 4) & 1) + 4 (i16 & 3).  The swizzle only
  // depends on the row modulo 16, which kt and s do not change, so every
  // offset is a per-lane base (computed once here) plus a constant.
  int kofs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int r = lr;
    kofs[ks] = r * D * 2 + (((2 * ks + hi) ^ swz<D>(r)) * 16);
  }
  int vofs[DT][2];
  {
    const int i16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) {
        const int r = 4 * hi + 8 * rd + (i16 >> 2);
        const int dcol = dt * 32 + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
        vofs[dt][rd] = TB + r * D * 2 + (((dcol >> 3) ^ swz<D>(r)) * 16) + (dcol & 7) * 2;
      }
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float l_part = 0.f;  // this lane's half of the row's softmax denominator
  float m_run = kNegBig;  // running max (raw score units) of this lane's row
  const float c = a.scale_log2e;

  auto compute_tile = [&](int j, int bufoff) {
    // S^T = K Q^T for the two 32-key halves of the tile.
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    u32x4 ka[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) ka[ks][kt] = *(const u32x4*)(lds + bufoff + kofs[ks] + kt * 32 * D * 2);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) sacc[kt] = mfma32(ka[ks][kt], qb[ks], sacc[kt]);
    }
    // Keep 8 K operand reads in flight ahead of the MFMAs (left alone, the
    // scheduler waits on each pair of reads before its two MFMAs; all 16
    // ahead does not fit in the registers of two waves per SIMD).
    constexpr int kAhead = 2 * KS < 8 ? 2 * KS : 8;
#pragma unroll
    for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
#pragma unroll
    for (int i = 0; i < 2 * KS - kAhead; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    // Mask keys past this row's position (and keys of invalid blocks).
    const int k0 = j * kBN;
    if (k0 + kBN - 1 > P + t0 || has_bad || clipped) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = k0 + kt * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          bool ok = kk <= pos && (!clipped || kk < cached);
          if (has_bad && kk < cached) ok = ok && block_of(kk) >= 0;
          sacc[kt][i] = ok ? sacc[kt][i] : -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
    }
    mx = halves_max(mx);
    // Lazy rescale: keep the stale max unless it grew by more than 2^8.
    const bool grow = (mx - m_run) * c > kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      l_part *= alpha;
    }
    const float mc = m_run * c;
    u32x4 pb[4];  // P^T operands of the four 16-key steps, bf16
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s4 >> 1][(s4 & 1) * 8 + 2 * e], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s4 >> 1][(s4 & 1) * 8 + 2 * e + 1], c, -mc));
        wv[e] = pack_bf16(p0, p1);
      }
      pb[s4] = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
    // O^T += V^T P^T and l += the same bf16 weights.  The V^T operand of lane l is column
    // 32 dt + (l & 31) at keys 16 s + {4 hi .. 4 hi + 3, 8 + 4 hi .. 8 + 4 hi + 3},
    // gathered by two transposing reads: source lane i of a 16-lane group reads
    // row (kb + i / 4), elements dbase + 4 (i % 4) .. + 3.
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        short4_t part[2];
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
          const char* src = lds + bufoff + vofs[dt][rd] + s4 * 16 * D * 2;
          part[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (short4_t __attribute__((address_space(3)))*)src);
        }
        const u32x4 va = __builtin_bit_cast(u32x4, short8_t{part[0][0], part[0][1], part[0][2],
                                                            part[0][3], part[1][0], part[1][1],
                                                            part[1][2], part[1][3]});
        oacc[dt] = mfma32(va, pb[s4], oacc[dt]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) l_part = dot2_bf16(pb[s4][e], 0x3F803F80u, l_part);
    }
  };

  // The operand offsets point into buffer (j & 1): flipping the buffer bit of
  // every offset after each tile keeps the reads at "register + constant".
  // BUFB is a power of two larger than every in-buffer offset.
  if constexpr (KV8) {
    load_tile8(0);
    store_tile8(0);
  } else {
    issue_tile(0, 0);
  }
  for (int j = 0; j < ntiles; ++j) {
    if constexpr (!KV8)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile j are in LDS
    __syncthreads();                       // ... and every wave's; the other buffer is free again
    if (j + 1 < ntiles) {
      if constexpr (KV8) load_tile8(j + 1);
      else issue_tile(j + 1, (j + 1) & 1);
    }
    compute_tile(j, 0);
    if constexpr (KV8) {
      if (j + 1 < ntiles) store_tile8((j + 1) & 1);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kofs[ks] ^= BUFB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      vofs[dt][0] ^= BUFB;
      vofs[dt][1] ^= BUFB;
    }
  }

  const float l_tot = halves_sum(l_part);
  if (!row_ok) return;
  const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * (KV8 ? a.v_scale : 1.f);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = dt * 32 + 8 * g4 + 4 * hi;
      const float o0 = oacc[dt][4 * g4] * inv, o1 = oacc[dt][4 * g4 + 1] * inv;
      const float o2 = oacc[dt][4 * g4 + 2] * inv, o3 = oacc[dt][4 * g4 + 3] * inv;
      if (a.out_f32) {
        *(float4*)((float*)a.out + qrow + d) = make_float4(o0, o1, o2, o3);
      } else {
        *(uint2*)((uint16_t*)a.out + qrow + d) = make_uint2(pack_bf16(o0, o1), pack_bf16(o2, o3));
      }
    }
  }
}

template <int D>
constexpr size_t prefill_smem_bytes() {
  return (size_t)4 * kBN * D * sizeof(uint16_t) + (kMaxBt + 4) * sizeof(int);
}

template <int D, bool KV8>
int launch_prefill_d(const PrefillArgs& a, int tt_tokens, int ntt, int64_t nwg,
                     hipStream_t stream) {
  const int ranked = (int64_t)a.B * ntt <= kOrderMaxItems;
  constexpr size_t smem = prefill_smem_bytes<D>();
  // More than 64 KiB of dynamic LDS must be allowed once per device.
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(configured.load() & bit)) {
    if (hipFuncSetAttribute((const void*)paged_prefill_kernel<D, KV8>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
      return -1;
    configured.fetch_or(bit);
  }
  hipLaunchKernelGGL((paged_prefill_kernel<D, KV8>), dim3((unsigned)nwg), dim3(256), smem, stream,
                     a, tt_tokens, ntt, ranked);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_paged_prefill(const PrefillArgs& a, int head_dim, bool kv8, hipStream_t stream) {
  if (a.group > kRows) return -3;
  const int tt_tokens = kRows / a.group;
  const int ntt = (a.max_q_len + tt_tokens - 1) / tt_tokens;
  const int64_t nwg = (int64_t)ntt * a.B * a.Hkv;
  if (nwg == 0) return 0;
  if (nwg > INT32_MAX) return -2;
  if (head_dim == 128)
    return kv8 ? launch_prefill_d<128, true>(a, tt_tokens, ntt, nwg, stream)
               : launch_prefill_d<128, false>(a, tt_tokens, ntt, nwg, stream);
  if (head_dim == 64)
    return kv8 ? launch_prefill_d<64, true>(a, tt_tokens, ntt, nwg, stream)
               : launch_prefill_d<64, false>(a, tt_tokens, ntt, nwg, stream);
  return -3;
}

}  // namespace pa
