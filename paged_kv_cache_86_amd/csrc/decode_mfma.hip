// Paged decode on bf16 MFMA for large query-head groups (GQA), gfx950.
//
// Same operation, split-K decomposition and partial layout as the VALU decode
// kernel (MinivLLM guide "vLLM 技术路线", Step 4 §4.5-4.6; "Nano-vLLM源码学习(2)"
// §2): one workgroup per (sequence, KV head [sub-group], split), partials
// merged by the same combine kernel.  What changes is the arithmetic: with G
// query heads per KV head the VALU kernel spends about 2.7 G vector operations
// per K/V element, which for G >= 4 is more than the vector units can retire
// at HBM speed, so here both contractions of a split run on
// v_mfma_f32_16x16x32_bf16 with the G heads as one 16-wide operand side:
//
//   * S^T = K Q^T per 16-key tile; Q^T sits in registers for the whole split
//     (heads past G are zero);
//   * the softmax is per lane: lane l holds query head l % 16 and four keys of
//     each tile, and the row max takes two exchanges;
//   * O^T = V^T P^T: P^T comes from the S^T registers (bf16);
//   * K and V rows are loaded from the cache as whole 256-byte rows (four
//     rows per 64-lane load, the fully coalesced pattern), then pass through a
//     per-wave LDS area (16-byte chunks XOR-swizzled by row): K comes back in
//     the MFMA operand layout (ds_read_b128), V transposed
//     (ds_read_b64_tr_b16); the 32 keys of a chunk map to the MFMA's 32
//     contraction slots in the same (permuted) order on both operands;
//   * the softmax denominator is a third MFMA of P^T against ones, so it sums
//     exactly the bf16 weights the PV product uses.
//
// Masked keys (past the split's last cached token, or in a block the table
// does not map) get score -inf and read the query head's row instead of the
// cache (zeroed for KV8), so that p = 0 multiplies finite values.
//
// KV8 reads an FP8 (OCP E4M3) cache: a row of one head is D codes, a 16-byte
// load carries 16 of them, and they are widened exactly to bf16 (scale 1) on
// their way into the LDS area, so the MFMA part is unchanged; the per-tensor
// K scale is folded into the score scale and the V scale multiplies the merged
// outputs.  The fused store quantizes the new row exactly as the store kernel
// does, and the new token is attended with the values its codes decode to.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kW = 4;             // waves per workgroup
constexpr int kCK = 32;           // keys per wave chunk: two 16-key MFMA tiles
constexpr int kQR = 16;           // query heads per workgroup (one MFMA side)

__device__ __forceinline__ f32x4_t mfma16(const u32x4& a, const u32x4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}

// 16-byte chunk position of chunk c of staged V row r (XOR swizzle over the
// row's chunks, so the row-wise writes and the transposing reads both spread
// over the LDS banks).
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}

// One workgroup = one (sequence, head sub-group, split of S = kW * NCH * kCK
// tokens); wave w takes chunks w, w + 4, ...  DEPTH chunks of K and V are in
// flight per wave.  Three waves per SIMD (at most 168 registers per lane).
template <int D, int NCH, int DEPTH, bool KV8, bool APPEND, bool SCALAR_BLK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void paged_decode_mfma_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;           // 32-dim contraction steps of S^T
  constexpr int DT = D / 16;           // 16-dim tiles of O^T
  constexpr int EPL = KV8 ? 16 : 8;    // cache elements per 16-byte load
  constexpr int LPR = D / EPL;         // lanes per cache row of one head
  constexpr int RPI = 64 / LPR;        // rows per 64-lane load
  constexpr int NVL = kCK / RPI;       // K (and V) row loads per lane per chunk
  constexpr int EB = KV8 ? 1 : 2;      // bytes per cache element
  constexpr int S = kW * NCH * kCK;    // tokens per split
  constexpr int VROW = D * 2;          // bytes of a staged V row
  constexpr int VAREA = kCK * VROW;    // bytes of one wave's V area
  constexpr int NLB = D / 8;           // 16-byte vectors of a new K (or V) row
  static_assert(DEPTH >= 1 && DEPTH <= NCH, "prefetch depth");
  constexpr int OROW = D + 4;          // floats per head row of the merge area (padded:
                                       // the 16 heads of a write land on distinct banks)
  constexpr int LDS_V = kW * VAREA;
  constexpr int LDS_O = kW * kQR * OROW * 4;

  // V staging during the loop; the per-wave unnormalised O for the merge afterwards.
  __shared__ __align__(16) char s_v[LDS_V > LDS_O ? LDS_V : LDS_O];
  __shared__ int s_blk[SCALAR_BLK ? 1 : S];  // staged block ids of the split (block size >= 1)
  __shared__ float s_m[kW][kQR];
  __shared__ float s_l[kW][kQR];

  const int bid = blockIdx.x;
  int hg, split, seq;
  // Compacted items as in the VALU kernel; not in the bf16 fused-store
  // variant with block ids in scalars, which is at its 168-register limit
  // without the lookup.
  constexpr bool kCompactOk = KV8 || !APPEND || !SCALAR_BLK;
  if (kCompactOk && a.compact) {
    const int item = bid / a.hg;
    hg = bid - item * a.hg;
    if (!decode_work_item<kCompactPerLane>(a, item, S, false, seq, split)) return;
  } else {
    // Split-major from the last split slot down, as in the VALU kernel (a
    // 512-sequence 7B-shaped decode: 951 us in index order, 809 us first
    // split first, 800 us last slot first).
    hg = bid % a.hg;
    const int rest = bid / a.hg;
    const int blk = rest / a.batch;
    seq = rest - blk * a.batch;
    split = a.nsplit_max - 1 - blk;
  }
  const int kvh = hg / a.nsub;
  const int sub = hg - kvh * a.nsub;
  const int gt = (a.group + a.nsub - 1) / a.nsub;  // heads per sub-group (partial stride)
  const int h0 = kvh * a.group + sub * gt;
  const int gh = min(gt, a.group - sub * gt);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int qr = lane & 15;   // this lane's query head (MFMA column)
  const int g = lane >> 4;    // this lane's 8-slot group of the contraction
  const int t0 = split * S;
  const int b0 = t0 >> a.bs_log2;
  const int32_t* trow = a.block_tables + (int64_t)seq * a.mbs;

  // Issued before the context length is known: block ids and q.
  int blk0 = -1;
  if constexpr (SCALAR_BLK) {
    const int b = b0 < a.mbs ? trow[b0] : -1;
    blk0 = (b >= 0 && b < a.num_blocks) ? b : -1;
  } else {
    const int nb = S >> a.bs_log2;
#pragma unroll
    for (int k = 0; k < (S + 255) / 256; ++k) {
      const int i = tid + 256 * k;
      if (i < nb) {
        const int b = b0 + i < a.mbs ? trow[b0 + i] : -1;
        s_blk[i] = (b >= 0 && b < a.num_blocks) ? b : -1;
      }
    }
  }
  // Q^T operand of step ks: dims 32 ks + 8 g .. + 7 of head h0 + qr (zero past the group).
  const uint16_t* qhead = a.q + ((int64_t)seq * a.Hq + h0 + min(qr, gh - 1)) * D;
  u32x4 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 v = *(const u32x4*)(qhead + 32 * ks + 8 * g);
    qb[ks] = qr < gh ? v : u32x4{0u, 0u, 0u, 0u};
  }
  int ctx = a.context_lens[seq];
  const int cap = a.mbs << a.bs_log2;
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int nsplit = ctx == 0 ? 1 : (ctx + S - 1) / S;

  // APPEND: threads 0 .. 2*NLB-1 copy one 16-byte vector of the new K (V) row of
  // this KV head into the sequence's slot (head sub-group 0 only).  Loaded
  // here, at the end of one workgroup per sequence, to keep registers free.
  auto store_new = [&]() {
    const bool new_is_v = tid >= NLB;
    const int new_c = new_is_v ? tid - NLB : tid;
    if (tid < 2 * NLB && sub == 0) {
      const int slot = a.slot_mapping[seq];
      if (slot >= 0 && (int64_t)slot < a.num_slots) {
        const uint16_t* src = new_is_v ? a.v_new : a.k_new;
        const u32x4 x = *(const u32x4*)(src + ((int64_t)seq * a.Hkv + kvh) * D + new_c * 8);
        const int64_t dst = ((int64_t)slot * a.Hkv + kvh) * D + new_c * 8;  // element index
        if constexpr (KV8)
          *(u32x2*)((char*)(new_is_v ? a.v_cache_w : a.k_cache_w) + dst) =
              quantize8(x, new_is_v ? a.qscale_v : a.qscale_k);
        else
          *(u32x4*)((uint16_t*)(new_is_v ? a.v_cache_w : a.k_cache_w) + dst) = x;
      }
    }
  };
  if (ctx == 0) {  // padded row: output zeros
    if constexpr (APPEND) {
      if (split == 0 && w == 0) store_new();
    }
    if (split == 0) {
      for (int i = tid; i < gh * D; i += blockDim.x) {
        const int64_t o = ((int64_t)seq * a.Hq + h0) * D + i;
        if (a.out_f32) ((float*)a.out)[o] = 0.f;
        else ((uint16_t*)a.out)[o] = 0;
      }
    }
    return;
  }
  if (split >= nsplit) return;
  // Cached tokens of this split: t0 .. t1-1 (with APPEND position ctx-1 comes
  // from k_new / v_new, and its cache row may not be written yet).  Keys past
  // t1 are masked out and read the query head instead (finite).
  const int tc = APPEND ? ctx - 1 : ctx;
  const int t1 = min(tc, t0 + S);
  if constexpr (!SCALAR_BLK) __syncthreads();  // s_blk written

  const int64_t row_stride = (int64_t)a.Hkv * D;
  const int bs_mask = (1 << a.bs_log2) - 1;
  // Element offset of key j's row of this KV head, or -1 when its block is unmapped.
  auto row_of = [&](int j) -> int64_t {
    const int blk = SCALAR_BLK ? blk0 : s_blk[(j >> a.bs_log2) - b0];
    if (blk < 0) return -1;
    return (((int64_t)blk << a.bs_log2) + (j & bs_mask)) * row_stride + (int64_t)kvh * D;
  };
  // Unmapped rows are read from the query head instead (finite, also as FP8
  // codes; masked out).
  auto kv_ptr = [&](const uint16_t* base, int64_t row, int elem) -> const u32x4* {
    return row >= 0 ? (const u32x4*)((const char*)base + (row + elem) * EB)
                    : (const u32x4*)((const char*)qhead + elem * EB);
  };

  char* vmine = s_v + w * VAREA;
  // LDS byte offsets of this lane's row chunk writes (K, then V, of a chunk),
  // of its K operand reads (row 16 kt + qr, chunk 4 ks + g; the swizzle does
  // not depend on kt), and of its transposing V reads: read rd of tile dt
  // returns column 16 dt + qr at keys 16 rd + 4 g .. + 3.
  // (KV8: a load's 16 codes become two 16-byte bf16 chunks, 2c and 2c + 1.)
  constexpr int CPL = KV8 ? 2 : 1;
  int vw_off[NVL][CPL];
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int r = i * RPI + lane / LPR;
#pragma unroll
    for (int h = 0; h < CPL; ++h)
      vw_off[i][h] = r * VROW + ((((lane % LPR) * CPL + h) ^ vswz<D>(r)) * 16);
  }
  // Row chunks of a load into the wave's LDS area (widened for KV8; rows that
  // came from the query head instead of the cache are zeroed, since its bytes
  // read as E4M3 codes may be NaN).
  auto put_rows = [&](const u32x4 (&rows)[NVL], uint32_t ok) {
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      if constexpr (KV8) {
        const bool oki = (ok >> i) & 1u;
        const uint32_t cw[4] = {oki ? rows[i].x : 0u, oki ? rows[i].y : 0u, oki ? rows[i].z : 0u,
                                oki ? rows[i].w : 0u};
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b[2 * e] = fp8x2_to_bf16x2<false>(cw[e]);
          b[2 * e + 1] = fp8x2_to_bf16x2<true>(cw[e]);
        }
        *(u32x4*)(vmine + vw_off[i][0]) = u32x4{b[0], b[1], b[2], b[3]};
        *(u32x4*)(vmine + vw_off[i][1]) = u32x4{b[4], b[5], b[6], b[7]};
      } else {
        *(u32x4*)(vmine + vw_off[i][0]) = rows[i];
      }
    }
  };
  int kr_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kr_off[ks] = qr * VROW + (((4 * ks + g) ^ vswz<D>(qr)) * 16);
  // The transposing read of (dt, rd) starts at element 16 dt + 4 (qr & 3) of row r:
  // chunk 2 dt + ((qr & 3) >> 1), element (qr & 1) * 4; with the swizzle that is
  // vr_base[rd] + ((2 dt ^ vr_swz[rd]) << 4) (2 dt has no bit 0).
  int vr_base[2], vr_swz[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int r = 16 * rd + 4 * g + (qr >> 2);
    const int sw = vswz<D>(r);
    vr_base[rd] = r * VROW + ((((qr & 3) >> 1) ^ (sw & 1)) << 4) + (qr & 1) * 8;
    vr_swz[rd] = sw & ~1;
  }

  struct Chunk {
    u32x4 k[NVL];  // K rows i * RPI + lane / LPR, chunk lane % LPR
    u32x4 v[NVL];  // V rows, the same
    uint32_t ok;   // bit i: row i came from the cache (KV8 only)
  };
  auto load_chunk = [&](int it, Chunk& ch) {
    const int k0 = t0 + (it * kW + w) * kCK;
    ch.ok = 0;
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int j = k0 + i * RPI + lane / LPR;
      const int64_t row = j < t1 ? row_of(j) : -1;
      if constexpr (KV8) ch.ok |= (row >= 0 ? 1u : 0u) << i;
      ch.k[i] = __builtin_nontemporal_load(kv_ptr(a.k_cache, row, (lane % LPR) * EPL));
      ch.v[i] = __builtin_nontemporal_load(kv_ptr(a.v_cache, row, (lane % LPR) * EPL));
    }
  };

  f32x4_t oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegBig;  // running max (log2 units) of this lane's query head
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0

  // `refill` runs once the chunk's rows are in LDS (its registers are free).
  auto compute_chunk = [&](int it, const Chunk& ch, auto&& refill) {
    const int k0 = t0 + (it * kW + w) * kCK;
    // K rows through this wave's LDS area into the operand layout, then V rows
    // (read back transposed below; the wave's LDS accesses stay in order).
    put_rows(ch.k, ch.ok);
    f32x4_t sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ka = *(const u32x4*)(vmine + kr_off[ks] + kt * 16 * VROW);
        sacc[kt] = mfma16(ka, qb[ks], sacc[kt]);
      }
    }
    put_rows(ch.v, ch.ok);
    refill();
    // Scores of keys k0 + 16 kt + 4 g + e (log2 units), masked to -inf.
    float s[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = k0 + 16 * kt + 4 * g + e;
        bool ok = j < t1;
        if constexpr (SCALAR_BLK) ok = ok && blk0 >= 0;
        else ok = ok && s_blk[(j >> a.bs_log2) - b0] >= 0;
        s[kt][e] = ok ? mul_rn(sacc[kt][e], a.scale_log2e) : -INFINITY;
        mx = fmaxf(mx, s[kt][e]);
      }
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    if (__builtin_amdgcn_ballot_w64(mnew > m) != 0) {  // alpha == 1 exactly otherwise
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      lacc *= alpha;
      m = mnew;
    }
    // P^T operand: contraction slots 8 g .. 8 g + 3 are keys 4 g .. + 3 of tile 0,
    // slots 8 g + 4 .. + 7 keys 16 + 4 g .. + 3 (tile 1).
    const u32x4 pb = {
        pack_bf16(__builtin_amdgcn_exp2f(s[0][0] - m), __builtin_amdgcn_exp2f(s[0][1] - m)),
        pack_bf16(__builtin_amdgcn_exp2f(s[0][2] - m), __builtin_amdgcn_exp2f(s[0][3] - m)),
        pack_bf16(__builtin_amdgcn_exp2f(s[1][0] - m), __builtin_amdgcn_exp2f(s[1][1] - m)),
        pack_bf16(__builtin_amdgcn_exp2f(s[1][2] - m), __builtin_amdgcn_exp2f(s[1][3] - m))};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      short4_t part[2];
#pragma unroll
      for (int rd = 0; rd < 2; ++rd)
        part[rd] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (short4_t __attribute__((address_space(3)))*)(vmine + vr_base[rd] +
                                                           (((2 * dt) ^ vr_swz[rd]) << 4)));
      const u32x4 va = __builtin_bit_cast(
          u32x4, short8_t{part[0][0], part[0][1], part[0][2], part[0][3], part[1][0], part[1][1],
                          part[1][2], part[1][3]});
      oacc[dt] = mfma16(va, pb, oacc[dt]);
    }
    lacc = mfma16(ones, pb, lacc);
  };

  // Chunks in groups of DEPTH (a loop: unrolled over all NCH chunks, the
  // compiler keeps more chunks' rows live than the registers of three waves
  // per SIMD hold); buffer d serves chunks it0 + d and is refilled with chunk
  // it0 + d + DEPTH as soon as its rows are staged in LDS, so at most DEPTH
  // chunks are held in registers.
  static_assert(NCH % DEPTH == 0, "whole groups of DEPTH chunks");
  Chunk buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_chunk(d, buf[d]);
#pragma unroll 1
  for (int it0 = 0; it0 < NCH; it0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      compute_chunk(it0 + d, buf[d], [&]() {
        if (it0 + d + DEPTH < NCH) load_chunk(it0 + d + DEPTH, buf[d]);
      });
    }
  }

  // APPEND: wave 0 of the sequence's last split folds in the new token
  // (position ctx - 1) from k_new / v_new, and writes it to its slot.
  if constexpr (APPEND) {
    if (split == nsplit - 1 && w == 0) {
      store_new();
      const uint16_t* kn = a.k_new + ((int64_t)seq * a.Hkv + kvh) * D;
      const uint16_t* vn = a.v_new + ((int64_t)seq * a.Hkv + kvh) * D;
      float d = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 kx = *(const u32x4*)(kn + 32 * ks + 8 * g);
        if constexpr (KV8) {  // the values its codes decode to (unscaled, exact in bf16)
          const u32x2 cw = quantize8(kx, a.qscale_k);
          kx = u32x4{fp8x2_to_bf16x2<false>(cw.x), fp8x2_to_bf16x2<true>(cw.x),
                     fp8x2_to_bf16x2<false>(cw.y), fp8x2_to_bf16x2<true>(cw.y)};
        }
        d = dot2_bf16(qb[ks].x, kx.x, d);
        d = dot2_bf16(qb[ks].y, kx.y, d);
        d = dot2_bf16(qb[ks].z, kx.z, d);
        d = dot2_bf16(qb[ks].w, kx.w, d);
      }
      d += shfl_xor(d, 16);
      d += shfl_xor(d, 32);
      const float sn = mul_rn(d, a.scale_log2e);
      const float mnew = fmaxf(m, sn);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      const float p = __builtin_amdgcn_exp2f(sn - mnew);
      m = mnew;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x2 vx = *(const u32x2*)(vn + 16 * dt + 4 * g);
        float vf[4] = {bf16lo(vx.x), bf16hi(vx.x), bf16lo(vx.y), bf16hi(vx.y)};
        if constexpr (KV8) {
          const uint32_t c2 = fp8_code_pair(vf[0], vf[1], a.qscale_v) |
                              (fp8_code_pair(vf[2], vf[3], a.qscale_v) << 16);
          const float2_t lo = fp8x2_to_f32x2<false>(c2), hi = fp8x2_to_f32x2<true>(c2);
          vf[0] = lo.x;
          vf[1] = lo.y;
          vf[2] = hi.x;
          vf[3] = hi.y;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[dt][e] = fmaf(p, vf[e], oacc[dt][e] * alpha);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) lacc[e] = fmaf(lacc[e], alpha, p);
    }
  }

  // Merge the four waves: (m, l) per head in s_m / s_l, unnormalised O^T in the
  // V areas (reused: [wave][head][dim] floats, rows padded).
  __syncthreads();  // every wave is done with its V area
  float* s_o = (float*)s_v;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s_o[(w * kQR + qr) * OROW + 16 * dt + 4 * g + e] = oacc[dt][e];
  }
  if (g == 0) {
    s_m[w][qr] = m;
    s_l[w][qr] = lacc[0];
  }
  __syncthreads();

  const int64_t unit = (int64_t)seq * a.hg + hg;
  for (int i = tid; i < gh * D; i += blockDim.x) {
    const int h = i / D;
    const int dd = i - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kW; ++ww) M = fmaxf(M, s_m[ww][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) {
      const float f = __builtin_amdgcn_exp2f(s_m[ww][h] - M);
      L += s_l[ww][h] * f;
      O += s_o[(ww * kQR + h) * OROW + dd] * f;
    }
    if constexpr (KV8) O *= a.v_scale;
    if (nsplit == 1) {
      const int64_t o = ((int64_t)seq * a.Hq + h0 + h) * D + dd;
      const float val = L > 0.f ? O / L : 0.f;
      if (a.out_f32) ((float*)a.out)[o] = val;
      else ((uint16_t*)a.out)[o] = (uint16_t)f32_to_bf16_rne(val);
    } else {
      const int64_t p = (unit * a.nsplit_max + split) * gt + h;
      a.ws_o[p * D + dd] = O;
      if (dd == 0) {
        a.ws_ml[2 * p] = M;
        a.ws_ml[2 * p + 1] = L;
      }
    }
  }
}

// Production tilings.  Short splits: 2 chunks of 32 keys per wave (a split
// is 256 tokens), both in flight.  Long splits: 16 chunks per wave (2048
// tokens), one in flight (refilled as soon as the current chunk is staged
// in LDS; two held in registers would spill at three waves per SIMD).  The
// long split pays the workgroup's set-up, merge and partial write over 8x
// the tokens: 7B-shaped decode (256 sequences, 28/4 heads, block 16)
// 460 -> 386-389 us per step.
constexpr int kNch = 2;
constexpr int kNchLong = 16;
static_assert(kW * kNch * kCK == kMfmaSplitTokens, "short split length");
static_assert(kW * kNchLong * kCK == kMfmaLongSplitTokens, "long split length");
// Chunks in flight per wave in a short split: both for bf16 pools; one for
// FP8 pools, whose widening work per chunk already hides the load latency
// (7B-shaped FP8 decode: 292-298 -> 279-281 us; bf16 is level or slower with
// one).
constexpr int kDepth = 2;
constexpr int kDepthFp8 = 1;

// t_start / t_end (either may be null) are attached to the launch itself
// (hipExtLaunchKernel), so they carry the kernel's own start and end times.
template <int D, int NCH, int DEPTH, bool KV8, bool APPEND>
void launch_mfma_kernel(const DecodeArgs& a, unsigned nwg, hipStream_t stream, hipEvent_t t_start,
                        hipEvent_t t_end) {
  constexpr int S = kW * NCH * kCK;
  if ((1 << a.bs_log2) >= S)
    hipExtLaunchKernelGGL((paged_decode_mfma_kernel<D, NCH, DEPTH, KV8, APPEND, true>), dim3(nwg),
                          dim3(256), 0, stream, t_start, t_end, 0u, a);
  else
    hipExtLaunchKernelGGL((paged_decode_mfma_kernel<D, NCH, DEPTH, KV8, APPEND, false>),
                          dim3(nwg), dim3(256), 0, stream, t_start, t_end, 0u, a);
}

template <int D, bool KV8, bool APPEND>
int launch_mfma_d(const DecodeArgs& a, int B, hipStream_t stream) {
  const unsigned nwg = (unsigned)((int64_t)B * a.hg * a.nsplit_max);
  const bool long_split = (1 << a.split_log2) == kMfmaLongSplitTokens;
  if (!long_split && (1 << a.split_log2) != kMfmaSplitTokens) return -2;
  hipEvent_t t_start = nullptr, t_end = nullptr;
  take_decode_timing(&t_start, &t_end);
  if (long_split)
    launch_mfma_kernel<D, kNchLong, 1, KV8, APPEND>(a, nwg, stream, t_start, t_end);
  else
    launch_mfma_kernel<D, kNch, KV8 ? kDepthFp8 : kDepth, KV8, APPEND>(a, nwg, stream, t_start,
                                                                        t_end);
  if (hipGetLastError() != hipSuccess) return -1;
  const int gt = (a.group + a.nsub - 1) / a.nsub;
  return a.nsplit_max > 1 ? launch_decode_combine(a, B, D, gt, stream) : 0;
}

template <int D>
int launch_mfma_dd(const DecodeArgs& a, int B, bool kv8, bool append, hipStream_t stream) {
  if (kv8) return append ? launch_mfma_d<D, true, true>(a, B, stream)
                         : launch_mfma_d<D, true, false>(a, B, stream);
  return append ? launch_mfma_d<D, false, true>(a, B, stream)
                : launch_mfma_d<D, false, false>(a, B, stream);
}

}  // namespace

int launch_paged_decode_mfma(const DecodeArgs& a, int B, int head_dim, bool kv8, bool append,
                             hipStream_t stream) {
  if (head_dim == 128) return launch_mfma_dd<128>(a, B, kv8, append, stream);
  if (head_dim == 64) return launch_mfma_dd<64>(a, B, kv8, append, stream);
  return -2;
}

}  // namespace pa
