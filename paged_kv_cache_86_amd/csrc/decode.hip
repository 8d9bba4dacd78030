// Paged decode attention for gfx950: one query token per sequence reads its
// K/V through the block table (MinivLLM guide "vLLM 技术路线", Step 4 §4.5
// prepare_decode and §4.6 run_model; "Nano-vLLM源码学习(2)" §2, the decode
// path reads paged KV via block_table).
//
// Work decomposition (this library's design, not the pages'):
//   * one workgroup (4 waves) per (sequence, KV head [sub-group], split of
//     2^split_log2 tokens); all query heads sharing that KV head (GQA) are
//     served from the same K/V registers, so each K/V byte is read once;
//   * a wave walks chunks of U*RPW tokens: RPW rows per 64-lane load with
//     D/8 lanes per row, each lane loading 16 contiguous bytes (fully
//     coalesced 128-bit loads; a row of one head is D*2 contiguous bytes);
//   * q.k uses v_dot2_f32_bf16 on the packed bf16 pairs, reduced across the
//     lanes of a row with DPP; each row slot keeps its own online-softmax
//     state (running max, sum, fp32 accumulator) so the loop has no
//     cross-row traffic; states are merged once at the end (shuffles, then
//     LDS across waves);
//   * split-K partials (m, l, unnormalised o) go to the workspace and a
//     second, small kernel merges them in split order (deterministic); a
//     context that fits in one split writes its output directly;
//   * splits come in two lengths when the grid is large enough: a context
//     that would need more short splits than the grid has slots per sequence
//     takes splits of twice the length instead;
//   * the grid has a slot for every split of the longest possible context
//     (the host does not know the lengths); for batches of up to 256
//     sequences each workgroup looks its (sequence, split) up in the
//     compacted list of the splits that exist, and larger batches take their
//     slots split-major from the last slot down, so the empty slots do not
//     sit between the real ones all through the grid.  The
//     kernel boundary is what makes one XCD's partials visible to another:
//     an in-kernel "last workgroup merges" scheme needs a device-scope
//     release/acquire per workgroup, which on this chip writes back and
//     invalidates the whole L2 of an XCD and costs far more than a launch.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kMaxSplitBlocks = 512;  // short-split tokens / block size (block size >= 1)
constexpr float kStaleLog2 = 8.f;     // KV8: growth of a running max (exp2 units) that forces a rescale

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// {lo, hi} -> a bf16 pair, each rounded to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_v));
}

// One workgroup = one (sequence, head group, split).
//
// Splits.  A short split is S = kWaves * NIT chunks of U * RPW tokens (wave w
// takes chunks w, w + 4, ...).  With LONG, a context needing more than
// long_above short splits (nsplit_max, or 1 on FP8 pools) is cut into long
// splits of 2S tokens instead (at most nsplit_max of them), so
// one grid of nsplit_max workgroups per (sequence, head group) serves every
// context the table allows: short contexts leave fewer workgroups idle, long
// ones run fewer, longer workgroups (their per-workgroup set-up and merge are
// paid half as often).  The chunk loop is fully unrolled: a short split issues
// every load of the wave before the first is consumed (DEPTH == NIT); a long
// split keeps DEPTH chunks in flight, issuing chunk it + DEPTH as it consumes
// chunk it.
//
// KV8 selects an FP8 (OCP E4M3) cache: a 16-byte load then carries 16 codes
// instead of 8 bf16 values.  K codes are widened to bf16 pairs and take the
// same v_dot2 path as bf16 keys.  V: a lane holds U = 2 rows of each chunk;
// for each element its codes in the two rows are interleaved (v_perm) and
// widened to one bf16 pair, so a single v_dot2 per element and query head adds
// both rows' weighted values.  The weights p enter that product rounded to
// bf16 and the softmax denominator sums the same rounded weights (relative
// error of each weight at most 2^-9).  The per-tensor K scale is folded into
// the score scale and the V scale into the outputs.
//
// With KV8 a row slot's running max m may also go stale: scores are weighted
// by p = 2^(s - m) with m kept until some score of the wave exceeds its slot's
// m by more than 2^8 (exp2 units), and only then do the slots move to their
// true maxima and rescale l and the outputs.  The state (m, l, o) is valid for
// any m, p stays <= 256, and the merges below take each slot's own m.  (The
// bf16 kernel keeps the exact update: the branch costs it more registers than
// it saves.)
//
// APPEND fuses the store of each sequence's new token: position ctx-1 is not
// read from the cache but from k_new / v_new (quantized first for KV8, exactly
// as the store kernel does).  The first 2*D/8 lanes of wave 0 load the row at
// the start; after the main loop the workgroup of the split that holds the
// token passes it between lanes of wave 0 (no LDS, no barrier) and folds it
// into row slot 0's softmax state, and the one of head sub-group 0 writes it
// into its cache slot.
//
// SCALAR_BLK is set when a cache block holds at least one short split
// (block_size >= S): the split's block ids (one for a short split, two for a
// long one) are then scalar loads, with no LDS staging and no barrier before
// the K/V loads.  Otherwise the ids of the split are staged in LDS while the
// context length is still in flight (long splits need SCALAR_BLK).
template <int D, int GT, int U, int NIT, int DEPTH, int DEPTH_LONG, bool LONG, bool NT, bool KV8,
          bool APPEND, bool SCALAR_BLK>
__device__ __forceinline__ void paged_decode_body(const DecodeArgs& a) {
  constexpr int EB = KV8 ? 1 : 2;   // bytes per K/V element
  constexpr int EPL = 16 / EB;      // elements per lane per 16-byte load
  constexpr int LPR = D / EPL;      // lanes per K/V row of one head
  constexpr int RPW = 64 / LPR;     // rows per 64-lane load
  constexpr int QW = EPL / 8;       // 16-byte chunks of q per lane and head
  constexpr int CH = U * RPW;       // tokens per wave chunk
  constexpr int S = kWaves * NIT * CH;  // tokens per short split
  constexpr int SL = LONG ? 2 * S : S;  // tokens per long split
  constexpr bool PAIR_V = KV8 && U == 2;  // V rows of a lane as bf16 pairs (see above)
  static_assert(!LONG || SCALAR_BLK, "long splits read scalar block ids");

  __shared__ int s_blk[SCALAR_BLK ? 1 : kMaxSplitBlocks];
  __shared__ float s_m[kWaves][GT];
  __shared__ float s_l[kWaves][GT];
  __shared__ float s_acc[kWaves][GT][D];
  constexpr int NLB = D / 8;  // 16-byte bf16 vectors per new K (or V) row of one head

  const int bid = blockIdx.x;
  int hg, split, seq;
  if (a.compact) {
    // Item bid / hg of the compacted list (its head groups on consecutive
    // workgroups, as in index order); workgroups past the last item exit.
    int item = bid / a.hg;
    hg = bid - item * a.hg;
    if constexpr (KV8) {
      // FP8 pools: inside each whole group of 8 items x hg head groups,
      // workgroup r takes item r % 8 and head group r / 8.  Workgroups go to
      // the 8 XCDs round-robin, so an XCD then serves every head group of its
      // items instead of one head group of every item; with one head group per
      // XCD, the XCD holding one of them ran 10-15% behind the others.
      const int gsz = 8 * a.hg;
      const int g = bid / gsz;
      if ((g + 1) * gsz <= (int)gridDim.x) {
        const int r = bid - g * gsz;
        item = g * 8 + (r & 7);
        hg = r >> 3;
      }
    }
    if (!decode_work_item<kCompactPerLane>(a, item, S, LONG, seq, split)) return;
  } else {
    // Split-major from the last split slot down: every sequence's last slot,
    // then every second-to-last, ..., every first split at the end.  The
    // empty slots of short contexts are then gone early, between the longest
    // contexts' splits, instead of taking workgroup slots from real work all
    // through the grid, and the grid ends on the dense first splits (the
    // 512-sequence decode: 361-364 us in index order, 346-348 first split
    // first, 336 last slot first).
    hg = bid % a.hg;
    const int rest = bid / a.hg;
    const int blk = rest / a.batch;
    seq = rest - blk * a.batch;
    split = a.nsplit_max - 1 - blk;
  }
  const int kvh = hg / a.nsub;
  const int sub = hg - kvh * a.nsub;
  const int h0 = kvh * a.group + sub * GT;
  const int gh = min(GT, a.group - sub * GT);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int r = lane / LPR;
  const int c = lane - r * LPR;
  const int b0s = (split * S) >> a.bs_log2;   // first table entry of the short split
  const int b0l = (split * SL) >> a.bs_log2;  // ... and of the long one

  // Issued before the context length is known, so the loads overlap: the
  // table entries of both candidate splits (clamped to the table row), q, the
  // context length.
  const int32_t* trow = a.block_tables + (int64_t)seq * a.mbs;
  auto entry = [&](int b) -> int {
    int blk = -1;
    if (b < a.mbs) blk = trow[b];
    return (blk >= 0 && blk < a.num_blocks) ? blk : -1;
  };
  int blk_s = -1, blk_l0 = -1, blk_l1 = -1;
  if constexpr (SCALAR_BLK) {
    blk_s = entry(b0s);
    if constexpr (LONG) {
      blk_l0 = entry(b0l);
      blk_l1 = entry(b0l + 1);
    }
  } else {
    const int nbs = S >> a.bs_log2;
#pragma unroll
    for (int k = 0; k < kMaxSplitBlocks / 256; ++k) {
      const int i = tid + 256 * k;
      if (i < nbs) s_blk[i] = entry(b0s + i);
    }
  }
  // Heads past the group's end (last sub-group) re-read its last head; their
  // results are never stored.
  u32x4 qv[GT][QW];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    const int hh = h < gh ? h : gh - 1;
#pragma unroll
    for (int qw = 0; qw < QW; ++qw)
      qv[h][qw] = *(const u32x4*)(a.q + ((int64_t)seq * a.Hq + h0 + hh) * D + c * EPL + qw * 8);
  }
  // APPEND: threads 0 .. 2*NLB-1 fetch one 16-byte vector of the new K (V) row
  // of this KV head, and the sequence's slot.
  const bool new_lane = APPEND && tid < 2 * NLB;
  const bool new_is_v = tid >= NLB;
  const int new_c = new_is_v ? tid - NLB : tid;
  u32x4 xnew{};
  int slot = -1;
  if constexpr (APPEND) {
    if (new_lane) {
      const uint16_t* src = new_is_v ? a.v_new : a.k_new;
      xnew = *(const u32x4*)(src + ((int64_t)seq * a.Hkv + kvh) * D + new_c * 8);
      slot = a.slot_mapping[seq];
    }
  }
  int ctx = a.context_lens[seq];
  const int cap = a.mbs << a.bs_log2;
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  const int nshort = ctx == 0 ? 1 : (ctx + S - 1) / S;
  const bool lng = LONG && nshort > a.long_above;
  const int nsplit = lng ? (ctx + SL - 1) / SL : nshort;

  // APPEND: lanes 0 .. 2*NLB-1 of wave 0 write the new row (bf16, or E4M3
  // codes for KV8) into its slot when this is the sequence's last split and
  // head sub-group 0; every lane returns its vector (codes in .x, .y for KV8).
  auto store_new = [&]() -> u32x4 {
    u32x4 v = xnew;
    if constexpr (KV8) {
      const u32x2 cw = quantize8(xnew, new_is_v ? a.qscale_v : a.qscale_k);
      v = u32x4{cw.x, cw.y, 0u, 0u};
    }
    if (new_lane && sub == 0 && slot >= 0 && (int64_t)slot < a.num_slots) {
      const int64_t dst = ((int64_t)slot * a.Hkv + kvh) * D + new_c * 8;  // element index
      if constexpr (KV8) *(u32x2*)((char*)(new_is_v ? a.v_cache_w : a.k_cache_w) + dst) = u32x2{v.x, v.y};
      else *(u32x4*)((uint16_t*)(new_is_v ? a.v_cache_w : a.k_cache_w) + dst) = v;
    }
    return v;
  };

  if (ctx == 0) {  // padded row: output zeros
    if constexpr (APPEND) {
      if (split == 0 && w == 0) (void)store_new();
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
  // Cached tokens of this split are t0 .. t1-1 (with APPEND the last position
  // comes from k_new / v_new instead; t1 <= t0 when the split holds only it).
  // Loads past t1 re-read row `jfill`, which is in bounds and masked out.
  const int t0 = split * (lng ? SL : S);
  const int tc = APPEND ? ctx - 1 : ctx;
  const int t1 = min(tc, t0 + (lng ? SL : S));
  const int jfill = t1 > t0 ? t1 - 1 : t0;
  if constexpr (!SCALAR_BLK) __syncthreads();  // s_blk written

  const int64_t row_stride = (int64_t)a.Hkv * D;
  const int64_t head_off = (int64_t)kvh * D + c * EPL;  // elements
  const int bs_mask = (1 << a.bs_log2) - 1;

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  // Partial q.k of query head h over this lane's EPL elements of one K row.
  auto kdot = [&](int h, const u32x4& k) -> float {
    float d = 0.f;
    if constexpr (KV8) {
      const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
      const uint32_t qwv[8] = {qv[h][0].x, qv[h][0].y, qv[h][0].z, qv[h][0].w,
                               qv[h][QW - 1].x, qv[h][QW - 1].y, qv[h][QW - 1].z, qv[h][QW - 1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = dot2_bf16(qwv[2 * e], fp8x2_to_bf16x2<false>(kw[e]), d);
        d = dot2_bf16(qwv[2 * e + 1], fp8x2_to_bf16x2<true>(kw[e]), d);
      }
    } else {
      d = dot2_bf16(qv[h][0].x, k.x, d);
      d = dot2_bf16(qv[h][0].y, k.y, d);
      d = dot2_bf16(qv[h][0].z, k.z, d);
      d = dot2_bf16(qv[h][0].w, k.w, d);
    }
    return d;
  };
  // This lane's EPL elements of one V row as fp32.
  auto vconv = [&](const u32x4& v, float (&vf)[EPL]) {
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (KV8) {
        const float2_t lo = fp8x2_to_f32x2<false>(vw[e]);
        const float2_t hi = fp8x2_to_f32x2<true>(vw[e]);
        vf[4 * e] = lo.x;
        vf[4 * e + 1] = lo.y;
        vf[4 * e + 2] = hi.x;
        vf[4 * e + 3] = hi.y;
      } else {
        vf[2 * e] = bf16lo(vw[e]);
        vf[2 * e + 1] = bf16hi(vw[e]);
      }
    }
  };

  // Stream the split: NI chunks per wave, DP of them in flight.  IS_LONG picks
  // the long split's block ids.
  auto stream = [&](auto ni_c, auto dp_c, auto long_c) {
    constexpr int NI = decltype(ni_c)::value;
    constexpr int DP = decltype(dp_c)::value;
    constexpr bool IS_LONG = decltype(long_c)::value;
    static_assert(DP >= 1 && DP <= NI, "prefetch depth");
    const int b0 = IS_LONG ? b0l : b0s;
    auto load_chunk = [&](int it, u32x4 (&kc)[U], u32x4 (&vc)[U], bool (&ok)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // Rows past the split end re-read the split's last row (in bounds, finite) and
        // are masked out of the softmax below.
        const int j = t0 + (it * kWaves + w) * CH + u * RPW + r;
        const int jj = j < t1 ? j : jfill;
        int blk;
        if constexpr (SCALAR_BLK) {
          if constexpr (IS_LONG) blk = ((jj >> a.bs_log2) != b0) ? blk_l1 : blk_l0;
          else blk = blk_s;
        } else {
          blk = s_blk[(jj >> a.bs_log2) - b0];
        }
        ok[u] = (j < t1) && (blk >= 0);
        blk = blk < 0 ? 0 : blk;
        const int64_t off = (((int64_t)blk << a.bs_log2) + (jj & bs_mask)) * row_stride + head_off;
        const u32x4* kp = (const u32x4*)((const char*)a.k_cache + off * EB);
        const u32x4* vp = (const u32x4*)((const char*)a.v_cache + off * EB);
        if constexpr (NT) {
          kc[u] = __builtin_nontemporal_load(kp);
          vc[u] = __builtin_nontemporal_load(vp);
        } else {
          kc[u] = *kp;
          vc[u] = *vp;
        }
      }
    };

    u32x4 kpre[NI][U], vpre[NI][U];
    bool okpre[NI][U];
#pragma unroll
    for (int it = 0; it < DP; ++it) load_chunk(it, kpre[it], vpre[it], okpre[it]);

#pragma unroll
    for (int it = 0; it < NI; ++it) {
      if (it + DP < NI) load_chunk(it + DP, kpre[it + DP], vpre[it + DP], okpre[it + DP]);
      u32x4 kc[U], vc[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        kc[u] = kpre[it][u];
        vc[u] = vpre[it][u];
        ok[u] = okpre[it][u];
      }

      float s[U][GT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const float d = group_sum<LPR>(kdot(h, kc[u]));
          // mul_rn: the score is rounded once and the same value is compared
          // with and subtracted from the running max (the maximum gives p = 1).
          s[u][h] = ok[u] ? mul_rn(d, a.scale_log2e) : -INFINITY;
        }
      }
      uint32_t pp[GT];  // PAIR_V: the weights of rows u = 0, 1 as a bf16 pair
      if constexpr (PAIR_V) {
        // Stale max: a row slot keeps its running max until a score exceeds
        // it by more than kStaleLog2 (so p <= 2^8); then every lane of the
        // wave moves to its true max and rescales.
        float mx[GT];
        bool need = false;
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          mx[h] = fmaxf(s[0][h], s[1][h]);
          need |= mx[h] > m[h] + kStaleLog2;
        }
        if (__any(need)) {
#pragma unroll
          for (int h = 0; h < GT; ++h) {
            const float mnew = fmaxf(m[h], mx[h]);
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mnew);
            m[h] = mnew;
            l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
          }
        }
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          pp[h] = pack_bf16_pair(__builtin_amdgcn_exp2f(s[0][h] - m[h]),
                                 __builtin_amdgcn_exp2f(s[1][h] - m[h]));
          l[h] += bf16lo(pp[h]) + bf16hi(pp[h]);
        }
      } else {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          float mx = s[0][h];
#pragma unroll
          for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][h]);
          const float mnew = fmaxf(m[h], mx);
          const float alpha = __builtin_amdgcn_exp2f(m[h] - mnew);
          m[h] = mnew;
          float psum = 0.f;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            s[u][h] = __builtin_amdgcn_exp2f(s[u][h] - mnew);
            psum += s[u][h];
          }
          l[h] = l[h] * alpha + psum;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        }
      }
      // Masked rows contribute p = 0; zeroing V as well keeps a NaN in an
      // unused slot from turning 0 * NaN into NaN.
      // (Selected per component: a select of the whole vector makes the
      // compiler keep extra copies of the preloaded rows live.)
      u32x4 vm[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        vm[u].x = ok[u] ? vc[u].x : 0u;
        vm[u].y = ok[u] ? vc[u].y : 0u;
        vm[u].z = ok[u] ? vc[u].z : 0u;
        vm[u].w = ok[u] ? vc[u].w : 0u;
      }
      if constexpr (PAIR_V) {
        const uint32_t w0[4] = {vm[0].x, vm[0].y, vm[0].z, vm[0].w};
        const uint32_t w1[4] = {vm[1].x, vm[1].y, vm[1].z, vm[1].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // codes of elements 4e, 4e+1 (lo) and 4e+2, 4e+3 (hi) as {row 0, row 1} byte pairs
          const uint32_t lo = __builtin_amdgcn_perm(w1[e], w0[e], 0x05010400u);
          const uint32_t hi = __builtin_amdgcn_perm(w1[e], w0[e], 0x07030602u);
          const uint32_t vb[4] = {fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo),
                                  fp8x2_to_bf16x2<false>(hi), fp8x2_to_bf16x2<true>(hi)};
#pragma unroll
          for (int h = 0; h < GT; ++h) {
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[h][4 * e + k] = dot2_bf16(pp[h], vb[k], acc[h][4 * e + k]);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float vf[EPL];
          vconv(vm[u], vf);
#pragma unroll
          for (int h = 0; h < GT; ++h) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(s[u][h], vf[e], acc[h][e]);
          }
        }
      }
    }
  };
  using std_false = std::integral_constant<bool, false>;
  using std_true = std::integral_constant<bool, true>;
  if (LONG && lng)
    stream(std::integral_constant<int, 2 * NIT>{}, std::integral_constant<int, DEPTH_LONG>{}, std_true{});
  else
    stream(std::integral_constant<int, NIT>{}, std::integral_constant<int, DEPTH>{}, std_false{});

  // APPEND: row slot 0 of wave 0 takes the new token (last split only).
  if constexpr (APPEND) {
    if (split == nsplit - 1 && w == 0) {
      const u32x4 nv = store_new();
      // lane c's part of the row: vector c (bf16) or the codes of vectors 2c, 2c+1 (KV8)
      u32x4 kx, vx;
      if constexpr (KV8) {
        const int sk = 2 * c, sv = NLB + 2 * c;
        kx = u32x4{(uint32_t)__shfl((int)nv.x, sk), (uint32_t)__shfl((int)nv.y, sk),
                   (uint32_t)__shfl((int)nv.x, sk + 1), (uint32_t)__shfl((int)nv.y, sk + 1)};
        vx = u32x4{(uint32_t)__shfl((int)nv.x, sv), (uint32_t)__shfl((int)nv.y, sv),
                   (uint32_t)__shfl((int)nv.x, sv + 1), (uint32_t)__shfl((int)nv.y, sv + 1)};
      } else {
        kx = u32x4{(uint32_t)__shfl((int)nv.x, c), (uint32_t)__shfl((int)nv.y, c),
                   (uint32_t)__shfl((int)nv.z, c), (uint32_t)__shfl((int)nv.w, c)};
        vx = u32x4{(uint32_t)__shfl((int)nv.x, NLB + c), (uint32_t)__shfl((int)nv.y, NLB + c),
                   (uint32_t)__shfl((int)nv.z, NLB + c), (uint32_t)__shfl((int)nv.w, NLB + c)};
      }
      float sn[GT];
#pragma unroll
      for (int h = 0; h < GT; ++h) sn[h] = mul_rn(group_sum<LPR>(kdot(h, kx)), a.scale_log2e);
      if (r == 0) {
        float vf[EPL];
        vconv(vx, vf);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const float mnew = fmaxf(m[h], sn[h]);
          const float alpha = __builtin_amdgcn_exp2f(m[h] - mnew);
          const float p = __builtin_amdgcn_exp2f(sn[h] - mnew);
          m[h] = mnew;
          l[h] = l[h] * alpha + p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e] * alpha);
        }
      }
    }
  }

  // Merge the row slots of this wave (lanes differing in the row bits).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float mo = shfl_xor(m[h], off);
      const float lo = shfl_xor(l[h], off);
      const float mn = fmaxf(m[h], mo);
      const float a1 = __builtin_amdgcn_exp2f(m[h] - mn);
      const float a2 = __builtin_amdgcn_exp2f(mo - mn);
      l[h] = l[h] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * a1 + ao * a2;
      }
      m[h] = mn;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[w][h][c * EPL + e] = acc[h][e];
      if (c == 0) {
        s_m[w][h] = m[h];
        s_l[w][h] = l[h];
      }
    }
  }
  __syncthreads();

  const int64_t unit = (int64_t)seq * a.hg + hg;
  for (int i = tid; i < GT * D; i += blockDim.x) {
    const int h = i / D;
    const int d = i - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = __builtin_amdgcn_exp2f(s_m[ww][h] - M);
      L += s_l[ww][h] * f;
      O += s_acc[ww][h][d] * f;
    }
    if constexpr (KV8) O *= a.v_scale;
    if (nsplit == 1) {
      if (h < gh) {
        const int64_t o = ((int64_t)seq * a.Hq + h0 + h) * D + d;
        const float val = L > 0.f ? O / L : 0.f;
        if (a.out_f32) ((float*)a.out)[o] = val;
        else ((uint16_t*)a.out)[o] = (uint16_t)f32_to_bf16_rne(val);
      }
    } else {
      const int64_t p = (unit * a.nsplit_max + split) * GT + h;
      a.ws_o[p * D + d] = O;
      if (d == 0) {
        a.ws_ml[2 * p] = M;
        a.ws_ml[2 * p + 1] = L;
      }
    }
  }
}

template <int D, int GT, int U, int NIT, int DEPTH, int DEPTH_LONG, bool LONG, bool NT, bool KV8,
          bool APPEND, bool SCALAR_BLK>
__global__ __launch_bounds__(256) void paged_decode_kernel(DecodeArgs a) {
  paged_decode_body<D, GT, U, NIT, DEPTH, DEPTH_LONG, LONG, NT, KV8, APPEND, SCALAR_BLK>(a);
}

// Merge the split-K partials of one (sequence, head group):
// out = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s, in split order.
// The context length, every slot's (m, l) and the first two splits' partial
// outputs (every merged context has two) are loaded together (entries past
// the sequence's last split are read but ignored); the other partial outputs
// follow once the split count is known, kCombineChunk splits at a time,
// slots past the last split re-reading it (cached) rather than stale
// workspace lines from HBM.  Loading the first 16 slots before the count was
// known cost the headline step 1.3 us; loading none before it cost the
// 7B-shaped merge (at most 4 splits) 2 us.
constexpr int kCombineChunk = 16;

template <int D, int GT>
__global__ __launch_bounds__(256) void paged_decode_combine_kernel(DecodeArgs a) {
  const int S = 1 << a.split_log2;  // tokens per (short) split
  constexpr int ITEMS = (GT * D + 255) / 256;  // (head, dim) outputs per thread
  __shared__ float s_w[kDecodeMaxSplits][GT];  // per split: 2^(m_s - M) / L
  const int unit = blockIdx.x;
  const int hg = unit % a.hg;
  const int seq = unit / a.hg;
  const int tid = threadIdx.x;
  const int64_t p0 = (int64_t)unit * a.nsplit_max * GT;

  int ctx = a.context_lens[seq];
  // The first two splits' partial outputs (every merged context has them).
  float pre[ITEMS][kCombineChunk];
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int i = min(tid + 256 * k, GT * D - 1);
    const int h = i / D;
    const int d = i - h * D;
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
      pre[k][sp] = a.ws_o[(p0 + (int64_t)min(sp, a.nsplit_max - 1) * GT + h) * D + d];
  }
  // (m, l) of every split: wave w reduces heads w, w + 4, ...; lane i holds
  // splits i, i + 64, ...  (loaded before the context length is known).
  const int w = tid >> 6;
  const int lane = tid & 63;
  constexpr int HPW = (GT + kWaves - 1) / kWaves;           // heads per wave
  constexpr int SPL = (kDecodeMaxSplits + 63) / 64;         // splits per lane
  float mv[HPW][SPL], lv[HPW][SPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = min(w + kWaves * hh, GT - 1);
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int sp = lane + 64 * k;
      mv[hh][k] = kNegBig;
      lv[hh][k] = 0.f;
      if (sp < a.nsplit_max) {
        mv[hh][k] = a.ws_ml[2 * (p0 + (int64_t)sp * GT + h)];
        lv[hh][k] = a.ws_ml[2 * (p0 + (int64_t)sp * GT + h) + 1];
      }
    }
  }
  const int cap = a.mbs << a.bs_log2;
  ctx = ctx < 0 ? 0 : (ctx > cap ? cap : ctx);
  int nsplit = (ctx + S - 1) / S;
  if (a.long_splits && nsplit > a.long_above) nsplit = (ctx + 2 * S - 1) / (2 * S);
  if (nsplit <= 1) return;  // written directly by the main kernel
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int i = min(tid + 256 * k, GT * D - 1);
    const int h = i / D;
    const int d = i - h * D;
#pragma unroll
    for (int sp = 2; sp < kCombineChunk; ++sp) {
      const int spc = min(sp, nsplit - 1);
      pre[k][sp] = a.ws_o[(p0 + (int64_t)spc * GT + h) * D + d];
    }
  }
  const int kvh = hg / a.nsub;
  const int sub = hg - kvh * a.nsub;
  const int h0 = kvh * a.group + sub * GT;
  const int gh = min(GT, a.group - sub * GT);
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const int h = w + kWaves * hh;
    if (h >= GT) break;  // wave-uniform
    float M = kNegBig;
#pragma unroll
    for (int k = 0; k < SPL; ++k)
      if (lane + 64 * k < nsplit) M = fmaxf(M, mv[hh][k]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
    float L = 0.f;
#pragma unroll
    for (int k = 0; k < SPL; ++k)
      if (lane + 64 * k < nsplit) L += lv[hh][k] * __builtin_amdgcn_exp2f(mv[hh][k] - M);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += shfl_xor(L, off);
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int sp = lane + 64 * k;
      if (sp < nsplit) s_w[sp][h] = __builtin_amdgcn_exp2f(mv[hh][k] - M) * inv;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const int i = tid + 256 * k;
    if (i >= gh * D) continue;
    const int h = i / D;
    const int d = i - h * D;
    float O = 0.f;
#pragma unroll
    for (int sp = 0; sp < kCombineChunk; ++sp)
      if (sp < nsplit) O += pre[k][sp] * s_w[sp][h];
    // Longer contexts: further splits in batches whose loads are issued together.
    for (int base = kCombineChunk; base < nsplit; base += kCombineChunk) {
      float t[kCombineChunk];
#pragma unroll
      for (int sp = 0; sp < kCombineChunk; ++sp)
        t[sp] = a.ws_o[(p0 + (int64_t)min(base + sp, nsplit - 1) * GT + h) * D + d];
#pragma unroll
      for (int sp = 0; sp < kCombineChunk; ++sp)
        if (base + sp < nsplit) O += t[sp] * s_w[base + sp][h];
    }
    const int64_t o = ((int64_t)seq * a.Hq + h0 + h) * D + d;
    if (a.out_f32) ((float*)a.out)[o] = O;
    else ((uint16_t*)a.out)[o] = (uint16_t)f32_to_bf16_rne(O);
  }
}

// Production tiling (measured on the Qwen3-0.6B-shaped decode, 64 x 16/8 heads,
// contexts up to 4096, and the 512-sequence decode): non-temporal (streaming)
// loads; bf16: U = 2 rows per lane per chunk, NIT = 8 chunks per wave; FP8:
// U = 2, NIT = 4 (a 16-byte load carries twice the elements).  Either way a
// short split is 256 tokens at D = 128 and 512 tokens at D = 64.  A wave
// keeps 4 chunks of loads in flight in a short split (all of them on FP8
// pools; 4 instead of all 8 on bf16 pools measured level at 64 sequences and
// 4% faster at 512); in a long split one chunk on bf16 pools and two on FP8
// pools (FP8 headline step 1 us faster than with one; four: 2 us slower).
constexpr bool kNontemporal = true;

template <bool KV8> constexpr int tile_u() { return 2; }
template <bool KV8> constexpr int tile_nit() { return KV8 ? 4 : 8; }
template <bool KV8> constexpr int tile_depth() { return 4; }
template <bool KV8> constexpr int tile_depth_long() { return KV8 ? 2 : 1; }
template <bool KV8> constexpr int max_gt() { return KV8 ? 4 : 8; }

template <int D, bool KV8>
constexpr int split_tokens() {
  return kWaves * tile_nit<KV8>() * tile_u<KV8>() * (64 / (D / (KV8 ? 16 : 8)));
}

// t_start / t_end (either may be null) are attached to the launch itself
// (hipExtLaunchKernel), so they carry the kernel's own start and end times.
template <int D, int GT, bool KV8, bool APPEND, bool LONG, bool SCALAR_BLK>
void launch_main(const DecodeArgs& a, unsigned nwg, hipStream_t stream, hipEvent_t t_start,
                 hipEvent_t t_end) {
  hipExtLaunchKernelGGL((paged_decode_kernel<D, GT, tile_u<KV8>(), tile_nit<KV8>(),
                                             tile_depth<KV8>(), tile_depth_long<KV8>(), LONG,
                                             kNontemporal, KV8, APPEND, SCALAR_BLK>),
                        dim3(nwg), dim3(256), 0, stream, t_start, t_end, 0u, a);
}

template <int D, int GT, bool KV8, bool APPEND>
int launch_d(const DecodeArgs& a, int B, hipStream_t stream) {
  const unsigned nwg = (unsigned)((int64_t)B * a.hg * a.nsplit_max);
  const bool scalar_blk = (1 << a.bs_log2) >= split_tokens<D, KV8>();
  if (a.long_splits && !scalar_blk) return -2;  // planned only when a block holds a short split
  hipEvent_t t_start = nullptr, t_end = nullptr;
  take_decode_timing(&t_start, &t_end);
  if (a.long_splits) {
    launch_main<D, GT, KV8, APPEND, true, true>(a, nwg, stream, t_start, t_end);
  } else {
    if (scalar_blk) launch_main<D, GT, KV8, APPEND, false, true>(a, nwg, stream, t_start, t_end);
    else launch_main<D, GT, KV8, APPEND, false, false>(a, nwg, stream, t_start, t_end);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  return a.nsplit_max > 1 ? launch_decode_combine(a, B, D, GT, stream) : 0;
}

template <int D, int GT>
int launch_combine(const DecodeArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL((paged_decode_combine_kernel<D, GT>), dim3((unsigned)((int64_t)B * a.hg)),
                     dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int D>
int launch_combine_d(const DecodeArgs& a, int B, int gt, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_combine<D, 1>(a, B, stream);
    case 2: return launch_combine<D, 2>(a, B, stream);
    case 3: return launch_combine<D, 3>(a, B, stream);
    case 4: return launch_combine<D, 4>(a, B, stream);
    case 5: return launch_combine<D, 5>(a, B, stream);
    case 6: return launch_combine<D, 6>(a, B, stream);
    case 7: return launch_combine<D, 7>(a, B, stream);
    case 8: return launch_combine<D, 8>(a, B, stream);
    case 9: return launch_combine<D, 9>(a, B, stream);
    case 10: return launch_combine<D, 10>(a, B, stream);
    case 11: return launch_combine<D, 11>(a, B, stream);
    case 12: return launch_combine<D, 12>(a, B, stream);
    case 13: return launch_combine<D, 13>(a, B, stream);
    case 14: return launch_combine<D, 14>(a, B, stream);
    case 15: return launch_combine<D, 15>(a, B, stream);
    case 16: return launch_combine<D, 16>(a, B, stream);
  }
  return -2;
}

template <int D, bool KV8, bool APPEND>
int launch_gt(const DecodeArgs& a, int B, int gt, hipStream_t stream) {
  switch (gt) {
    case 1: return launch_d<D, 1, KV8, APPEND>(a, B, stream);
    case 2: return launch_d<D, 2, KV8, APPEND>(a, B, stream);
    case 3: return launch_d<D, 3, KV8, APPEND>(a, B, stream);
    case 4: return launch_d<D, 4, KV8, APPEND>(a, B, stream);
    default:
      if constexpr (!KV8) {
        switch (gt) {
          case 5: return launch_d<D, 5, KV8, APPEND>(a, B, stream);
          case 6: return launch_d<D, 6, KV8, APPEND>(a, B, stream);
          case 7: return launch_d<D, 7, KV8, APPEND>(a, B, stream);
          case 8: return launch_d<D, 8, KV8, APPEND>(a, B, stream);
        }
      }
      return -2;
  }
}

template <bool KV8, bool APPEND>
int launch_head_dim(const DecodeArgs& a, int B, int head_dim, int gt, hipStream_t stream) {
  if (head_dim == 128) return launch_gt<128, KV8, APPEND>(a, B, gt, stream);
  if (head_dim == 64) return launch_gt<64, KV8, APPEND>(a, B, gt, stream);
  return -2;
}

}  // namespace

namespace {
thread_local hipEvent_t t_pending_start = nullptr;
thread_local hipEvent_t t_pending_end = nullptr;
}  // namespace

void set_decode_timing(hipEvent_t start, hipEvent_t end) {
  t_pending_start = start;
  t_pending_end = end;
}

void take_decode_timing(hipEvent_t* start, hipEvent_t* end) {
  *start = t_pending_start;
  *end = t_pending_end;
  t_pending_start = t_pending_end = nullptr;
}

int launch_decode_combine(const DecodeArgs& a, int B, int head_dim, int gt, hipStream_t stream) {
  if (head_dim == 128) return launch_combine_d<128>(a, B, gt, stream);
  if (head_dim == 64) return launch_combine_d<64>(a, B, gt, stream);
  return -2;
}

DecodePlan plan_decode(int B, int Hq, int Hkv, int head_dim, int block_size, int mbs, bool kv8) {
  DecodePlan p{};
  p.group = Hq / Hkv;
  // Groups of kMfmaMinGroup (FP8 pools: kMfmaMinGroupFp8) or more query heads
  // per KV head run the MFMA kernel: the VALU kernel's vector work grows with
  // the group.
  p.mfma = p.group >= (kv8 ? kMfmaMinGroupFp8 : kMfmaMinGroup);
  const int gmax = p.mfma ? kMfmaMaxGt : (kv8 ? max_gt<true>() : max_gt<false>());
  p.nsub = (p.group + gmax - 1) / gmax;
  p.gt = (p.group + p.nsub - 1) / p.nsub;
  const int64_t max_ctx = (int64_t)mbs * block_size;
  const int64_t units = (int64_t)B * Hkv * p.nsub;
  int S = p.mfma ? kMfmaSplitTokens
          : head_dim == 64 ? (kv8 ? split_tokens<64, true>() : split_tokens<64, false>())
                           : (kv8 ? split_tokens<128, true>() : split_tokens<128, false>());
  if (p.mfma && max_ctx > kMfmaSplitTokens &&
      units * ((max_ctx + kMfmaLongSplitTokens - 1) / kMfmaLongSplitTokens) >= kMfmaLongMinGrid)
    S = kMfmaLongSplitTokens;
  int sl = 0;
  while ((1 << sl) < S) ++sl;
  p.split_log2 = sl;
  p.nsplit_short = (int)((max_ctx + S - 1) / S);
  if (p.nsplit_short < 1) p.nsplit_short = 1;
  // Long splits halve the grid's slots per sequence.  They are taken only
  // when a cache block holds a whole short split (the block ids stay scalar
  // loads), the longest context needs many short splits, and the halved grid
  // still gives every compute unit many workgroups (coarser work items make
  // the end of a small grid ragged).
  const int64_t half = (p.nsplit_short + 1) / 2;
  p.long_splits = !p.mfma && block_size >= S && p.nsplit_short >= kLongSplitMinShort &&
                  units * half >= (kv8 ? kLongSplitMinGridFp8 : kLongSplitMinGrid);
  p.nsplit_max = p.long_splits ? (int)half : p.nsplit_short;
  // FP8 pools take long splits for every context of more than one short
  // split (fewer, longer items: the FP8 headline step 1 us faster); bf16
  // pools only for contexts that do not fit the halved slots (for all of
  // them, the 512-sequence decode was 414-419 against 361-364 us).
  p.long_above = kv8 ? 1 : p.nsplit_max;
  p.compact = B <= kCompactMaxSeqs;
  const int64_t parts = units * p.nsplit_max * p.gt;
  auto round256 = [](size_t x) { return (x + 255) / 256 * 256; };
  p.units = units;
  p.ml_bytes = round256((size_t)parts * 2 * sizeof(float));
  p.o_bytes = round256((size_t)parts * head_dim * sizeof(float));
  return p;
}

int launch_paged_decode(const DecodeArgs& a, int B, int head_dim, int gt, bool kv8, bool append,
                        bool mfma, hipStream_t stream) {
  if (B == 0) return 0;
  if (mfma) return launch_paged_decode_mfma(a, B, head_dim, kv8, append, stream);
  if (kv8) {
    return append ? launch_head_dim<true, true>(a, B, head_dim, gt, stream)
                  : launch_head_dim<true, false>(a, B, head_dim, gt, stream);
  }
  return append ? launch_head_dim<false, true>(a, B, head_dim, gt, stream)
                : launch_head_dim<false, false>(a, B, head_dim, gt, stream);
}

}  // namespace pa
