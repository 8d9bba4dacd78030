// Shared device helpers for the gfx950 kernels of libpagedattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 8 bf16 = one 128-bit load
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Running-max start value: finite, so exp2(m_old - m_new) never sees inf - inf.
constexpr float kNegBig = -3.0e38f;

__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// A rounded fp32 product that is never contracted into a later add or
// subtract (hipcc contracts a * b - c into one fma by default, and
// __fmul_rn is a plain multiply that contracts the same way).
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// Two bf16 products summed into an fp32 accumulator (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// Two OCP E4M3 codes (bytes 0,1 or 2,3 of `w`) widened exactly to a bf16 pair
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1) or to two fp32 (v_cvt_pk_f32_fp8).
template <bool HIGH>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
}
template <bool HIGH>
__device__ __forceinline__ float2_t fp8x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HIGH);
}

// bf16 -> OCP E4M3 code of x / s: the division in fp32 (correctly rounded),
// clamped to +-448 so that large magnitudes saturate (the hardware conversion
// would give NaN from 480 on), NaN kept as S.1111.111 with the input's sign,
// then v_cvt_pk_fp8_f32 (round to nearest even).  Two codes in bits 0..15.
__device__ __forceinline__ uint32_t fp8_code_pair(float x0, float x1, float s) {
  float q0 = x0 / s, q1 = x1 / s;
  const bool n0 = q0 != q0, n1 = q1 != q1;
  q0 = n0 ? 0.f : fminf(fmaxf(q0, -448.f), 448.f);
  q1 = n1 ? 0.f : fminf(fmaxf(q1, -448.f), 448.f);
  uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false) & 0xFFFFu;
  if (n0) c = (c & 0xFF00u) | 0x7Fu | ((__float_as_uint(x0) >> 24) & 0x80u);
  if (n1) c = (c & 0x00FFu) | 0x7F00u | ((__float_as_uint(x1) >> 16) & 0x8000u);
  return c;
}

// Eight bf16 values (one 16-byte vector) -> eight E4M3 codes, in element order.
__device__ __forceinline__ u32x2 quantize8(const u32x4& a, float s) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  uint32_t o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t p0 = fp8_code_pair(bf16lo(w[2 * i]), bf16hi(w[2 * i]), s);
    const uint32_t p1 = fp8_code_pair(bf16lo(w[2 * i + 1]), bf16hi(w[2 * i + 1]), s);
    o[i] = p0 | (p1 << 16);
  }
  return u32x2{o[0], o[1]};
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16) inside a DPP row; every lane
// of the group ends up holding the group total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) v += dpp<0x141>(v);  // row_half_mirror: quads 0<->1 inside each 8
  if constexpr (N == 16) v += dpp<0x140>(v);  // row_mirror: halves 0<->1 inside 16
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Compacted decode work list.  The (sequence, split) items of a decode call,
// where a sequence of context ctx (clamped to [0, cap]) has max(1, ceil(ctx /
// S)) splits, or ceil(ctx / 2S) when long splits are on and it needs more
// than long_above short ones: first every sequence's first split (items
// 0 .. B-1, known without the lengths, so those workgroups skip the lookup's
// round trip: the plain decode of the headline workload 1.5 us faster), then
// the later splits, sequences in order and each sequence's splits in order.
// Finds item `item` for the calling wave: lane l counts the later splits of
// sequences l*k .. l*k+k-1 (k = ceil(B / 64) <= PER_LANE), a wave scan turns
// the counts into each lane's first item, and the lane holding `item` walks
// its sequences.  Every lane returns the same result; false when `item` is
// past the last item.
template <int PER_LANE, class Args>
__device__ __forceinline__ bool decode_work_item(const Args& a, int item, int S, bool long_ok,
                                                 int& seq, int& split) {
  const int lane = threadIdx.x & 63;
  const int B = a.batch;
  if (item < B) {  // a first split
    seq = item;
    split = 0;
    return true;
  }
  item -= B;
  const int k = (B + 63) >> 6;
  const int s0 = lane * k;
  const int cap = a.mbs << a.bs_log2;
  int cnt[PER_LANE];
  int ctxs[PER_LANE];
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) ctxs[j] = (j < k && s0 + j < B) ? a.context_lens[s0 + j] : 0;
  int tot = 0;
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) {
    int n = 0;
    if (j < k && s0 + j < B) {
      const int ctx = ctxs[j] < 0 ? 0 : (ctxs[j] > cap ? cap : ctxs[j]);
      const int nshort = ctx == 0 ? 1 : (ctx + S - 1) / S;
      n = (long_ok && nshort > a.long_above) ? (ctx + 2 * S - 1) / (2 * S) : nshort;
    }
    cnt[j] = n > 0 ? n - 1 : 0;  // splits after the first
    tot += cnt[j];
  }
  int incl = tot;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  const int excl = incl - tot;
  const bool mine = item >= excl && item < incl;
  const uint64_t bal = __builtin_amdgcn_ballot_w64(mine);
  if (bal == 0) return false;
  int fs = 0, fsplit = 0;
  if (mine) {
    int rem = item - excl;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      if (rem >= 0 && rem < cnt[j]) {
        fs = s0 + j;
        fsplit = rem + 1;
      }
      rem -= cnt[j];
    }
  }
  const int src = (int)__builtin_ctzll(bal);
  seq = __builtin_amdgcn_readlane(fs, src);
  split = __builtin_amdgcn_readlane(fsplit, src);
  return true;
}

}  // namespace pa
