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
//     KV head (GQA rows share every K/V tile), and walks 64-key tiles;
//   * it computes S^T = K Q^T and O^T = V^T P^T, so the accumulator layout
//     gives each lane one query row: the softmax is per lane (plus one
//     exchange with the lane holding the row's other 32 keys) and P feeds the
//     second MFMA straight from registers, with no trip through LDS;
//   * the K tile is staged in LDS row-major; the V tile is staged transposed
//     (V^T rows of 64 keys), with key positions permuted inside each group of
//     16 (bits 2 and 3 swapped) to match the order in which a lane holds P;
//   * the next tile's global loads are issued before the current tile's math.
#include "common.h"
#include "kernels.h"

namespace pa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 128;  // query rows per workgroup
constexpr int kBN = 64;     // keys per tile
constexpr int kPadK = 8;    // bf16 padding per LDS row (bank spread)
constexpr int kPadV = 8;

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Position of key k (0..63) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D>
struct TileRegs {
  static constexpr int KCH = kBN * D / 8 / 256;       // 16-byte K chunks per thread
  static constexpr int VIT = (kBN / 2) * D / 8 / 256;  // (key pair, 8 dims) items per thread
  u32x4 k[KCH];
  u32x4 v0[VIT], v1[VIT];
};

template <int D>
__global__ __launch_bounds__(256) void paged_prefill_kernel(PrefillArgs a, int tt_tokens,
                                                               int ntt) {
  constexpr int KS = D / 16;  // 16-wide K steps over head_dim
  constexpr int DT = D / 32;  // 32-row tiles of O^T
  constexpr int LPR = D / 8;  // 16-byte chunks per K/V row
  using Regs = TileRegs<D>;

  __shared__ __align__(16) uint16_t sK[kBN][D + kPadK];
  __shared__ __align__(16) uint16_t sVt[D][kBN + kPadV];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;  // this lane's query row within the wave
  const int hi = lane >> 5;  // which half of the 16-wide K step

  // Heaviest token tiles first (later tiles attend to more keys).  The token
  // tiles of one (sequence, KV head) are B * Hkv workgroups apart, so they
  // land on one XCD when B * Hkv is a multiple of 8 and share its L2.
  const int per_tt = a.B * a.Hkv;
  const int tt = ntt - 1 - (int)(blockIdx.x / per_tt);
  const int rem = blockIdx.x % per_tt;
  const int seq = rem / a.Hkv;
  const int kvh = rem - seq * a.Hkv;

  const int qa = a.cu_seqlens_q[seq];
  const int n = a.cu_seqlens_q[seq + 1] - qa;
  const int t0 = tt * tt_tokens;
  if (n <= 0 || t0 >= n) return;
  int ctx = a.context_lens[seq];
  const int cap = a.mbs << a.bs_log2;
  int P = ctx - n;
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
  for (int ks = 0; ks < KS; ++ks) {
    qb[ks] = row_ok ? *(const u32x4*)(a.q + qrow + ks * 16 + hi * 8) : u32x4{0u, 0u, 0u, 0u};
  }

  const int bs_mask = (1 << a.bs_log2) - 1;
  const int64_t kv_stride = (int64_t)a.Hkv * D;

  // Source of key kk: the paged cache below P, k_new / v_new from P on.
  // Returns false (and a safe offset) for keys past kend or in an invalid block.
  auto key_src = [&](int kk, int dchunk, int64_t& off, bool& from_new) -> bool {
    from_new = kk >= P;
    off = 0;
    if (kk >= kend) return false;
    if (from_new) {
      off = (int64_t)(qa + kk - P) * kv_stride + kvh * D + dchunk * 8;
      return true;
    }
    const int blk = a.block_tables[(int64_t)seq * a.mbs + (kk >> a.bs_log2)];
    if (blk < 0 || blk >= a.num_blocks) return false;
    off = (((int64_t)blk << a.bs_log2) + (kk & bs_mask)) * kv_stride + kvh * D + dchunk * 8;
    return true;
  };
  auto load16 = [&](const uint16_t* cache, const uint16_t* fresh, int kk, int dchunk) -> u32x4 {
    int64_t off;
    bool from_new;
    const bool ok = key_src(kk, dchunk, off, from_new);
    const uint16_t* base = from_new ? fresh : cache;
    const u32x4 v = *(const u32x4*)(base + off);
    return ok ? v : u32x4{0u, 0u, 0u, 0u};
  };

  auto load_tile = [&](int j, Regs& rg) {
    const int k0 = j * kBN;
#pragma unroll
    for (int i = 0; i < Regs::KCH; ++i) {
      const int c = tid + 256 * i;
      rg.k[i] = load16(a.k_cache, a.k_new, k0 + c / LPR, c % LPR);
    }
#pragma unroll
    for (int i = 0; i < Regs::VIT; ++i) {
      const int c = tid + 256 * i;
      const int kp = c % (kBN / 2);
      const int dchunk = c / (kBN / 2);
      rg.v0[i] = load16(a.v_cache, a.v_new, k0 + 2 * kp, dchunk);
      rg.v1[i] = load16(a.v_cache, a.v_new, k0 + 2 * kp + 1, dchunk);
    }
  };

  auto store_tile = [&](const Regs& rg) {
#pragma unroll
    for (int i = 0; i < Regs::KCH; ++i) {
      const int c = tid + 256 * i;
      *(u32x4*)&sK[c / LPR][(c % LPR) * 8] = rg.k[i];
    }
#pragma unroll
    for (int i = 0; i < Regs::VIT; ++i) {
      const int c = tid + 256 * i;
      const int kp = c % (kBN / 2);
      const int d0 = (c / (kBN / 2)) * 8;
      const int col = vt_pos(2 * kp);
      const uint32_t x[4] = {rg.v0[i].x, rg.v0[i].y, rg.v0[i].z, rg.v0[i].w};
      const uint32_t y[4] = {rg.v1[i].x, rg.v1[i].y, rg.v1[i].z, rg.v1[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dims d0+2e and d0+2e+1: (key 2kp, key 2kp+1) pairs
        *(uint32_t*)&sVt[d0 + 2 * e][col] = __builtin_amdgcn_perm(y[e], x[e], 0x05040100u);
        *(uint32_t*)&sVt[d0 + 2 * e + 1][col] = __builtin_amdgcn_perm(y[e], x[e], 0x07060302u);
      }
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = kNegBig;  // running max of raw scores for this lane's row
  float l_run = 0.f;      // this lane's share of the softmax denominator
  const float c = a.scale_log2e;

  Regs rg;
  load_tile(0, rg);
  for (int j = 0; j < ntiles; ++j) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile(rg);
    __syncthreads();
    if (j + 1 < ntiles) load_tile(j + 1, rg);

    // S^T = K Q^T for the two 32-key halves of the tile.
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sacc[kt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 ka = *(const u32x4*)&sK[kt * 32 + lr][ks * 16 + hi * 8];
        sacc[kt] = mfma32(ka, qb[ks], sacc[kt]);
      }
    }
    // Causal / range mask: key k0 + key_local is visible to this row iff <= pos.
    const int k0 = j * kBN;
    const bool need_mask = k0 + kBN - 1 > P + t0;  // some row of the workgroup may not see all keys
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sv = sacc[kt][i];
        if (need_mask) {
          const int kk = k0 + kt * 32 + 8 * (i >> 2) + 4 * hi + (i & 3);
          sv = kk <= pos ? sv : -INFINITY;
        }
        sacc[kt][i] = sv;
        mx = fmaxf(mx, sv);
      }
    }
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
    m_run = m_new;
    const float mc = m_new * c;
    u32x4 pb[4];  // P^T operands of the four 16-key steps, bf16
    float psum = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][(s & 1) * 8 + 2 * e], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][(s & 1) * 8 + 2 * e + 1], c, -mc));
        const uint32_t b0 = f32_to_bf16_rne(p0);
        const uint32_t b1 = f32_to_bf16_rne(p1);
        psum += __uint_as_float(b0 << 16) + __uint_as_float(b1 << 16);  // sum of what the MFMA sees
        wv[e] = b0 | (b1 << 16);
      }
      pb[s] = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 va = *(const u32x4*)&sVt[dt * 32 + lr][s * 16 + hi * 8];
        oacc[dt] = mfma32(va, pb[s], oacc[dt]);
      }
    }
  }

  const float l_tot = l_run + shfl_xor(l_run, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
        const uint32_t w0 = f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16);
        const uint32_t w1 = f32_to_bf16_rne(o2) | (f32_to_bf16_rne(o3) << 16);
        *(uint2*)((uint16_t*)a.out + qrow + d) = make_uint2(w0, w1);
      }
    }
  }
}

}  // namespace

int launch_paged_prefill(const PrefillArgs& a, int head_dim, hipStream_t stream) {
  if (a.group > kRows) return -3;
  const int tt_tokens = kRows / a.group;
  const int ntt = (a.max_q_len + tt_tokens - 1) / tt_tokens;
  const int64_t nwg = (int64_t)ntt * a.B * a.Hkv;
  if (nwg == 0) return 0;
  if (nwg > INT32_MAX) return -2;
  if (head_dim == 128) {
    hipLaunchKernelGGL(paged_prefill_kernel<128>, dim3((unsigned)nwg), dim3(256), 0, stream, a,
                       tt_tokens, ntt);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(paged_prefill_kernel<64>, dim3((unsigned)nwg), dim3(256), 0, stream, a,
                       tt_tokens, ntt);
  } else {
    return -3;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace pa
