// QJL stage kernels for gfx950: encode with the 1-bit residual sketch, and
// dequantize with the QJL correction ([Scratch] §2 "QJL residual";
// [README] two-stage description and combined estimator).
//
// The residual's sign bits sign((S r)_p) are only meaningful to the
// estimator if they agree with the exact projection.  head_dim 128 encodes in
// fp32 with the projection on fp16 MFMA in split precision (hi/lo pieces of
// both operands, fp32 accumulation), whose error (about 1e-7 of the residual
// norm in the median, as for fp32 products) leaves a sign bit wrong only
// where |z| is within a few 1e-6 of rho; the other head sizes encode in
// float64, exact except within ~1e-15 of an edge.  S~ = S D H
// (host-prepared) is staged in LDS; because H and D are symmetric
// involutions, S (u - D H c) = S~ (y - c), so the residual never leaves the
// rotated domain.
#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

template <int BITS>
__device__ __forceinline__ uint32_t magnitude_index64(double a, const double* T) {
  if constexpr (BITS == 1) {
    return 0u;
  } else if constexpr (BITS == 2) {
    return a > T[0] ? 1u : 0u;
  } else if constexpr (BITS == 3) {
    const bool c1 = a > T[1];
    const double t = c1 ? T[2] : T[0];
    return (c1 ? 2u : 0u) + (a > t ? 1u : 0u);
  } else {
    const bool c1 = a > T[3];
    const double t2 = c1 ? T[5] : T[1];
    const bool c2 = a > t2;
    const double lo = c1 ? T[4] : T[0];
    const double hi = c1 ? T[6] : T[2];
    const double t3 = c2 ? hi : lo;
    return (c1 ? 4u : 0u) + (c2 ? 2u : 0u) + (a > t3 ? 1u : 0u);
  }
}

template <int BITS, int LPU, bool IN_F32, bool NORM_F32>
__global__ __launch_bounds__(kBlock) void qjl_encode_kernel(QjlEncodeArgs a, const float* __restrict__ s_rot32) {
  constexpr int DT = 32 * LPU;
  extern __shared__ float s_lds[];  // S~ [m][DT] float32
  const int m = a.m;
  for (int i = threadIdx.x; i < m * DT; i += kBlock) s_lds[i] = s_rot32[i];
  __syncthreads();
  const double* lvl = a.level;  // read from the kernel-argument segment (the LDS budget goes to S~)

  const int q = (int)(threadIdx.x % LPU);
  const uint32_t dword = a.dbits[q];
  const double inv_sqrt_dt = 1.0 / __builtin_sqrt((double)DT);
  const int64_t n_groups = a.n_units * LPU;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t g0 = (int64_t)blockIdx.x * kBlock; g0 < n_groups; g0 += stride) {
    const int64_t g = g0 + threadIdx.x;
    const bool valid = g < n_groups;
    const int64_t u = g / LPU;
    double v[32];
    if (valid) {
      if constexpr (IN_F32) {
        const float* p = static_cast<const float*>(a.x) + u * a.ld_x + 32 * q;
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = (double)p[j];
      } else {
        const __half* p = static_cast<const __half*>(a.x) + u * a.ld_x + 32 * q;
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = (double)__half2float(p[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = 0.0;
    }
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      ss = __builtin_fma(v[j], v[j], ss);
      if ((dword >> j) & 1u) v[j] = -v[j];
    }
    ss = unit_sum<LPU>(ss);
    const double n = __builtin_sqrt(ss);
    double T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = a.thr[k] * n;
    fwht32_inlane(v);
    fwht_crosslane<LPU>(v, q);

    // codes, and the rotated-domain residual e = y - c (unit-vector scale)
    uint32_t word[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) word[k] = 0u;
    const double yscale = n > 0.0 ? inv_sqrt_dt / n : 0.0;
    double e[32];
    double rr = 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const double y = v[j];
      const uint32_t neg = (y > 0.0) ? 0u : 1u;
      const uint32_t code = (neg << (BITS - 1)) | magnitude_index64<BITS>(__builtin_fabs(y), T);
      put_code<BITS>(word, j, code);
      e[j] = y * yscale - lvl[code] * inv_sqrt_dt;
      rr = __builtin_fma(e[j], e[j], rr);
    }
    rr = unit_sum<LPU>(rr);

    // z_p = sum_i S~[p][i] e_i; bit p = [z_p >= 0]
    uint32_t sbits[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) sbits[w] = 0u;
    for (int p = 0; p < m; ++p) {
      const float* row = s_lds + p * DT + 32 * q;
      double part = 0.0;
#pragma unroll
      for (int j = 0; j < 32; ++j) part = __builtin_fma((double)row[j], e[j], part);
      part = unit_sum<LPU>(part);
      if (part >= 0.0) sbits[p >> 5] |= 1u << (p & 31);
    }
    if (valid) {
      uint32_t* cp = reinterpret_cast<uint32_t*>(a.codes + g * (4 * BITS));
#pragma unroll
      for (int k = 0; k < BITS; ++k) cp[k] = word[k];
      uint32_t* bp = reinterpret_cast<uint32_t*>(a.qjl_bits) + u * (m / 32);
      for (int w = q; w < m / 32; w += LPU) bp[w] = sbits[w];
      if (q == 0) {
        if constexpr (NORM_F32)
          static_cast<float*>(a.norms)[u] = (float)n;
        else
          static_cast<__half*>(a.norms)[u] = __float2half_rn((float)n);
        a.rnorm[u] = __half_as_ushort(__float2half_rn((float)__builtin_sqrt(rr)));
      }
    }
  }
}

// Encode for head_dim = 128 in fp32, with the projection z = S~ e on fp16 MFMA
// (v_mfma_f32_16x16x32_f16) in split precision: e and S~ are each split into fp16 pieces x = hi + lo
// (hi = fp16(x), lo = fp16(x - hi), about 22 significant bits), and z accumulates hi.hi + hi.lo + lo.hi in
// fp32.  The products of fp16 pieces are exact in fp32, the dropped lo.lo term is 2^-22 of a product, so z
// carries the error of an fp32 dot product (about 1e-7 of rho, the residual norm, in the median): a sign
// bit can only differ from the exact one where |z| is within a few 1e-6 of rho, about as often as with
// fp32 products, and three fp16 passes cost a fifth of one fp32 pass.  e is scaled by 2^10 before the
// split (the sign of z is all that is kept), so its low pieces stay in fp16's normal range.
//
// Eight waves share one LDS copy of the S~ pieces; a wave encodes 16 keys: lane l holds the 32 coordinates
// 32 (l / 16) .. + 31 of key l % 16, and each lane packs one whole 32-group.  The contraction over the
// 128 coordinates is taken in the order in which the lanes hold them: K-step s of the MFMA takes
// coordinates 32 g + 8 s .. + 7 from lane group g, for both operands, so the A operand of step s is 8
// consecutive coordinates of the lane's own 32, and S~ sits in LDS as B-operand fragments in the same
// order.  The sign bit [z_p >= 0] of (key 4 (l / 16) + r, p = 16 pt + l % 16) comes out of the
// accumulator as a wave ballot; the ballots are regrouped into each key's m-bit row through a small LDS
// table.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kEncBlock = 512;  // 8 waves share one copy of S~ in LDS
constexpr float kResidualScale = 1024.0f;  // 2^10: e's fp16 pieces stay normal; z's sign does not change

template <int BITS, bool IN_F32, bool NORM_F32>
__global__ __launch_bounds__(kEncBlock) void qjl_encode128_kernel(QjlEncodeArgs a, const float* __restrict__ s_rot32) {
  constexpr int W = kEncBlock / 64;
  // [m/16][4 s][hi, lo][64 lanes] x 8 halves: S~[16 pt + l%16][32 (l/16) + 8 s + i] split into fp16 pieces
  extern __shared__ u32x4 sfrag[];
  __shared__ uint64_t ballots[W][32];             // per wave: [pt * 4 + r]
  __shared__ float lvl_s[16];
  const int m = a.m, npt = m / 16, words = m / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < npt * 256; e += kEncBlock) {
    const int pt = e >> 8, st = (e >> 6) & 3, ln = e & 63;
    const v4f* src = reinterpret_cast<const v4f*>(s_rot32 + (16 * pt + (ln & 15)) * 128 + 32 * (ln >> 4) + 8 * st);
    const v4f x0 = src[0], x1 = src[1];
    const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 h0 = (_Float16)xs[2 * i], h1 = (_Float16)xs[2 * i + 1];
      const _Float16 l0 = (_Float16)(xs[2 * i] - (float)h0), l1 = (_Float16)(xs[2 * i + 1] - (float)h1);
      hi[i] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      lo[i] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    sfrag[(pt * 8 + 2 * st) * 64 + ln] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    sfrag[(pt * 8 + 2 * st + 1) * 64 + ln] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  }
  if (tid < 16) lvl_s[tid] = (float)a.level[tid];
  __syncthreads();

  const int q = lane >> 4, kl = lane & 15;
  const uint32_t dword = q == 0 ? a.dbits[0] : q == 1 ? a.dbits[1] : q == 2 ? a.dbits[2] : a.dbits[3];
  const float s16 = (q & 1) ? -1.0f : 1.0f, s32 = (q & 2) ? -1.0f : 1.0f;  // cross-lane butterfly signs
  float thr[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) thr[k] = (float)a.thr[k];
  const int64_t n_tiles = (a.n_units + 15) / 16;
  for (int64_t tile = (int64_t)blockIdx.x * W + wave; tile < n_tiles; tile += (int64_t)gridDim.x * W) {
    const int64_t key = tile * 16 + kl;
    const bool valid = key < a.n_units;
    float v[32];
    if (valid) {
      if constexpr (IN_F32) {
        const v4f* p = reinterpret_cast<const v4f*>(static_cast<const float*>(a.x) + key * a.ld_x + 32 * q);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const v4f w = p[c];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[4 * c + i] = w[i];
        }
      } else {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const __half*>(a.x) + key * a.ld_x + 32 * q);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4 w = p[c];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[8 * c + 2 * i] = __half2float(__ushort_as_half((unsigned short)(w[i] & 0xFFFFu)));
            v[8 * c + 2 * i + 1] = __half2float(__ushort_as_half((unsigned short)(w[i] >> 16)));
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) v[j] = 0.0f;
    }
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      ss = __builtin_fmaf(v[j], v[j], ss);
      if ((dword >> j) & 1u) v[j] = -v[j];
    }
    ss = xlane_sum<32>(xlane_sum<16>(ss));
    const float n = __builtin_sqrtf(ss);
    // unnormalised FWHT over the 128 coordinates: bits 0..4 in the lane, bits 5 and 6 across lanes 16 and 32 apart
    fwht32_inlane(v);
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = xlane_butterfly<16>(v[j], s16);
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = xlane_butterfly<32>(v[j], s32);
    // codes (|y| against the N(0,1) edges scaled by n) and the residual e' = y / n - c in N(0,1) units
    float T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = thr[k] * n;
    const float inv_n = n > 0.0f ? 1.0f / n : 0.0f;
    uint32_t word[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) word[k] = 0u;
    float rr = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float y = v[j], ay = __builtin_fabsf(y);
      uint32_t mag = 0u;
      if constexpr (BITS == 2) {
        mag = ay > T[0] ? 1u : 0u;
      } else if constexpr (BITS == 3) {
        const bool c1 = ay > T[1];
        mag = (c1 ? 2u : 0u) + (ay > (c1 ? T[2] : T[0]) ? 1u : 0u);
      } else if constexpr (BITS == 4) {
        const bool c1 = ay > T[3];
        const bool c2 = ay > (c1 ? T[5] : T[1]);
        const float t3 = c1 ? (c2 ? T[6] : T[4]) : (c2 ? T[2] : T[0]);
        mag = (c1 ? 4u : 0u) + (c2 ? 2u : 0u) + (ay > t3 ? 1u : 0u);
      }
      const uint32_t code = ((y > 0.0f ? 0u : 1u) << (BITS - 1)) | mag;
      put_code<BITS>(word, j, code);
      v[j] = __builtin_fmaf(y, inv_n, -lvl_s[code]);
      rr = __builtin_fmaf(v[j], v[j], rr);
    }
    rr = xlane_sum<32>(xlane_sum<16>(rr));
    // fp16 pieces of 2^10 e, two coordinates per register: eh[4 s + i / 2] holds coordinates 8 s + i
    uint32_t eh[16], el[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float x0 = v[2 * j] * kResidualScale, x1 = v[2 * j + 1] * kResidualScale;
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
      eh[j] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      el[j] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }

    // z = S~ e for the 16 keys, 16 projections per pass, passes 2k and 2k + 1 on two accumulators
    // (independent MFMA chains; m is a multiple of 32); ballots of z >= 0
    for (int pt = 0; pt < npt; pt += 2) {
      v4f acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
      const u32x4* bf = sfrag + pt * 512 + lane;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const v8h ah = __builtin_bit_cast(v8h, u32x4{eh[4 * st], eh[4 * st + 1], eh[4 * st + 2], eh[4 * st + 3]});
        const v8h al = __builtin_bit_cast(v8h, u32x4{el[4 * st], el[4 * st + 1], el[4 * st + 2], el[4 * st + 3]});
        const v8h bh0 = __builtin_bit_cast(v8h, bf[128 * st]), bl0 = __builtin_bit_cast(v8h, bf[128 * st + 64]);
        const v8h bh1 = __builtin_bit_cast(v8h, bf[512 + 128 * st]), bl1 = __builtin_bit_cast(v8h, bf[512 + 128 * st + 64]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh1, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl1, acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh1, acc1, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint64_t bal0 = __ballot(acc0[r] >= 0.0f), bal1 = __ballot(acc1[r] >= 0.0f);
        if (lane == 0) {
          ballots[wave][pt * 4 + r] = bal0;
          ballots[wave][(pt + 1) * 4 + r] = bal1;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane t writes sign word t % words of key t / words: bits 16 h + (0..15) of ballots (2 w, r) and (2 w + 1, r)
    if (lane < 16 * words) {
      const int kk = lane / words, w = lane - kk * words, h = kk >> 2, r = kk & 3;
      const uint32_t lo = (uint32_t)(ballots[wave][(2 * w) * 4 + r] >> (16 * h)) & 0xFFFFu;
      const uint32_t hi = (uint32_t)(ballots[wave][(2 * w + 1) * 4 + r] >> (16 * h)) & 0xFFFFu;
      if (tile * 16 + kk < a.n_units)
        reinterpret_cast<uint32_t*>(a.qjl_bits)[tile * 16 * words + lane] = lo | (hi << 16);
    }
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      uint32_t* cp = reinterpret_cast<uint32_t*>(a.codes + key * (16 * BITS) + q * (4 * BITS));
#pragma unroll
      for (int k = 0; k < BITS; ++k) cp[k] = word[k];
      if (q == 0) {
        if constexpr (NORM_F32)
          static_cast<float*>(a.norms)[key] = n;
        else
          static_cast<__half*>(a.norms)[key] = __float2half_rn(n);
        a.rnorm[key] = __half_as_ushort(__float2half_rn(__builtin_sqrtf(rr) * 0.08838834764831845f));
      }
    }
  }
}

template <int BITS, int LPU, bool OUT_F32, bool NORM_F32, bool NC>
__global__ __launch_bounds__(kBlock) void qjl_decode_kernel(QjlDecodeArgs a) {
  constexpr int DT = 32 * LPU;
  extern __shared__ float s_lds[];  // S~ [m][DT] float32
  const int m = a.m;
  for (int i = threadIdx.x; i < m * DT; i += kBlock) s_lds[i] = a.s_rot[i];
  __syncthreads();
  const float* lut = a.level;  // read from the kernel-argument segment (the LDS budget goes to S~)
  const int q = (int)(threadIdx.x % LPU);
  const uint32_t dword = a.dbits[q];
  const int64_t n_groups = a.n_units * LPU;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t g0 = (int64_t)blockIdx.x * kBlock; g0 < n_groups; g0 += stride) {
    const int64_t g = g0 + threadIdx.x;
    const bool valid = g < n_groups;
    const int64_t u = g / LPU;
    uint32_t word[BITS];
    uint32_t sb[8];
    float n = 0.0f, rho = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sb[w] = 0u;
    if (valid) {
      const uint32_t* cp = reinterpret_cast<const uint32_t*>(a.codes + g * (4 * BITS));
#pragma unroll
      for (int k = 0; k < BITS; ++k) word[k] = cp[k];
      const uint32_t* bp = reinterpret_cast<const uint32_t*>(a.qjl_bits) + u * (m / 32);
      for (int w = 0; w < m / 32; ++w) sb[w] = bp[w];
      if constexpr (NORM_F32)
        n = static_cast<const float*>(a.norms)[u];
      else
        n = __half2float(static_cast<const __half*>(a.norms)[u]);
      rho = __half2float(__ushort_as_half(a.rnorm[u]));
    } else {
#pragma unroll
      for (int k = 0; k < BITS; ++k) word[k] = 0u;
    }
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = lut[get_code<BITS>(word, j)];
    // QJL correction in the rotated domain, in the N(0,1)-per-coordinate scale:
    // c += sqrt(dt) * sqrt(pi/2) * rho / m * (S~^T sigma)
    const float cs = a.qjl_scale * rho;
    float corr[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) corr[j] = 0.0f;
    for (int p = 0; p < m; ++p) {
      const float sg = ((sb[p >> 5] >> (p & 31)) & 1u) ? 1.0f : -1.0f;
      const float* row = s_lds + p * DT + 32 * q;
#pragma unroll
      for (int j = 0; j < 32; ++j) corr[j] = __builtin_fmaf(row[j], sg, corr[j]);
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = __builtin_fmaf(cs, corr[j], v[j]);
    float scale;
    if constexpr (NC) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) ss = __builtin_fmaf(v[j], v[j], ss);
      ss = unit_sum<LPU>(ss);
      scale = n * a.inv_sqrt_dt / __builtin_sqrtf(ss);
    } else {
      scale = n * a.inv_dt;
    }
    fwht32_inlane(v);
    fwht_crosslane<LPU>(v, q);
    if (!valid) continue;
    if constexpr (OUT_F32) {
      float* p = static_cast<float*>(a.y) + u * a.ld_y + 32 * q;
#pragma unroll
      for (int j = 0; j < 32; ++j) p[j] = ((dword >> j) & 1u) ? -(v[j] * scale) : v[j] * scale;
    } else {
      __half* p = static_cast<__half*>(a.y) + u * a.ld_y + 32 * q;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float o = v[j] * scale;
        p[j] = __float2half_rn(((dword >> j) & 1u) ? -o : o);
      }
    }
  }
}

int cu_count() { return device_cu_count(); }

int64_t qjl_grid(int64_t n_groups) {
  int64_t need = (n_groups + kBlock - 1) / kBlock;
  int64_t cap = (int64_t)cu_count() * 4;
  return need < cap ? need : cap;
}

template <int BITS, int LPU>
hipError_t qjl_encode_dispatch(const tq_config& cfg, const QjlEncodeArgs& a, hipStream_t s) {
  const float* s32 = reinterpret_cast<const float*>(a.s_rot + (size_t)a.m * 32 * LPU);
  const size_t lds = (size_t)a.m * 32 * LPU * sizeof(float);
  dim3 grid((unsigned)qjl_grid(a.n_units * LPU)), block(kBlock);
  const bool in32 = cfg.x_dtype == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (!in32 && !n32) hipLaunchKernelGGL((qjl_encode_kernel<BITS, LPU, false, false>), grid, block, lds, s, a, s32);
  if (!in32 && n32) hipLaunchKernelGGL((qjl_encode_kernel<BITS, LPU, false, true>), grid, block, lds, s, a, s32);
  if (in32 && !n32) hipLaunchKernelGGL((qjl_encode_kernel<BITS, LPU, true, false>), grid, block, lds, s, a, s32);
  if (in32 && n32) hipLaunchKernelGGL((qjl_encode_kernel<BITS, LPU, true, true>), grid, block, lds, s, a, s32);
  return hipGetLastError();
}

template <int BITS>
hipError_t qjl_encode128(const tq_config& cfg, const QjlEncodeArgs& a, hipStream_t s) {
  const float* s32 = reinterpret_cast<const float*>(a.s_rot + (size_t)a.m * 128);
  const size_t lds = (size_t)a.m * 128 * sizeof(float);
  const int64_t tiles = (a.n_units + 15) / 16;
  int64_t wgs = (tiles + kEncBlock / 64 - 1) / (kEncBlock / 64), cap = 2 * (int64_t)cu_count();
  dim3 grid((unsigned)(wgs < cap ? wgs : cap)), block(kEncBlock);
  const bool in32 = cfg.x_dtype == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (!in32 && !n32) hipLaunchKernelGGL((qjl_encode128_kernel<BITS, false, false>), grid, block, lds, s, a, s32);
  if (!in32 && n32) hipLaunchKernelGGL((qjl_encode128_kernel<BITS, false, true>), grid, block, lds, s, a, s32);
  if (in32 && !n32) hipLaunchKernelGGL((qjl_encode128_kernel<BITS, true, false>), grid, block, lds, s, a, s32);
  if (in32 && n32) hipLaunchKernelGGL((qjl_encode128_kernel<BITS, true, true>), grid, block, lds, s, a, s32);
  return hipGetLastError();
}

template <int BITS>
hipError_t qjl_encode_lpu(const tq_config& cfg, const QjlEncodeArgs& a, hipStream_t s) {
  if (cfg.dt == 128 && a.m % 32 == 0) return qjl_encode128<BITS>(cfg, a, s);
  switch (cfg.dt) {
    case 32: return qjl_encode_dispatch<BITS, 1>(cfg, a, s);
    case 64: return qjl_encode_dispatch<BITS, 2>(cfg, a, s);
    case 128: return qjl_encode_dispatch<BITS, 4>(cfg, a, s);
    default: return qjl_encode_dispatch<BITS, 8>(cfg, a, s);
  }
}

template <int BITS, int LPU, bool NC>
hipError_t qjl_decode_dispatch(const tq_config& cfg, const QjlDecodeArgs& a, tq_dtype yt, hipStream_t s) {
  const size_t lds = (size_t)a.m * 32 * LPU * sizeof(float);
  dim3 grid((unsigned)qjl_grid(a.n_units * LPU)), block(kBlock);
  const bool o32 = yt == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (!o32 && !n32) hipLaunchKernelGGL((qjl_decode_kernel<BITS, LPU, false, false, NC>), grid, block, lds, s, a);
  if (!o32 && n32) hipLaunchKernelGGL((qjl_decode_kernel<BITS, LPU, false, true, NC>), grid, block, lds, s, a);
  if (o32 && !n32) hipLaunchKernelGGL((qjl_decode_kernel<BITS, LPU, true, false, NC>), grid, block, lds, s, a);
  if (o32 && n32) hipLaunchKernelGGL((qjl_decode_kernel<BITS, LPU, true, true, NC>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t qjl_decode_lpu(const tq_config& cfg, const QjlDecodeArgs& a, bool nc, tq_dtype yt, hipStream_t s) {
  switch (cfg.dt) {
    case 32: return nc ? qjl_decode_dispatch<BITS, 1, true>(cfg, a, yt, s) : qjl_decode_dispatch<BITS, 1, false>(cfg, a, yt, s);
    case 64: return nc ? qjl_decode_dispatch<BITS, 2, true>(cfg, a, yt, s) : qjl_decode_dispatch<BITS, 2, false>(cfg, a, yt, s);
    case 128: return nc ? qjl_decode_dispatch<BITS, 4, true>(cfg, a, yt, s) : qjl_decode_dispatch<BITS, 4, false>(cfg, a, yt, s);
    default: return nc ? qjl_decode_dispatch<BITS, 8, true>(cfg, a, yt, s) : qjl_decode_dispatch<BITS, 8, false>(cfg, a, yt, s);
  }
}

}  // namespace

hipError_t launch_qjl_encode(const tq_config& cfg, const QjlEncodeArgs& a, hipStream_t s) {
  switch (cfg.bits) {
    case 1: return qjl_encode_lpu<1>(cfg, a, s);
    case 2: return qjl_encode_lpu<2>(cfg, a, s);
    case 3: return qjl_encode_lpu<3>(cfg, a, s);
    default: return qjl_encode_lpu<4>(cfg, a, s);
  }
}

hipError_t launch_qjl_decode(const tq_config& cfg, const QjlDecodeArgs& a, bool nc, tq_dtype y_dtype, hipStream_t s) {
  switch (cfg.bits) {
    case 1: return qjl_decode_lpu<1>(cfg, a, nc, y_dtype, s);
    case 2: return qjl_decode_lpu<2>(cfg, a, nc, y_dtype, s);
    case 3: return qjl_decode_lpu<3>(cfg, a, nc, y_dtype, s);
    default: return qjl_decode_lpu<4>(cfg, a, nc, y_dtype, s);
  }
}

}  // namespace tq
