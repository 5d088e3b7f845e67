// QJL stage kernels for gfx950: encode with the 1-bit residual sketch, and
// dequantize with the QJL correction ([Scratch] §2 "QJL residual";
// [README] two-stage description and combined estimator).
//
// The residual's sign bits sign((S r)_p) are only meaningful to the
// estimator if they agree with the exact projection.  head_dim 128 encodes in
// fp32 with the projection on fp32 MFMA, whose error (about 2e-7 of the
// residual norm) stays inside the 1e-6-of-rho band around z = 0; the other
// head sizes encode in float64, exact except within ~1e-15 of an edge.
// S~ = S D H (host-prepared) is staged in LDS; because H and D are symmetric
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

// Encode for head_dim = 128 in fp32, with the projection z = S~ e on fp32 MFMA
// (v_mfma_f32_16x16x4_f32).  Eight waves share one LDS copy of S~; a wave encodes 16 keys: lane l holds the 32
// coordinates 32 (l / 16) .. + 31 of key l % 16, so the A operand of k-step s
// is the lane's coordinate s and each lane packs one whole 32-group.  S~ sits
// in LDS as B-operand fragments, four k-steps per 16-byte read.  The sign bit
// [z_p >= 0] of (key 4 (l / 16) + r, p = 16 pt + l % 16) comes out of the
// accumulator as a wave ballot; the ballots are regrouped into each key's
// m-bit row through a small LDS table.  fp32 moves z by ~2e-7 of rho (the
// residual norm), so a sign bit can only differ from the exact one inside
// the |z| < 1e-6 rho band that the parity contract allows.
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kEncBlock = 512;  // 8 waves share one copy of S~ in LDS

template <int BITS, bool IN_F32, bool NORM_F32>
__global__ __launch_bounds__(kEncBlock) void qjl_encode128_kernel(QjlEncodeArgs a, const float* __restrict__ s_rot32) {
  constexpr int W = kEncBlock / 64;
  extern __shared__ v4f sfrag[];                  // [m/16][8][64]: S~[16 pt + ln%16][32 (ln/16) + 4 s4 + i]
  __shared__ uint64_t ballots[W][32];             // per wave: [pt * 4 + r]
  __shared__ float lvl_s[16];
  const int m = a.m, npt = m / 16, words = m / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < npt * 512; e += kEncBlock) {
    const int pt = e >> 9, s4 = (e >> 6) & 7, ln = e & 63;
    sfrag[e] = *reinterpret_cast<const v4f*>(s_rot32 + (16 * pt + (ln & 15)) * 128 + 32 * (ln >> 4) + 4 * s4);
  }
  if (tid < 16) lvl_s[tid] = (float)a.level[tid];
  __syncthreads();

  const int q = lane >> 4, kl = lane & 15;
  const uint32_t dword = q == 0 ? a.dbits[0] : q == 1 ? a.dbits[1] : q == 2 ? a.dbits[2] : a.dbits[3];
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
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float n = __builtin_sqrtf(ss);
    // unnormalised FWHT over the 128 coordinates: bits 0..4 in the lane, bits 5 and 6 across lanes 16 and 32 apart
    fwht32_inlane(v);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bool upper = (q >> b) & 1;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float o = __shfl_xor(v[j], 16 << b);
        v[j] = upper ? o - v[j] : v[j] + o;
      }
    }
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
    rr += __shfl_xor(rr, 16);
    rr += __shfl_xor(rr, 32);

    // z = S~ e' for the 16 keys, 16 projections per pass; ballots of z >= 0
    for (int pt = 0; pt < npt; ++pt) {
      v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
      const v4f* bf = sfrag + pt * 512 + lane;
#pragma unroll
      for (int s4 = 0; s4 < 8; ++s4) {
        const v4f b = bf[64 * s4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(v[4 * s4 + i], b[i], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint64_t bal = __ballot(acc[r] >= 0.0f);
        if (lane == 0) ballots[wave][pt * 4 + r] = bal;
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
  if (cfg.dt == 128 && a.m % 16 == 0) return qjl_encode128<BITS>(cfg, a, s);
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
