// Encode and decode kernels (no QJL stage) for gfx950.
//
// Work split: one lane owns one 32-coordinate group (64 contiguous bytes of
// fp16 input, or 128 of fp32).  A unit of dt coordinates spans LPU = dt/32
// consecutive lanes, so coordinate c of a unit lives in lane c/32, register
// c%32.  The Walsh-Hadamard butterflies of coordinate bits 0..4 run inside a
// lane's registers; bits 5.. (dt >= 64) pair lanes of the same quad with DPP
// (or a swizzle for the third lane bit).  Norms are lane reductions.  The
// packed code word of a group is built in registers and written with one
// vector store, so loads and stores are contiguous across the wavefront.
//
// Encode ([Scratch] §2 steps 1-3; [Fork] "How it works"):
//   n = ||x||, yhat = H_unnorm (D x), code from comparing |yhat| with t_k * n
//   (t_k the N(0,1) cell edges; sqrt(dt) * y = yhat / n so no per-element
//   division is needed).
// Decode: c = level(code), optional norm correction, x~ = n * D H_unnorm c / dt
//   (or n * D H_unnorm c / (sqrt(dt) ||c||) with norm correction).
#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

__device__ __forceinline__ int64_t group_offset(int64_t g, int32_t gpr, int64_t ld, int32_t contiguous) {
  if (contiguous) return g * 32;
  const int64_t row = g / gpr;
  return row * ld + (g - row * gpr) * 32;
}

// Magnitude index m = #{k : t_k < a} over the 2^(BITS-1) - 1 positive edges T (binary search).
template <int BITS>
__device__ __forceinline__ uint32_t magnitude_index(float a, const float* T) {
  if constexpr (BITS == 1) {
    return 0u;
  } else if constexpr (BITS == 2) {
    return a > T[0] ? 1u : 0u;
  } else if constexpr (BITS == 3) {
    const bool c1 = a > T[1];
    const float t = c1 ? T[2] : T[0];
    return (c1 ? 2u : 0u) + (a > t ? 1u : 0u);
  } else {
    const bool c1 = a > T[3];
    const float t2 = c1 ? T[5] : T[1];
    const bool c2 = a > t2;
    const float lo = c1 ? T[4] : T[0];
    const float hi = c1 ? T[6] : T[2];
    const float t3 = c2 ? hi : lo;
    return (c1 ? 4u : 0u) + (c2 ? 2u : 0u) + (a > t3 ? 1u : 0u);
  }
}

template <int BITS, int LPU, bool IN_F32, bool NORM_F32>
__global__ __launch_bounds__(kBlock) void encode_kernel(EncodeArgs a) {
  const int q = (int)(threadIdx.x % LPU);
  const uint32_t dword = a.dbits[q];
  uint32_t dmask[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) dmask[i] = pair_sign_mask(dword, i);
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t g0 = (int64_t)blockIdx.x * kBlock; g0 < a.n_groups; g0 += stride) {
    const int64_t g = g0 + threadIdx.x;
    const bool valid = g < a.n_groups;
    float v[32];
    float ss = 0.0f;
    if constexpr (!IN_F32) {
      uint32_t w[16];
      if (valid) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.x) +
                                                        group_offset(g, a.groups_per_row, a.ld_x, a.contiguous));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          u32x4 t = __builtin_nontemporal_load(p + k);
          w[4 * k] = t.x;
          w[4 * k + 1] = t.y;
          w[4 * k + 2] = t.z;
          w[4 * k + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = 0u;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        half2v h = __builtin_bit_cast(half2v, w[i]);
        ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        h = __builtin_bit_cast(half2v, w[i] ^ dmask[i]);
        v[2 * i] = (float)h.x;
        v[2 * i + 1] = (float)h.y;
      }
    } else {
      if (valid) {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(a.x) +
                                                        group_offset(g, a.groups_per_row, a.ld_x, a.contiguous));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          // copy the elements out as integers first: bit-casting an ext-vector
          // element expression directly reads element 0 with this compiler
          const u32x4 t = __builtin_nontemporal_load(p + k);
          const uint32_t e0 = t.x, e1 = t.y, e2 = t.z, e3 = t.w;
          v[4 * k] = __builtin_bit_cast(float, e0);
          v[4 * k + 1] = __builtin_bit_cast(float, e1);
          v[4 * k + 2] = __builtin_bit_cast(float, e2);
          v[4 * k + 3] = __builtin_bit_cast(float, e3);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        ss = __builtin_fmaf(v[i], v[i], ss);
        v[i] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[i]) ^ (((dword >> i) & 1u) << 31));
      }
    }
    ss = unit_sum<LPU>(ss);
    const float n = __builtin_sqrtf(ss);
    float T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = a.thr[k] * n;

    fwht32_inlane(v);
    fwht_crosslane<LPU>(v, q);

    uint32_t word[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) word[k] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float y = v[j];
      const uint32_t neg = (y > 0.0f) ? 0u : 1u;  // a zero coordinate belongs to the lower cell
      const uint32_t code = (neg << (BITS - 1)) | magnitude_index<BITS>(__builtin_fabsf(y), T);
      put_code<BITS>(word, j, code);
    }
    if (valid) {
      uint32_t* cp = reinterpret_cast<uint32_t*>(a.codes + g * (4 * BITS));
#pragma unroll
      for (int k = 0; k < BITS; ++k) __builtin_nontemporal_store(word[k], cp + k);
      if (q == 0) {
        const int64_t u = g / LPU;
        if constexpr (NORM_F32)
          static_cast<float*>(a.norms)[u] = n;
        else
          static_cast<__half*>(a.norms)[u] = __float2half_rn(n);
      }
    }
  }
}

template <int BITS, int LPU, bool OUT_F32, bool NORM_F32, bool NC>
__global__ __launch_bounds__(kBlock) void decode_kernel(DecodeArgs a) {
  __shared__ float lut[16];
  if (threadIdx.x < 16) lut[threadIdx.x] = a.level[threadIdx.x];
  __syncthreads();
  const int q = (int)(threadIdx.x % LPU);
  const uint32_t dword = a.dbits[q];
  uint32_t dmask[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) dmask[i] = pair_sign_mask(dword, i);
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t g0 = (int64_t)blockIdx.x * kBlock; g0 < a.n_groups; g0 += stride) {
    const int64_t g = g0 + threadIdx.x;
    const bool valid = g < a.n_groups;
    uint32_t word[BITS];
    float n = 0.0f;
    if (valid) {
      const uint32_t* cp = reinterpret_cast<const uint32_t*>(a.codes + g * (4 * BITS));
#pragma unroll
      for (int k = 0; k < BITS; ++k) word[k] = __builtin_nontemporal_load(cp + k);
      const int64_t u = g / LPU;
      if constexpr (NORM_F32)
        n = static_cast<const float*>(a.norms)[u];
      else
        n = __half2float(static_cast<const __half*>(a.norms)[u]);
    } else {
#pragma unroll
      for (int k = 0; k < BITS; ++k) word[k] = 0u;
    }
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = lut[get_code<BITS>(word, j)];
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
    if constexpr (!OUT_F32) {
      uint32_t o[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const __half lo = __float2half_rn(v[2 * i] * scale);
        const __half hi = __float2half_rn(v[2 * i + 1] * scale);
        o[i] = ((uint32_t)__half_as_ushort(lo) | ((uint32_t)__half_as_ushort(hi) << 16)) ^ dmask[i];
      }
      u32x4* p = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.y) +
                                          group_offset(g, a.groups_per_row, a.ld_y, a.contiguous));
#pragma unroll
      for (int k = 0; k < 4; ++k)
        __builtin_nontemporal_store(u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]}, p + k);
    } else {
      uint32_t o[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        o[i] = __builtin_bit_cast(uint32_t, v[i] * scale) ^ (((dword >> i) & 1u) << 31);
      u32x4* p = reinterpret_cast<u32x4*>(static_cast<float*>(a.y) +
                                          group_offset(g, a.groups_per_row, a.ld_y, a.contiguous));
#pragma unroll
      for (int k = 0; k < 8; ++k)
        __builtin_nontemporal_store(u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]}, p + k);
    }
  }
}

// Workgroups per launch: enough resident waves to cover HBM latency, with a
// grid-stride loop over the rest (amortises the per-lane set-up).
int64_t grid_for(int64_t n_groups) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      cus = prop.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  int64_t need = (n_groups + kBlock - 1) / kBlock;
  int64_t cap = (int64_t)cus * 16;
  return need < cap ? need : cap;
}

template <int BITS, int LPU>
hipError_t encode_dispatch_dtype(const tq_config& cfg, const EncodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)grid_for(a.n_groups)), block(kBlock);
  const bool in32 = cfg.x_dtype == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (!in32 && !n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, false, false>), grid, block, 0, s, a);
  if (!in32 && n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, false, true>), grid, block, 0, s, a);
  if (in32 && !n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, true, false>), grid, block, 0, s, a);
  if (in32 && n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, true, true>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t encode_dispatch_lpu(const tq_config& cfg, const EncodeArgs& a, hipStream_t s) {
  switch (cfg.dt) {
    case 32: return encode_dispatch_dtype<BITS, 1>(cfg, a, s);
    case 64: return encode_dispatch_dtype<BITS, 2>(cfg, a, s);
    case 128: return encode_dispatch_dtype<BITS, 4>(cfg, a, s);
    default: return encode_dispatch_dtype<BITS, 8>(cfg, a, s);
  }
}

template <int BITS, int LPU, bool NC>
hipError_t decode_dispatch_dtype(const tq_config& cfg, const DecodeArgs& a, tq_dtype yt, hipStream_t s) {
  dim3 grid((unsigned)grid_for(a.n_groups)), block(kBlock);
  const bool o32 = yt == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (!o32 && !n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, false, false, NC>), grid, block, 0, s, a);
  if (!o32 && n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, false, true, NC>), grid, block, 0, s, a);
  if (o32 && !n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, true, false, NC>), grid, block, 0, s, a);
  if (o32 && n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, true, true, NC>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BITS, int LPU>
hipError_t decode_dispatch_nc(const tq_config& cfg, const DecodeArgs& a, bool nc, tq_dtype yt, hipStream_t s) {
  return nc ? decode_dispatch_dtype<BITS, LPU, true>(cfg, a, yt, s) : decode_dispatch_dtype<BITS, LPU, false>(cfg, a, yt, s);
}

template <int BITS>
hipError_t decode_dispatch_lpu(const tq_config& cfg, const DecodeArgs& a, bool nc, tq_dtype yt, hipStream_t s) {
  switch (cfg.dt) {
    case 32: return decode_dispatch_nc<BITS, 1>(cfg, a, nc, yt, s);
    case 64: return decode_dispatch_nc<BITS, 2>(cfg, a, nc, yt, s);
    case 128: return decode_dispatch_nc<BITS, 4>(cfg, a, nc, yt, s);
    default: return decode_dispatch_nc<BITS, 8>(cfg, a, nc, yt, s);
  }
}

}  // namespace

hipError_t launch_encode(const tq_config& cfg, const EncodeArgs& a, hipStream_t s) {
  switch (cfg.bits) {
    case 1: return encode_dispatch_lpu<1>(cfg, a, s);
    case 2: return encode_dispatch_lpu<2>(cfg, a, s);
    case 3: return encode_dispatch_lpu<3>(cfg, a, s);
    default: return encode_dispatch_lpu<4>(cfg, a, s);
  }
}

hipError_t launch_decode(const tq_config& cfg, const DecodeArgs& a, bool nc, tq_dtype y_dtype, hipStream_t s) {
  switch (cfg.bits) {
    case 1: return decode_dispatch_lpu<1>(cfg, a, nc, y_dtype, s);
    case 2: return decode_dispatch_lpu<2>(cfg, a, nc, y_dtype, s);
    case 3: return decode_dispatch_lpu<3>(cfg, a, nc, y_dtype, s);
    default: return decode_dispatch_lpu<4>(cfg, a, nc, y_dtype, s);
  }
}

}  // namespace tq
