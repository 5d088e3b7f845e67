// Device helpers shared by the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang diagnostic ignored "-Winline-asm"

namespace tq {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Value of v held by lane (lane ^ mask), mask in {1, 2, 4}.  The partner
// lanes always belong to the same unit, so they are active together.
__device__ __forceinline__ float lane_xor(float v, int mask) {
  int iv = __builtin_bit_cast(int, v);
  int r;
  if (mask == 1)
    r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
  else if (mask == 2)
    r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
  else
    r = __builtin_amdgcn_ds_swizzle(iv, 0x1F | (4 << 10));   // bitmask swizzle: xor 4 within 32 lanes
  return __builtin_bit_cast(float, r);
}

__device__ __forceinline__ double lane_xor(double v, int mask) {
  uint64_t u = __builtin_bit_cast(uint64_t, v);
  float lo = __builtin_bit_cast(float, (uint32_t)u), hi = __builtin_bit_cast(float, (uint32_t)(u >> 32));
  lo = lane_xor(lo, mask);
  hi = lane_xor(hi, mask);
  return __builtin_bit_cast(double, (uint64_t)__builtin_bit_cast(uint32_t, lo) |
                                        ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32));
}

// One v_permlane16_swap / v_permlane32_swap exchange with the lane DIST (16 or 32) lanes away: in a lane
// whose DIST bit is clear, r0 is its own value and r1 its partner's; in the other lane of the pair the reverse.
template <int DIST>
__device__ __forceinline__ void lane_swap_pair(float v, float& r0, float& r1) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if constexpr (DIST == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    r0 = __builtin_bit_cast(float, (uint32_t)r[0]);
    r1 = __builtin_bit_cast(float, (uint32_t)r[1]);
  } else {
    static_assert(DIST == 32, "lanes 16 or 32 apart");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r0 = __builtin_bit_cast(float, (uint32_t)r[0]);
    r1 = __builtin_bit_cast(float, (uint32_t)r[1]);
  }
}

// Butterfly across lanes DIST apart: a + b in the lane whose DIST bit is clear (own a, partner b), a - b in its
// partner; s is +1 in the first lane and -1 in the second, so both are one fma of the swapped pair.
template <int DIST>
__device__ __forceinline__ float xlane_butterfly(float v, float s) {
  float r0, r1;
  lane_swap_pair<DIST>(v, r0, r1);
  return __builtin_fmaf(s, r1, r0);
}

// v plus the value of the lane DIST apart (the same sum in both lanes).
template <int DIST>
__device__ __forceinline__ float xlane_sum(float v) {
  float r0, r1;
  lane_swap_pair<DIST>(v, r0, r1);
  return r0 + r1;
}

// Sum of v over the LPU consecutive lanes of a unit (LPU in {1,2,4,8}).
template <int LPU, typename T>
__device__ __forceinline__ T unit_sum(T v) {
#pragma unroll
  for (int m = 1; m < LPU; m <<= 1) v += lane_xor(v, m);
  return v;
}

// In-register Walsh-Hadamard butterflies over the 32 values of one lane
// (coordinate bits 0..4), unnormalised: (a, b) -> (a + b, a - b).
template <typename T>
__device__ __forceinline__ void fwht32_inlane(T* v) {
#pragma unroll
  for (int bit = 1; bit < 32; bit <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & bit)) {
        T a = v[i], b = v[i | bit];
        v[i] = a + b;
        v[i | bit] = a - b;
      }
    }
  }
}

// Butterflies over coordinate bits 5.. held in lane bits 0.. (LPU lanes per
// unit): the lane whose bit is clear keeps a + b, its partner keeps a - b.
template <int LPU, typename T>
__device__ __forceinline__ void fwht_crosslane(T* v, int q) {
#pragma unroll
  for (int m = 1; m < LPU; m <<= 1) {
    const bool upper = (q & m) != 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      T p = lane_xor(v[i], m);
      v[i] = upper ? p - v[i] : v[i] + p;
    }
  }
}

// Sign mask of D for the coordinate pair (2i, 2i+1) of a lane's 32-group,
// placed on the two binary16 sign bits of a packed pair.
__device__ __forceinline__ uint32_t pair_sign_mask(uint32_t dword, int i) {
  return (((dword >> (2 * i)) & 1u) << 15) | (((dword >> (2 * i + 1)) & 1u) << 31);
}

// Place code (BITS wide) of coordinate j into a little-endian group stream.
template <int BITS>
__device__ __forceinline__ void put_code(uint32_t* w, int j, uint32_t code) {
  const int pos = BITS * j;
  w[pos >> 5] |= code << (pos & 31);
  if ((pos & 31) + BITS > 32) w[(pos >> 5) + 1] |= code >> (32 - (pos & 31));
}

template <int BITS>
__device__ __forceinline__ uint32_t get_code(const uint32_t* w, int j) {
  const int pos = BITS * j;
  uint32_t c = w[pos >> 5] >> (pos & 31);
  if ((pos & 31) + BITS > 32) c |= w[(pos >> 5) + 1] << (32 - (pos & 31));
  return c & ((1u << BITS) - 1);
}

// Asynchronous copies global -> LDS (global_load_lds): lane l's data lands at m0 + 16 l (12- and
// 16-byte copies) or m0 + 4 l (4- and 2-byte copies); m0 must be wave-uniform.  Written as inline
// assembly: the compiler neither waits for them nor orders later LDS reads behind them, so a copy
// for the next iteration can stay in flight across this iteration's stores; the caller waits by
// hand (vmcnt counts these copies, loads and stores together, in issue order).
// (An LDS-direct load needs one wait state after the SALU write of M0: the s_nop.)
template <int BYTES>
__device__ __forceinline__ void lds_copy(const void* g, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory");
  else if constexpr (BYTES == 12)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx3 %0, off" ::"v"(g), "s"(m0) : "memory");
  else if constexpr (BYTES == 4)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off" ::"v"(g), "s"(m0) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations have completed, nothing is
// waited for on the global-memory side, so prefetched data stays in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace tq
