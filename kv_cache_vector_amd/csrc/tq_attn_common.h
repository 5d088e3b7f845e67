// Helpers shared by the attention kernels (tq_attn.hip: decode attention and the merge;
// tq_prefill.hip: many-row attention).  Device code only.
#pragma once

#include <hip/hip_fp16.h>

#include <cstdint>

namespace tq {
namespace attn {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) short lds_short;

constexpr int kTile = 64;     // tokens per tile
constexpr float kSlack = 8.0f;  // softmax weights relative to the running reference stay below e^8
// Initial softmax reference: finite, so a row whose tokens are all masked so far gets weights
// exp(-inf - kNoRef) = 0 rather than NaN, and any live score moves it.
constexpr float kNoRef = -1e30f;

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Reduction over the lanes that hold the same query head: the 16 lanes of a row
// (DPP: quad swaps, then rotations by 4 and 8 within the row) and, when S
// subtiles are stacked, the S rows that share the head (lanes l ^ 32 and
// l ^ 16, exchanged with the gfx950 permlane swaps).
template <int S, bool MAX>
__device__ __forceinline__ float head_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp<0x124>(v));  // row_ror:4
  v = op(v, dpp<0x128>(v));  // row_ror:8
  if (S >= 2) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    v = op(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  }
  if (S >= 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                    false, false);
    v = op(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  }
  return v;
}

// Word of a replicated pair table: entry ((w >> sh) & (2^width - 1)), copy selected by the
// lane's byte offset off (< 4 << lgc), i.e. byte address (entry << (lgc + 2)) | off.
__device__ __forceinline__ uint32_t lut_word(const uint32_t* table, uint32_t w, int sh, int width, int lgc,
                                             uint32_t off) {
  const int up = lgc + 2 - sh;
  const uint32_t mask = ((1u << width) - 1u) << (lgc + 2);
  const uint32_t shifted = up >= 0 ? (w << up) : (w >> -up);
  const uint32_t byte = (shifted & mask) | off;
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(table) + byte);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace attn
}  // namespace tq
