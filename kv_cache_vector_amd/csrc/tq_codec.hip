// Encode and decode kernels (no QJL stage) for gfx950.
//
// Encode ([Scratch] §2 steps 1-3; [Fork] "How it works"):
//   n = ||x||, yhat = H_unnorm (D x); since sqrt(dt) * y = yhat / n the cell
//   of a coordinate is found by comparing |yhat| with t_k * n (t_k the N(0,1)
//   cell edges), with no per-element division.  The code bits are produced
//   most-significant first and shifted straight into the packed word, so
//   bucketize and bit-pack are one chain: per bit one compare and one
//   add-with-carry (w = 2 w + [|yhat| > t]); the sign bit is shifted in from
//   the float's sign.
// Decode: c = level(code), optional norm correction, x~ = n D H_unnorm c / dt
//   (with norm correction n D H_unnorm c / ||H_unnorm c||).
//
// Both directions work on 32-coordinate groups: a unit of dt coordinates is
// LPU = dt / 32 consecutive groups, and H_dt = H_LPU (x) H_32.  fp16 rows are
// encoded, and every decode runs, with the 32-point transforms of 32 groups at
// a time on v_mfma_f32_32x32x16_f16 against the +-1 matrix (exact products,
// fp32 sums) and the LPU-point part as butterflies between neighbouring lanes
// (encode_mfma_kernel, decode_mfma_kernel).  fp32 rows are encoded by
// encode_kernel, one group per lane with in-register fp32 butterflies (the
// fp32 inputs do not fit an exact fp16 MFMA operand).
//
// Memory: each wave moves its 64 groups through a private LDS tile, so every
// global load and store instruction of the rows covers one contiguous 1 KiB
// span across the wavefront (lane l <-> bytes [16 l, 16 l + 16)); the tile
// re-deals the 16-byte chunks so that each lane ends up with its own group.
#include <hip/hip_fp16.h>

#include <atomic>

#include "tq_device.h"
#include "tq_internal.h"

// the LDS copy statements set M0 themselves; nothing else in these kernels uses it
#pragma clang diagnostic ignored "-Winline-asm"

namespace tq {
namespace {

constexpr int kWaves = kBlock / 64;

// Streaming hints and launch widths (nontemporal loads and stores, 32 workgroups per compute unit
// for encode, 96 for the store-heavy block-32 decode and 32 for decodes of longer units measured
// fastest on MI355X).
#ifndef TQ_LOAD_NT
#define TQ_LOAD_NT 1
#endif
#ifndef TQ_STORE_NT
#define TQ_STORE_NT 1
#endif
// Encode grids: at most 56 workgroups per compute unit (each a persistent loop over 64-group tiles per
// wave).  Measured in a captured K+V step against 32: 2 % faster at 3 bits, 2 % at 4, 4 % for 8-bit keys,
// records no slower; 80 starts to slow the records.
#ifndef TQ_GRID_PER_CU
#define TQ_GRID_PER_CU 56
#endif
#ifndef TQ_DEC_GRID_PER_CU
#define TQ_DEC_GRID_PER_CU 96
#endif
#ifndef TQ_DEC_LGC
#define TQ_DEC_LGC 1
#endif
#ifndef TQ_DEC_GRID_PER_CU_UNITS
#define TQ_DEC_GRID_PER_CU_UNITS 32
#endif

__device__ __forceinline__ u32x4 load_stream(const u32x4* p) {
#if TQ_LOAD_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

__device__ __forceinline__ void store_stream(u32x4 v, u32x4* p) {
#if TQ_STORE_NT
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// Element offset of group g: rows of ld elements, gpr groups per row.
template <bool CONTIG>
__device__ __forceinline__ int64_t group_offset(int64_t g, int32_t gpr, int64_t ld) {
  if constexpr (CONTIG) {
    return g * 32;
  } else {
    const int64_t row = g / gpr;
    return row * ld + (g - row * gpr) * 32;
  }
}

// Load the wave's 64 groups (CH 16-byte chunks each) from global memory into
// registers: instruction k moves chunks 64k .. 64k+63 of the wave's span, so
// each instruction covers one contiguous 1 KiB when rows are contiguous.  In
// the last, partial wave the groups past the end re-read the last group (the
// caller has w0 < n_groups): every load stays in bounds, full waves take no
// branch, and those groups' results are never stored.
template <int CH, int ES, bool CONTIG>
__device__ __forceinline__ void stage_load(u32x4* t, const char* base, int64_t w0, int64_t n_groups, int32_t gpr,
                                           int64_t ld, int lane) {
  const int64_t room = n_groups - 1 - w0;
  const uint32_t last = room < 63 ? (uint32_t)room : 63u;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int ci = 64 * k + lane;
    const int c = ci % CH;
    const uint32_t grp = min((uint32_t)(ci / CH), last);
    if constexpr (CONTIG) {  // uniform base + unsigned 32-bit lane offset
      const char* wb = base + (int64_t)ES * 32 * w0;
      t[k] = load_stream(reinterpret_cast<const u32x4*>(wb + (grp * (ES * 32u) + 16u * (uint32_t)c)));
    } else {
      t[k] = load_stream(reinterpret_cast<const u32x4*>(base + ES * group_offset<CONTIG>(w0 + grp, gpr, ld) + 16 * c));
    }
  }
}

// ... and their copy into the wave's LDS tile, group grp at tile + grp * PITCH
template <int CH, int PITCH>
__device__ __forceinline__ void stage_put(uint8_t* tile, const u32x4* t, int lane) {
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int ci = 64 * k + lane;
    *reinterpret_cast<u32x4*>(tile + (ci / CH) * PITCH + 16 * (ci % CH)) = t[k];
  }
}

// Both: every load of a full wave goes out before the first LDS write.
template <int CH, int PITCH, int ES, bool CONTIG>
__device__ __forceinline__ void stage_in(uint8_t* tile, const char* base, int64_t w0, int64_t n_groups, int32_t gpr,
                                         int64_t ld, int lane) {
  u32x4 t[CH];
  stage_load<CH, ES, CONTIG>(t, base, w0, n_groups, gpr, ld, lane);
  stage_put<CH, PITCH>(tile, t, lane);
}

// Write the wave's 64 staged groups from the LDS tile to global memory, one
// contiguous 1 KiB span per store instruction (the mirror of stage_in).
template <int CH, int PITCH, int ES, bool CONTIG>
__device__ __forceinline__ void stage_out(const uint8_t* tile, char* base, int64_t w0, int64_t n_groups, int32_t gpr,
                                          int64_t ld, int lane) {
  u32x4 t[CH];
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int ci = 64 * k + lane;
    t[k] = *reinterpret_cast<const u32x4*>(tile + (ci / CH) * PITCH + 16 * (ci % CH));
  }
  const bool full = w0 + 64 <= n_groups;
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int ci = 64 * k + lane;
    const int grp = ci / CH, c = ci % CH;
    if (full || w0 + grp < n_groups)
      store_stream(t[k], reinterpret_cast<u32x4*>(base + ES * group_offset<CONTIG>(w0 + grp, gpr, ld) + 16 * c));
  }
}

// w = 2 w + [|y| > t]; returns the lane mask of the comparison.  On gfx950 a VALU read of an SGPR
// (as carry-in or lane mask) needs two wait states after a VALU write of that SGPR, but none after
// an SALU write, and an SALU read of a VALU-written SGPR needs none either: the mask goes through
// a scalar copy into another register pair, which the add and every later select read.
__device__ __forceinline__ uint64_t shift_in_gt(uint32_t& w, float y, float t) {
  uint64_t c, m, carry;
  asm("v_cmp_gt_f32_e64 %1, |%4|, %5\n\t"
      "s_mov_b64 %2, %1\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, %0, %2"
      : "+v"(w), "=&s"(c), "=&s"(m), "=&s"(carry)
      : "v"(y), "v"(t));
  return m;
}

// The two magnitude bits of a 3-bit code: with c_k = [|y| > t_k] and t_0 < t_1 < t_2 (so
// c_0 >= c_1 >= c_2), the magnitude index is c_0 + c_1 + c_2, whose high bit is c_1 and whose low
// bit is c_0 ^ c_1 ^ c_2.  Three independent compares, the parity on the scalar unit, and each
// mask read by the adds is written by a scalar instruction (no wait states; see shift_in_gt).
__device__ __forceinline__ void shift_in_mag3(uint32_t& w1, uint32_t& w0, bool same, float y, const float* T) {
  uint64_t c0, c1, c2, m1, m0, carry;
  if (same) {
    asm("v_cmp_gt_f32_e64 %2, |%7|, %9\n\t"
        "v_cmp_gt_f32_e64 %1, |%7|, %8\n\t"
        "v_cmp_gt_f32_e64 %3, |%7|, %10\n\t"
        "s_mov_b64 %4, %2\n\t"
        "s_xor_b64 %5, %1, %2\n\t"
        "s_xor_b64 %5, %5, %3\n\t"
        "v_addc_co_u32_e64 %0, %6, %0, %0, %4\n\t"
        "v_addc_co_u32_e64 %0, %6, %0, %0, %5"
        : "+v"(w1), "=&s"(c0), "=&s"(c1), "=&s"(c2), "=&s"(m1), "=&s"(m0), "=&s"(carry)
        : "v"(y), "v"(T[0]), "v"(T[1]), "v"(T[2])
        : "scc");
  } else {
    asm("v_cmp_gt_f32_e64 %3, |%8|, %10\n\t"
        "v_cmp_gt_f32_e64 %2, |%8|, %9\n\t"
        "v_cmp_gt_f32_e64 %4, |%8|, %11\n\t"
        "s_mov_b64 %5, %3\n\t"
        "s_xor_b64 %6, %2, %3\n\t"
        "s_xor_b64 %6, %6, %4\n\t"
        "v_addc_co_u32_e64 %0, %7, %0, %0, %5\n\t"
        "v_addc_co_u32_e64 %1, %7, %1, %1, %6"
        : "+v"(w1), "+v"(w0), "=&s"(c0), "=&s"(c1), "=&s"(c2), "=&s"(m1), "=&s"(m0), "=&s"(carry)
        : "v"(y), "v"(T[0]), "v"(T[1]), "v"(T[2])
        : "scc");
  }
}

// w = (w << 1) | signbit(y)
__device__ __forceinline__ void shift_in_sign(uint32_t& w, float y) {
  w = __builtin_amdgcn_alignbit(w, __builtin_bit_cast(uint32_t, y), 31);
}

// Shift the code of one coordinate (1 to 3 bits; 4 and 8 bits use the bucket
// table) most significant bit first into the packed words.  Bit p of the
// 32-coordinate group (p = BITS*j + k) lives in word p/32; since the caller
// walks j downwards and the bits of one code from the top, every word
// receives its bits from bit 31 down to bit 0.
//
// y may come straight from an MFMA, and inline asm is exempt from the compiler's
// checks of MFMA-result hazards, so every compare must depend on a compiler-made
// read of y: the sign shift into the same word, or, where a 3-bit code's first
// magnitude bit starts the next lower word, a copy of |y| made here (one
// instruction per 32 bits).
template <int BITS>
__device__ __forceinline__ void code_chain(uint32_t* word, int j, float y, const float* T) {
  const int p_top = BITS * j + BITS - 1;
  shift_in_sign(word[p_top >> 5], y);
  if constexpr (BITS == 2) {
    shift_in_gt(word[(p_top - 1) >> 5], y, T[0]);
  } else if constexpr (BITS == 3) {
    const float ym = (p_top & 31) == 0 ? __builtin_fabsf(y) : y;
    shift_in_mag3(word[(p_top - 1) >> 5], word[(p_top - 2) >> 5], (p_top - 1) >> 5 == (p_top - 2) >> 5, ym, T);
  }
}

// Stored words of a zero unit: every coordinate takes the cell just below 0,
// i.e. code (sign 1, magnitude 0).
template <int BITS>
__device__ __forceinline__ uint32_t zero_unit_word(int k) {
  uint32_t w = 0;
  for (int j = 0; j < 32; ++j) {
    const int p = BITS * j + BITS - 1;
    if ((p >> 5) == k) w |= 1u << (p & 31);
  }
  return w;
}

// fp16 pair -> (lo + hi, lo - hi) in fp32 with one rounding each (fma_mix reads the halves directly).
__device__ __forceinline__ void butterfly_f16_pair(uint32_t w, float& s, float& d) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(s) : "v"(w));
  asm("v_fma_mix_f32 %0, -%1, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w));
}

// In-register butterflies over coordinate bits FIRST..4 (bits below FIRST already done).
template <int FIRST>
__device__ __forceinline__ void fwht32_from(float* v) {
#pragma unroll
  for (int bit = 1 << FIRST; bit < 32; bit <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (!(i & bit)) {
        const float a = v[i], b = v[i | bit];
        v[i] = a + b;
        v[i | bit] = a - b;
      }
    }
  }
}

// Records of the fork's block format ([Fork] "GGML Types"): per 32-coordinate
// group the fp16 norm of its unit, then the group's 4*BITS code bytes, so
// R = 2 + 4*BITS bytes (14 at 3 bits, 18 at 4).  R is even, so a record is a
// run of 16-bit words.  A full wave's 64 records are 64 R = 16 (4 R) bytes,
// 16-byte aligned (wave starts are multiples of 64 groups), and move between
// LDS and memory as 4 R whole 16-byte chunks.
template <int BITS>
struct Record {
  static constexpr int kBytes = 2 + 4 * BITS;
  static constexpr int kChunks = 4 * kBytes;
};

template <int BITS>
__device__ __forceinline__ void put_record(uint16_t* r, uint16_t norm_bits, const uint32_t* word) {
  r[0] = norm_bits;
#pragma unroll
  for (int k = 0; k < BITS; ++k) {
    r[1 + 2 * k] = (uint16_t)word[k];
    r[2 + 2 * k] = (uint16_t)(word[k] >> 16);
  }
}

template <int BITS>
__device__ __forceinline__ float get_record(const uint16_t* r, uint32_t* word) {
#pragma unroll
  for (int k = 0; k < BITS; ++k) word[k] = (uint32_t)r[1 + 2 * k] | ((uint32_t)r[2 + 2 * k] << 16);
  return __half2float(__ushort_as_half(r[0]));
}

// Bucket tables of the 4- and 8-bit encoders.  |u| = |y| / n is binned uniformly with kb = bin_scale / n
// bins per unit of |y| (bin_scale is 1.6 bins per narrowest cell, so consecutive edges lie at least 1.6
// bins apart).  The bin index of a coordinate is |y| kb rounded or truncated to an integer, so when it
// comes out as i, |y| kb lies in [i - 0.51, i + 1.01]: a window of 1.52 bins that holds at most one
// edge.  Entry i holds the number m0 of edges at or below the window's start and the first edge e above
// it (+inf past the last one); the magnitude is m0 + [|y| > e n], the comparison the narrow codes make
// against t n, so the codes do not depend on the binning.  Entries: 256 at 4 bits (every index a
// saturating byte conversion can give), n_bins at 8 bits (indices clamped to the last, whose window
// starts above every edge).
template <int BITS>
__device__ __forceinline__ void setup_lut(const EncodeArgs& a, float* edge, uint2* lut) {
  constexpr int H = 1 << (BITS - 1);  // edges t_1 .. t_{H-1}, then thr[H-1] = +inf
  if constexpr (BITS == 4) {  // seven edges: counted straight from the arguments
    for (int b = threadIdx.x; b < kLutEntries4; b += kBlock) {
      const float x = ((float)b - 0.51f) / a.bin_scale;
      uint32_t m0 = 0;
      float e = __builtin_inff();
#pragma unroll
      for (int k = 0; k < H - 1; ++k) {
        const float t = a.thr[k];
        if (t <= x)
          ++m0;
        else
          e = __builtin_fminf(e, t);
      }
      lut[b] = make_uint2(__builtin_bit_cast(uint32_t, e), m0);
    }
    __syncthreads();
    return;
  }
  for (int i = threadIdx.x; i < H; i += kBlock) edge[i] = a.thr[i];
  __syncthreads();
  for (int b = threadIdx.x; b < a.n_bins; b += kBlock) {
    const float x = ((float)b - 0.51f) / a.bin_scale;
    int lo = 0, hi = H - 1;  // first k with t_k > x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (edge[mid] <= x)
        lo = mid + 1;
      else
        hi = mid;
    }
    lut[b] = make_uint2(__builtin_bit_cast(uint32_t, edge[lo]), (uint32_t)lo);
  }
  __syncthreads();
}

// w = (w << SHIFT) + m0 + [|y| > t], the comparison's lane mask going through a scalar copy (see
// shift_in_gt).
template <int SHIFT>
__device__ __forceinline__ void shift_in_mag_lut(uint32_t& w, uint32_t m0, float y, float t) {
  uint64_t c, m, carry;
  asm("v_cmp_gt_f32_e64 %1, |%4|, %5\n\t"
      "s_mov_b64 %2, %1\n\t"
      "v_lshl_add_u32 %0, %0, %7, %6\n\t"
      "v_addc_co_u32_e64 %0, %3, %0, 0, %2"
      : "+v"(w), "=&s"(c), "=&s"(m), "=&s"(carry)
      : "v"(y), "v"(t), "v"(m0), "i"(SHIFT));
}

// The bucket-table entry of coordinate y (kb = bins per unit of |y|; top: the last entry at 8 bits).
template <int BITS>
__device__ __forceinline__ uint2 lut_entry(float y, float kb, float top, const uint2* lut) {
  const float u = __builtin_fabsf(y) * kb;
  if constexpr (BITS == 4)
    return lut[__builtin_amdgcn_cvt_pk_u8_f32(u, 0, 0u)];
  else
    return lut[(uint32_t)__builtin_fminf(u, top)];
}

// Codes of coordinates J-1 .. 0 of v (sign, then magnitude), shifted into their words most significant
// bit first like code_chain (BITS divides 32, so a code never straddles two words).  The table reads go
// out four at a time ahead of the compares that use them (the 4-bit block-32 encode measured 2-4 %
// faster than with one; 8 and 16 no better).  Each compare reads y after the compiler-made product
// |y| kb that its threshold depends on.
template <int BITS, int J>
__device__ __forceinline__ void code_lut(uint32_t* word, const float* v, float n, float kb, float top,
                                         const uint2* lut) {
  constexpr int LB = 4;
#pragma unroll
  for (int j0 = J - 1; j0 >= 0; j0 -= LB) {
    uint2 e[LB];
#pragma unroll
    for (int k = 0; k < LB; ++k) e[k] = lut_entry<BITS>(v[j0 - k], kb, top, lut);
#pragma unroll
    for (int k = 0; k < LB; ++k) {
      const int j = j0 - k;
      uint32_t& w = word[(BITS * j) >> 5];
      shift_in_sign(w, v[j]);
      shift_in_mag_lut<BITS - 1>(w, e[k].y, v[j], __builtin_bit_cast(float, e[k].x) * n);
    }
  }
}

template <int BITS, int LPU, bool IN_F32, bool NORM_F32, bool CONTIG, bool AOS>
__global__ __launch_bounds__(kBlock) void encode_kernel(EncodeArgs a) {
  static_assert(!(AOS && NORM_F32), "records carry fp16 norms");
  static_assert(BITS <= 4 || BITS == 8, "1..4 or 8 bits");
  constexpr bool LUT = BITS == 4 || BITS == 8;
  __shared__ float edge[BITS == 8 ? 128 : 1];
  __shared__ uint2 lut[BITS == 4 ? kLutEntries4 : BITS == 8 ? kMaxBins8 : 1];
  if constexpr (LUT) setup_lut<BITS>(a, edge, lut);
  constexpr int CH = IN_F32 ? 8 : 4;  // 16-byte chunks per group
  constexpr int PITCH = 16 * CH + 16;  // LDS bytes per staged group (padded against bank conflicts)
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][64 * PITCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint8_t* tile = stage[wave];
  const int q = lane % LPU;
  const uint32_t dword = a.dbits[q];
  float thr[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) thr[k] = a.thr[k];
  const char* xbase = static_cast<const char*>(a.x);
  constexpr int ES = IN_F32 ? 4 : 2;

  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t w0 = (int64_t)blockIdx.x * kBlock + wave * 64; w0 < a.n_groups; w0 += stride) {
    // ---- coalesced load of the wave's 64 groups, re-dealt through LDS ----
    stage_in<CH, PITCH, ES, CONTIG>(tile, xbase, w0, a.n_groups, a.groups_per_row, a.ld_x, lane);
    __builtin_amdgcn_wave_barrier();
    uint32_t w[4 * CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const u32x4 t = *reinterpret_cast<const u32x4*>(tile + lane * PITCH + 16 * c);
      w[4 * c] = t.x;
      w[4 * c + 1] = t.y;
      w[4 * c + 2] = t.z;
      w[4 * c + 3] = t.w;
    }
    __builtin_amdgcn_wave_barrier();

    const int64_t g = w0 + lane;
    const bool valid = g < a.n_groups;
    float v[32];
    float ss = 0.0f;
    if constexpr (!IN_F32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const half2v h = __builtin_bit_cast(half2v, w[i]);
        ss = __builtin_amdgcn_fdot2(h, h, ss, false);
        butterfly_f16_pair(w[i] ^ pair_sign_mask(dword, i), v[2 * i], v[2 * i + 1]);
      }
      fwht32_from<1>(v);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float x = __builtin_bit_cast(float, w[i]);
        ss = __builtin_fmaf(x, x, ss);
        v[i] = __builtin_bit_cast(float, w[i] ^ (((dword >> i) & 1u) << 31));
      }
      fwht32_from<0>(v);
    }
    ss = unit_sum<LPU>(ss);
    const float n = __builtin_sqrtf(ss);
    fwht_crosslane<LPU>(v, q);
    float T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = thr[k] * n;

    uint32_t word[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) word[k] = 0u;
    if constexpr (LUT) {
      const float kb = n > 0.0f ? a.bin_scale * __builtin_amdgcn_rcpf(n) : 0.0f;  // 1 ulp: only picks the bin
      const float top = (float)(a.n_bins - 1);
      code_lut<BITS, 32>(word, v, n, kb, top, lut);
    } else {
#pragma unroll
      for (int j = 31; j >= 0; --j) code_chain<BITS>(word, j, v[j], T);
    }
    if (n == 0.0f) {
#pragma unroll
      for (int k = 0; k < BITS; ++k) word[k] = zero_unit_word<BITS>(k);
    }
    if constexpr (AOS) {
      // every group of a unit carries the unit's norm (each lane of the unit holds n)
      constexpr int R = Record<BITS>::kBytes;
      const uint16_t nb = __half_as_ushort(__float2half_rn(n));
      if (w0 + 64 <= a.n_groups) {
        put_record<BITS>(reinterpret_cast<uint16_t*>(tile + R * lane), nb, word);
        __builtin_amdgcn_wave_barrier();
        u32x4* out = reinterpret_cast<u32x4*>(a.codes + w0 * R);
#pragma unroll
        for (int c = lane; c < Record<BITS>::kChunks; c += 64)
          store_stream(*reinterpret_cast<const u32x4*>(tile + 16 * c), out + c);
        __builtin_amdgcn_wave_barrier();
      } else if (valid) {
        put_record<BITS>(reinterpret_cast<uint16_t*>(a.codes + g * R), nb, word);
      }
    } else if (valid) {
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

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

// Record word k of a 32-coordinate group whose coordinates 0..15 were packed into lo[] and
// 16..31 into hi[] (16 BITS-bit codes each, little-endian bit streams).
template <int BITS>
__device__ __forceinline__ uint32_t join_halves(const uint32_t* lo, const uint32_t* hi, int k) {
  if constexpr (BITS == 1) {
    return (lo[0] & 0xFFFFu) | (hi[0] << 16);
  } else if constexpr (BITS == 2) {
    return k == 0 ? lo[0] : hi[0];
  } else if constexpr (BITS == 3) {
    return k == 0 ? lo[0] : k == 1 ? (lo[1] & 0xFFFFu) | (hi[0] << 16) : (hi[0] >> 16) | (hi[1] << 16);
  } else {  // 4 or 8 bits: whole words per half
    constexpr int W = 16 * BITS / 32;
    return k < W ? lo[k] : hi[k - W];
  }
}

// Butterflies of coordinate bits 5.. across the LPU consecutive group columns of a unit (lanes
// l ^ m, m < LPU, of the same lane half): the lane with bit m clear keeps a + b, its partner a - b.
template <int LPU, int N>
__device__ __forceinline__ void unit_butterflies(float* v, int q) {
#pragma unroll
  for (int m = 1; m < LPU; m <<= 1) {
    const bool upper = (q & m) != 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float p = lane_xor(v[i], m);
      v[i] = upper ? p - v[i] : v[i] + p;
    }
  }
}

// Encode of fp16 rows with the 32-point Walsh-Hadamard transforms on MFMA.
// For a set of 32 groups, Yhat^T = M X^T with M = H_unnorm (entries +-1,
// exact in fp16) and X the fp16 inputs: products are exact and the sums are
// accumulated in fp32, two v_mfma_f32_32x32x16_f16 per set and two sets per
// wave (the wave's 64 groups, staged through LDS as in encode_kernel).  The
// rows of M are permuted so that output lane half h holds coordinates
// 16h .. 16h+15 of its group in accumulator registers 0..15.
// A unit of dt = 32 LPU coordinates is LPU consecutive groups, i.e. LPU
// neighbouring group columns: H_dt = H_LPU (x) H_32 in Sylvester order, so the
// remaining log2(LPU) butterfly stages pair lanes l ^ 1, l ^ 2, l ^ 4.  The
// sign flip D folds into M when a unit is one group (LPU = 1); otherwise each
// group column has its own part of D, applied to the fp16 inputs' sign bits.
// Each lane bucketizes and packs its 16 coordinates with the
// most-significant-first chain of encode_kernel, and one permlane32 swap per
// segment word hands every lane both halves of the group it stores.  The norm
// comes from the fp16 inputs (dot2 of the lane's 16 values, the partner
// lane's, and the unit's other groups).  Outputs: code and norm planes, or
// (AOS) the fork's records, assembled in the wave's LDS tile and stored as
// whole 16-byte chunks; 8-bit codes also go through the tile so that every
// store instruction covers 1 KiB.
template <int BITS, int LPU, bool NORM_F32, bool CONTIG, bool AOS>
__global__ __launch_bounds__(kBlock) void encode_mfma_kernel(EncodeArgs a) {
  static_assert(!(AOS && NORM_F32), "records carry fp16 norms");
  constexpr int CH = 4, PITCH = 16 * CH + 16;
  constexpr int SEGW = (16 * BITS + 31) / 32;  // words of one lane's 16-code segment
  constexpr bool B8 = BITS == 8;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][64 * PITCH];
  constexpr bool LUT = BITS == 4 || BITS == 8;
  __shared__ float edge[BITS == 8 ? 128 : 1];
  __shared__ uint2 lut[BITS == 4 ? kLutEntries4 : BITS == 8 ? kMaxBins8 : 1];
  if constexpr (LUT) setup_lut<BITS>(a, edge, lut);
  // 4 and 8 bits: the next tile's loads go out before this tile's compute and stores (measured
  // faster at 4 and 8 bits, slower at 3)
  constexpr bool PIPE = BITS == 4 || BITS == 8;
  // Units of 2 groups at up to 3 bits and of 4 groups at up to 2: the whole H_dt = H_LPU (x) H_32 runs on
  // the MFMA.  A lane's B operand takes the LPU groups of its unit in turn (K = 32 LPU), each negated
  // where H_LPU[q][j] = -1, against the same H_32 A operand; D is applied to the inputs as they are
  // staged.  Against the cross-lane stages: 1-2 % faster for 3-bit units of 64 and 1-2 bit units of 128;
  // for the fork's 3-bit records (units of 128) once 14 % faster, now 8 % slower (0.297-0.307 against
  // 0.275-0.280 ms in a captured step) since the code chain lost its wait-state nops; 17 % slower at 4
  // bits.  Units of 8 groups keep the stages too (8 times the B reads and 7 sign flips per read).
  constexpr bool MH = (LPU == 2 && BITS <= 3) || (LPU == 4 && BITS <= 2);
  const int lane = threadIdx.x & 63;
  const int wave = PIPE ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int n32 = lane & 31, h = lane >> 5, q = n32 % LPU;
  uint8_t* tile = stage[wave];
  const uint32_t dword = a.dbits[LPU == 1 ? 0 : q];
  // A operand of K chunk kc: lane holds A[m][k] for row m = n32, k = 16 kc + 8 h + j, with
  // A[m][k] = H[pi(m)][k] (D[k] too when LPU = 1) and pi(m) the coordinate accumulator row m carries
  const int pm = 16 * ((n32 >> 2) & 1) + 4 * (n32 >> 3) + (n32 & 3);
  v8h_t am[2];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 16 * kc + 8 * h + j;
      const uint32_t neg = ((uint32_t)__builtin_popcount(pm & k) ^ (LPU == 1 ? dword >> k : 0u)) & 1u;
      am[kc][j] = neg ? (_Float16)-1.0f : (_Float16)1.0f;
    }
  }
  // MH: sign masks of D for the staged words of this lane's 16-byte input pieces (piece lane % 4 of a
  // group at position (lane / 4) % LPU in its unit), and of H_LPU[q][j] for the B operand read from
  // group j of the unit
  uint32_t smask[MH ? 4 : 1], hmask[MH ? LPU : 1];
  if constexpr (MH) {
    const uint32_t sd = a.dbits[(lane >> 2) % LPU] >> (8 * (lane & 3));
#pragma unroll
    for (int i = 0; i < 4; ++i) smask[i] = pair_sign_mask(sd, i);
#pragma unroll
    for (int j = 0; j < LPU; ++j) hmask[j] = (__builtin_popcount(q & j) & 1) ? 0x80008000u : 0u;
  }
  // LPU > 1 (no MH): sign masks of D for the lane's B-operand words (coordinates 8h + 2i, +1 and
  // 16 + 8h + 2i, +1)
  uint32_t dmask[LPU == 1 || MH ? 1 : 8];
  if constexpr (LPU > 1 && !MH) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dmask[i] = pair_sign_mask(dword >> (8 * h), i);
      dmask[4 + i] = pair_sign_mask(dword >> (16 + 8 * h), i);
    }
  }
  float thr[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) thr[k] = a.thr[k];
  const char* xbase = static_cast<const char*>(a.x);

  const int64_t stride = (int64_t)gridDim.x * kBlock;
  u32x4 pre[PIPE || MH ? CH : 1];
  auto put_tile = [&]() {  // pre -> the wave's tile (MH: with D's sign flips)
    if constexpr (MH) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) pre[c][i] ^= smask[i];
    }
    stage_put<CH, PITCH>(tile, pre, lane);
  };
  if constexpr (PIPE) {
    const int64_t f0 = (int64_t)blockIdx.x * kBlock + wave * 64;
    if (f0 < a.n_groups) stage_load<CH, 2, CONTIG>(pre, xbase, f0, a.n_groups, a.groups_per_row, a.ld_x, lane);
  }
  for (int64_t w0 = (int64_t)blockIdx.x * kBlock + wave * 64; w0 < a.n_groups; w0 += stride) {
    if constexpr (PIPE) {
      put_tile();
      if (w0 + stride < a.n_groups)
        stage_load<CH, 2, CONTIG>(pre, xbase, w0 + stride, a.n_groups, a.groups_per_row, a.ld_x, lane);
    } else if constexpr (MH) {
      stage_load<CH, 2, CONTIG>(pre, xbase, w0, a.n_groups, a.groups_per_row, a.ld_x, lane);
      put_tile();
    } else {
      stage_in<CH, PITCH, 2, CONTIG>(tile, xbase, w0, a.n_groups, a.groups_per_row, a.ld_x, lane);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t seg[2][SEGW];
    float nrm[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // B operand: coordinates 8h .. 8h+7 (chunk 0) and 16+8h .. 16+8h+7 (chunk 1) of group 32s + n32
      const uint8_t* gp = tile + (32 * s + n32) * PITCH + 16 * h;
      v8h_t b0 = *reinterpret_cast<const v8h_t*>(gp);
      v8h_t b1 = *reinterpret_cast<const v8h_t*>(gp + 32);
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2v p0 = {b0[2 * i], b0[2 * i + 1]}, p1 = {b1[2 * i], b1[2 * i + 1]};
        ss = __builtin_amdgcn_fdot2(p0, p0, ss, false);
        ss = __builtin_amdgcn_fdot2(p1, p1, ss, false);
      }
      if constexpr (LPU > 1 && !MH) {
        u32x4 w0v = __builtin_bit_cast(u32x4, b0), w1v = __builtin_bit_cast(u32x4, b1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          w0v[i] ^= dmask[i];
          w1v[i] ^= dmask[4 + i];
        }
        b0 = __builtin_bit_cast(v8h_t, w0v);
        b1 = __builtin_bit_cast(v8h_t, w1v);
      }
      const v16f_t z = {};
      v16f_t y;
      if constexpr (MH) {
        // y = sum_j H_LPU[q][j] H_32 x_j over the unit's groups j (D already in the tile)
        const uint8_t* up = tile + (32 * s + n32 - q) * PITCH + 16 * h;
        y = z;
#pragma unroll
        for (int j = 0; j < LPU; ++j) {
          u32x4 w0v = *reinterpret_cast<const u32x4*>(up + j * PITCH);
          u32x4 w1v = *reinterpret_cast<const u32x4*>(up + j * PITCH + 32);
          if (j > 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              w0v[i] ^= hmask[j];
              w1v[i] ^= hmask[j];
            }
          }
          y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[0], __builtin_bit_cast(v8h_t, w0v), y, 0, 0, 0);
          y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[1], __builtin_bit_cast(v8h_t, w1v), y, 0, 0, 0);
        }
      } else {
        y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[0], b0, z, 0, 0, 0);
        y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[1], b1, y, 0, 0, 0);
      }
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, ss), __builtin_bit_cast(uint32_t, ss),
                                                      false, false);
      float us = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
      float yv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) yv[j] = y[j];
      if constexpr (LPU > 1) {
        us = unit_sum<LPU>(us);
        if constexpr (!MH) unit_butterflies<LPU, 16>(yv, q);
      }
      // v_sqrt_f32 (1 ulp): the stored fp16 norm tolerates it, and the thresholds t n move by
      // ~1e-7 of a cell edge, inside the 1e-6 band the codes are held to
      const float n = __builtin_amdgcn_sqrtf(us);
      nrm[s] = n;
#pragma unroll
      for (int k = 0; k < SEGW; ++k) seg[s][k] = 0u;
      if constexpr (LUT) {
        const float kb = n > 0.0f ? a.bin_scale * __builtin_amdgcn_rcpf(n) : 0.0f;  // 1 ulp: only picks the bin
        const float top = (float)(a.n_bins - 1);
        code_lut<BITS, 16>(seg[s], yv, n, kb, top, lut);
      } else {
        float T[7];
#pragma unroll
        for (int k = 0; k < 7; ++k) T[k] = thr[k] * n;
#pragma unroll
        for (int j = 15; j >= 0; --j) code_chain<BITS>(seg[s], j, yv[j], T);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // lanes < 32 store group n32 (set 0), lanes >= 32 group 32 + n32 (set 1): the swap leaves the
    // half with coordinates 0..15 of the stored group in r[0] and the half with 16..31 in r[1]
    uint32_t lo[SEGW], hi[SEGW];
#pragma unroll
    for (int k = 0; k < SEGW; ++k) {
      const auto r = __builtin_amdgcn_permlane32_swap(seg[0][k], seg[1][k], false, false);
      lo[k] = r[0];
      hi[k] = r[1];
    }
    const float n = h ? nrm[1] : nrm[0];
    uint32_t word[BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) word[k] = n == 0.0f ? zero_unit_word<BITS>(k) : join_halves<BITS>(lo, hi, k);
    const int64_t g = w0 + lane;
    const bool full = w0 + 64 <= a.n_groups;
    if constexpr (AOS) {
      constexpr int R = Record<BITS>::kBytes;
      const uint16_t nb = __half_as_ushort(__float2half_rn(n));
      if (full) {
        put_record<BITS>(reinterpret_cast<uint16_t*>(tile + R * lane), nb, word);
        __builtin_amdgcn_wave_barrier();
        u32x4* out = reinterpret_cast<u32x4*>(a.codes + w0 * R);
#pragma unroll
        for (int c = lane; c < Record<BITS>::kChunks; c += 64)
          store_stream(*reinterpret_cast<const u32x4*>(tile + 16 * c), out + c);
        __builtin_amdgcn_wave_barrier();
      } else if (g < a.n_groups) {
        put_record<BITS>(reinterpret_cast<uint16_t*>(a.codes + g * R), nb, word);
      }
    } else {
      if constexpr (B8) {  // 32 bytes per group, re-dealt through the tile into two 1 KiB spans
        if (full) {
          u32x4* t16 = reinterpret_cast<u32x4*>(tile);
          t16[2 * lane] = u32x4{word[0], word[1], word[2], word[3]};
          t16[2 * lane + 1] = u32x4{word[4], word[5], word[6], word[7]};
          __builtin_amdgcn_wave_barrier();
          u32x4* out = reinterpret_cast<u32x4*>(a.codes + w0 * 32);
          store_stream(t16[lane], out + lane);
          store_stream(t16[64 + lane], out + 64 + lane);
          __builtin_amdgcn_wave_barrier();
        } else if (g < a.n_groups) {
          u32x4* cp = reinterpret_cast<u32x4*>(a.codes + g * 32);
          store_stream(u32x4{word[0], word[1], word[2], word[3]}, cp);
          store_stream(u32x4{word[4], word[5], word[6], word[7]}, cp + 1);
        }
      } else if (PIPE ? (full || g < a.n_groups) : g < a.n_groups) {
        uint32_t* cp = reinterpret_cast<uint32_t*>(a.codes + g * (4 * BITS));
#pragma unroll
        for (int k = 0; k < BITS; ++k) __builtin_nontemporal_store(word[k], cp + k);
      }
      if ((LPU == 1 || q == 0) && g < a.n_groups) {
        const int64_t u = g / LPU;
        if constexpr (NORM_F32)
          static_cast<float*>(a.norms)[u] = n;
        else
          static_cast<__half*>(a.norms)[u] = __float2half_rn(n);
      }
    }
  }
}

// Bytes of one wave's prefetched code records in LDS: 4- or 16-byte slots per lane for the planes
// (BITS = 1, 2: one 256-byte plane per word; 3, 4: 16-byte slots; 8: two 1 KiB halves); for the
// fork's record format the 64 records of a full wave, 4 R 16-byte chunks (copy instruction i puts
// chunk 64 i + l at 16 (64 i + l); lanes past the last chunk copy nothing).
template <int BITS, bool AOS>
constexpr int rec_lds_bytes() {
  return AOS ? 16 * Record<BITS>::kChunks : BITS == 8 ? 2048 : 1024;
}

// Decode with the 32-point inverse transforms on MFMA: for a set of 32 groups,
// Xhat^T = Minv C^T with Minv = H_unnorm (times diag(D) when a unit is one
// group) and C the centroids in the N(0,1) scale, each split into fp16 hi + lo
// parts.  Narrow codes (1..4 bits) use a pair table that yields, per lookup of
// two codes, (hi pair, lo pair); 8-bit codes use a one-code (hi, lo) table
// and byte permutes.  Two pairs form one B operand [hi hi lo lo hi hi lo lo]
// of four coordinates, and the A operand repeats each Minv entry on the hi and
// lo slot, so Minv (c_hi + c_lo) is summed in fp32 by four
// v_mfma_f32_32x32x16_f16 per set.  Output rows are permuted as in
// encode_mfma_kernel (lane half h: coordinates 16h..16h+15).  Units of LPU > 1
// groups take their remaining butterfly stages across lanes l ^ 1, 2, 4 and D
// at the output.  Scaled by n / dt (or n / ||Xhat|| with norm correction,
// ||Xhat||^2 = dt ||c||^2), staged in LDS and stored coalesced.  Codes and
// norms of the next iteration are copied into LDS with global_load_lds one
// iteration ahead (the fork's records: whole 16-byte chunks of a full wave;
// the last, partial wave reads its records directly).
template <int BITS, int LPU, bool OUT_F32, bool NORM_F32, bool NC, bool CONTIG, bool AOS>
__global__ __launch_bounds__(kBlock) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(!(AOS && NORM_F32), "records carry fp16 norms");
  constexpr bool B8 = BITS == 8;
  constexpr int L = 1 << BITS;
  constexpr int CH = OUT_F32 ? 8 : 4, PITCH = 16 * CH + 16, ES = OUT_F32 ? 4 : 2;
  constexpr int LGC = TQ_DEC_LGC, NCOPY = 1 << LGC;  // table copies (lane l reads copy l % NCOPY)
  constexpr int R = Record<BITS>::kBytes, RLDS = rec_lds_bytes<BITS, AOS>();
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][64 * PITCH];
  __shared__ __attribute__((aligned(16))) uint2 ptab[B8 ? 1 : L * L * NCOPY];
  __shared__ __attribute__((aligned(16))) uint32_t tab8[B8 ? 256 * NCOPY : 1];
  __shared__ __attribute__((aligned(16))) uint8_t pre_rec[kWaves][RLDS];
  __shared__ __attribute__((aligned(16))) uint8_t pre_norm[kWaves][AOS ? 16 : 256];
  if constexpr (B8) {
    for (int x = threadIdx.x; x < 256 * NCOPY; x += kBlock) {
      const float c = a.level[x >> LGC];
      const _Float16 hc = (_Float16)c, lc = (_Float16)(c - (float)hc);
      tab8[x] = (uint32_t)__builtin_bit_cast(uint16_t, hc) | ((uint32_t)__builtin_bit_cast(uint16_t, lc) << 16);
    }
  } else {
    for (int x = threadIdx.x; x < L * L * NCOPY; x += kBlock) {
      const int e = x >> LGC;
      const float ca = a.level[e & (L - 1)], cb = a.level[e >> BITS];
      const _Float16 ha = (_Float16)ca, hb = (_Float16)cb;
      const _Float16 la = (_Float16)(ca - (float)ha), lb = (_Float16)(cb - (float)hb);
      ptab[x] = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16),
                           (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16));
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n32 = lane & 31, h = lane >> 5, q = n32 % LPU;
  uint8_t* tile = stage[wave];
  const char* tabp = B8 ? reinterpret_cast<const char*>(tab8) : reinterpret_cast<const char*>(ptab);
  const uint32_t toff = (uint32_t)(lane & (NCOPY - 1)) * (B8 ? 4u : 8u);
  const uint32_t dword = a.dbits[LPU == 1 ? 0 : q];
  // A operand of MFMA f: row m = n32 carries output coordinate pm; slot 8h + j is code
  // coordinate 8f + 4h + {0,1,0,1,2,3,2,3}[j] (hi parts on slots 0,1,4,5, lo parts on 2,3,6,7)
  const int pm = 16 * ((n32 >> 2) & 1) + 4 * (n32 >> 3) + (n32 & 3);
  v8h_t am[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 8 * f + 4 * h + ((j >> 2) << 1) + (j & 1);
      const uint32_t neg = ((uint32_t)__builtin_popcount(pm & c) ^ (LPU == 1 ? dword >> pm : 0u)) & 1u;
      am[f][j] = neg ? (_Float16)-1.0f : (_Float16)1.0f;
    }
  }
  // LPU > 1: D of the lane's 16 output coordinates 16h .. 16h+15, as fp16 pair and fp32 sign masks
  const uint32_t dout = LPU == 1 ? 0u : dword >> (16 * h);
  char* ybase = static_cast<char*>(a.y);
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  uint8_t* rec_lds = pre_rec[wave];
  uint8_t* n_lds = pre_norm[wave];

  // copy the records (and norms) of the wave starting at group w into LDS; a full wave of records
  // moves as whole 16-byte chunks, a partial one is read directly in its iteration
  auto prefetch = [&](int64_t w) {
    if constexpr (AOS) {
      if (w + 64 <= a.n_groups) {
        const uint8_t* src = a.codes + w * R;
#pragma unroll
        for (int i = 0; 64 * i < Record<BITS>::kChunks; ++i) {
          const int c = 64 * i + lane;
          if (c < Record<BITS>::kChunks) lds_copy<16>(src + 16 * c, rec_lds + 1024 * i);
        }
      }
    } else {
      const int64_t g = w + lane < a.n_groups ? w + lane : a.n_groups - 1;
      const uint8_t* cp = a.codes + g * (4 * BITS);
      if constexpr (BITS == 3 || BITS == 4) {
        lds_copy<4 * BITS>(cp, rec_lds);
      } else if constexpr (B8) {
        lds_copy<16>(cp, rec_lds);
        lds_copy<16>(cp + 16, rec_lds + 1024);
      } else {
#pragma unroll
        for (int k = 0; k < BITS; ++k) lds_copy<4>(cp + 4 * k, rec_lds + 256 * k);
      }
      const int64_t u = g / LPU;
      if constexpr (NORM_F32)
        lds_copy<4>(static_cast<const float*>(a.norms) + u, n_lds);
      else
        lds_copy<2>(static_cast<const uint16_t*>(a.norms) + u, n_lds);
    }
  };

  // The records and norms of the next iteration are copied into LDS before this iteration's stores
  // are issued, so the wait for them at the top of an iteration leaves the previous iteration's
  // stores (CH for a full wave) in flight.
  const int64_t first = (int64_t)blockIdx.x * kBlock + wave * 64;
  prefetch(first);
  bool prev_full = false;
  for (int64_t w0 = first; w0 < a.n_groups; w0 += stride) {
    if (prev_full)
      wait_vm<CH>();
    else
      wait_vm<0>();
    const int64_t g = w0 + lane;
    const bool live = g < a.n_groups, full = w0 + 64 <= a.n_groups;
    uint32_t rec[BITS];
    float n = 0.0f;
    if constexpr (AOS) {
      const uint16_t* rp = reinterpret_cast<const uint16_t*>(full ? rec_lds + R * lane : a.codes + (live ? g : 0) * R);
      const float nf = get_record<BITS>(rp, rec);
      n = live ? nf : 0.0f;
#pragma unroll
      for (int k = 0; k < BITS; ++k) rec[k] = live ? rec[k] : 0u;
    } else {
      uint32_t pr[BITS];
      if constexpr (BITS == 3 || BITS == 4) {
#pragma unroll
        for (int k = 0; k < BITS; ++k) pr[k] = reinterpret_cast<const uint32_t*>(rec_lds)[4 * lane + k];
      } else if constexpr (B8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) pr[k] = reinterpret_cast<const uint32_t*>(rec_lds + 1024 * (k >> 2))[4 * lane + (k & 3)];
      } else {
#pragma unroll
        for (int k = 0; k < BITS; ++k) pr[k] = reinterpret_cast<const uint32_t*>(rec_lds + 256 * k)[lane];
      }
      const uint32_t pn = reinterpret_cast<const uint32_t*>(n_lds)[lane];
#pragma unroll
      for (int k = 0; k < BITS; ++k) rec[k] = live ? pr[k] : 0u;
      const float nf = NORM_F32 ? __builtin_bit_cast(float, pn) : __half2float(__ushort_as_half((uint16_t)pn));
      n = live ? nf : 0.0f;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slots read before the next copy lands
    if (w0 + stride < a.n_groups) prefetch(w0 + stride);
    prev_full = full;
    // every lane gets the records and norms of both sets (lanes 0..31: set 0, 32..63: set 1)
    uint32_t rs[2][BITS];
#pragma unroll
    for (int k = 0; k < BITS; ++k) {
      const auto r = __builtin_amdgcn_permlane32_swap(rec[k], rec[k], false, false);
      rs[0][k] = r[0];
      rs[1][k] = r[1];
    }
    const auto rn = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, n), __builtin_bit_cast(uint32_t, n),
                                                     false, false);
    const float ns[2] = {__builtin_bit_cast(float, (uint32_t)rn[0]), __builtin_bit_cast(float, (uint32_t)rn[1])};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v16f_t y = {};
      if constexpr (B8) {
        // this lane's 4 codes of chunk f are bytes 8f + 4h .. 8f + 4h + 3, i.e. record word 2f + h
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const uint32_t w = h ? rs[s][2 * f + 1] : rs[s][2 * f];
          uint32_t e[4];
#pragma unroll
          for (int k = 0; k < 4; ++k)
            e[k] = *reinterpret_cast<const uint32_t*>(tabp + ((__builtin_amdgcn_ubfe(w, 8 * k, 8) << (LGC + 2)) | toff));
          const u32x4 bw = {__builtin_amdgcn_perm(e[1], e[0], 0x05040100u), __builtin_amdgcn_perm(e[1], e[0], 0x07060302u),
                            __builtin_amdgcn_perm(e[3], e[2], 0x05040100u), __builtin_amdgcn_perm(e[3], e[2], 0x07060302u)};
          y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[f], __builtin_bit_cast(v8h_t, bw), y, 0, 0, 0);
        }
      } else {
        // this lane's codes start at coordinate 4h of each 8-coordinate chunk: shift the record by 4h codes
        uint32_t w[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k)
          w[k] = __builtin_amdgcn_alignbit(k + 1 < BITS ? rs[s][k + 1] : 0u, rs[s][k], 4 * BITS * h);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          uint2 e[2];
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const int pos = 8 * BITS * f + 2 * BITS * pp, wi = pos >> 5, sh = pos & 31;
            const uint32_t key = sh + 2 * BITS <= 32
                                     ? __builtin_amdgcn_ubfe(w[wi], sh, 2 * BITS)
                                     : __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh), 0, 2 * BITS);
            e[pp] = *reinterpret_cast<const uint2*>(tabp + ((key << (LGC + 3)) | toff));
          }
          const v8h_t b = __builtin_bit_cast(v8h_t, u32x4{e[0].x, e[0].y, e[1].x, e[1].y});
          y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[f], b, y, 0, 0, 0);
        }
      }
      float yv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) yv[j] = y[j];
      if constexpr (LPU > 1) unit_butterflies<LPU, 16>(yv, q);
      float scale;
      if constexpr (NC) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss = __builtin_fmaf(yv[i], yv[i], ss);
        const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, ss), __builtin_bit_cast(uint32_t, ss),
                                                        false, false);
        float us = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
        if constexpr (LPU > 1) us = unit_sum<LPU>(us);
        scale = ns[s] / __builtin_sqrtf(us);
      } else {
        scale = ns[s] * a.inv_dt;
      }
      uint8_t* dst = tile + (32 * s + n32) * PITCH + ES * 16 * h;
      if constexpr (!OUT_F32) {
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const __half lo = __float2half_rn(yv[2 * i] * scale), hi = __float2half_rn(yv[2 * i + 1] * scale);
          o[i] = ((uint32_t)__half_as_ushort(lo) | ((uint32_t)__half_as_ushort(hi) << 16)) ^ pair_sign_mask(dout, i);
        }
        reinterpret_cast<u32x4*>(dst)[0] = u32x4{o[0], o[1], o[2], o[3]};
        reinterpret_cast<u32x4*>(dst)[1] = u32x4{o[4], o[5], o[6], o[7]};
      } else {
        uint32_t o[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) o[j] = __builtin_bit_cast(uint32_t, yv[j] * scale) ^ (((dout >> j) & 1u) << 31);
#pragma unroll
        for (int c = 0; c < 4; ++c) reinterpret_cast<u32x4*>(dst)[c] = u32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
      }
    }
    __builtin_amdgcn_wave_barrier();
    stage_out<CH, PITCH, ES, CONTIG>(tile, ybase, w0, a.n_groups, a.groups_per_row, a.ld_y, lane);
    __builtin_amdgcn_wave_barrier();
  }
  wait_vm<0>();  // the last (unused) copy must land before the workgroup's LDS is released
}

// Workgroups per launch: enough resident waves to cover HBM latency, with a
// grid-stride loop over the rest (amortises the per-lane set-up).
// Workgroups for n_groups groups of one lane each, at most per_cu per compute unit.  A launch that
// would need more than four workgroups per CU gives each lane at least two groups instead, so that the
// second group's loads overlap the first's compute rather than waiting for a second round of
// workgroups: the Llama-3.2-1B-shaped cache (524288 groups of 32) decodes in 13.4 against 15.9 us
// and encodes in 14.5 against 14.9 us with 1024 workgroups instead of 2048.  Large launches keep
// their capped grids; small ones (one round at most four deep) are unchanged.
int64_t grid_for(int64_t n_groups, int per_cu) {
  const int cus = device_cu_count();
  int64_t need = (n_groups + kBlock - 1) / kBlock;
  const int64_t few = 4 * (int64_t)cus;
  if (need > few) {
    const int64_t two = (n_groups + 2 * kBlock - 1) / (2 * kBlock);
    need = two > few ? two : few;
  }
  const int64_t cap = (int64_t)cus * per_cu;
  return need < cap ? need : cap;
}

// The 3-bit block-32 kernels (fp16 rows, code and norm planes) run fastest with five workgroups per
// compute unit: on a Qwen3-8B-shaped half-cache the encode takes 255 us against 268 us with the
// eight that its 59 VGPRs and 20 KiB of LDS would otherwise allow (264 with six, 258 with four), and
// the decode 248 us against 257 with six; more waves in flight slow their mixed read/write streams.
// Dynamic LDS that the kernel never touches holds it at five.  The 4-bit block-32 encode (bucket
// table) also runs best with five: 270-276 us in a captured step against 288 with the seven its 71
// VGPRs and 22 KiB of LDS allow.  The 8-bit block-32 decode likewise runs best with four (302
// against 312 us with the five its LDS allows).  The 4-bit decode, the 8-bit encode and the fork's
// records run slower or no faster with fewer waves (records by 8-40 %) and get none.
constexpr unsigned kLdsPerCu = 160u * 1024u;
constexpr unsigned kResident3 = 5;
constexpr unsigned kResident4 = 5;
constexpr unsigned kResident8 = 4;

// Dynamic LDS bytes that leave room for `wgs` workgroups of `kernel` per compute unit.  The kernel's
// static LDS is read from its attributes once and cached; while the launch stream is being captured
// into a graph before that, the launch goes without the padding (same results, slower).
template <typename K>
unsigned lds_pad(std::atomic<int>& cache, K kernel, unsigned wgs, hipStream_t s) {
  const int known = cache.load(std::memory_order_relaxed);
  if (known >= 0) return (unsigned)known;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return 0u;
  }
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel)) != hipSuccess) {
    (void)hipGetLastError();
    return 0u;
  }
  const size_t per = kLdsPerCu / wgs - 512u;  // a margin under the per-workgroup share
  const int pad = attr.sharedSizeBytes < per ? (int)(per - attr.sharedSizeBytes) : 0;
  cache.store(pad, std::memory_order_relaxed);
  return (unsigned)pad;
}

// fp16 rows: the MFMA kernel for every unit length and output form; fp32 rows: the one-group-per-lane
// kernel (its transform is exact fp32 arithmetic on the fp32 inputs).
template <int BITS, int LPU, bool CONTIG>
hipError_t encode_dispatch_dtype(const tq_config& cfg, const EncodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)grid_for(a.n_groups, TQ_GRID_PER_CU)), block(kBlock);
  const bool in32 = cfg.x_dtype == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (cfg.flags & TQ_BLOCKS) {  // fp16 norms (checked on the host)
    if (in32)
      hipLaunchKernelGGL((encode_kernel<BITS, LPU, true, false, CONTIG, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((encode_mfma_kernel<BITS, LPU, false, CONTIG, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  constexpr unsigned kRes = BITS == 3 ? kResident3 : BITS == 4 ? kResident4 : 0;
  if (!in32 && !n32) {
    static std::atomic<int> known{-1};
    const unsigned pad =
        kRes && LPU == 1 ? lds_pad(known, encode_mfma_kernel<BITS, LPU, false, CONTIG, false>, kRes, s) : 0u;
    hipLaunchKernelGGL((encode_mfma_kernel<BITS, LPU, false, CONTIG, false>), grid, block, pad, s, a);
  }
  if (!in32 && n32) {
    static std::atomic<int> known{-1};
    const unsigned pad =
        kRes && LPU == 1 ? lds_pad(known, encode_mfma_kernel<BITS, LPU, true, CONTIG, false>, kRes, s) : 0u;
    hipLaunchKernelGGL((encode_mfma_kernel<BITS, LPU, true, CONTIG, false>), grid, block, pad, s, a);
  }
  if (in32 && !n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, true, false, CONTIG, false>), grid, block, 0, s, a);
  if (in32 && n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, true, true, CONTIG, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BITS, int LPU>
hipError_t encode_dispatch_contig(const tq_config& cfg, const EncodeArgs& a, hipStream_t s) {
  return a.contiguous ? encode_dispatch_dtype<BITS, LPU, true>(cfg, a, s) : encode_dispatch_dtype<BITS, LPU, false>(cfg, a, s);
}

template <int BITS>
hipError_t encode_dispatch_lpu(const tq_config& cfg, const EncodeArgs& a, hipStream_t s) {
  switch (cfg.dt) {
    case 32: return encode_dispatch_contig<BITS, 1>(cfg, a, s);
    case 64: return encode_dispatch_contig<BITS, 2>(cfg, a, s);
    case 128: return encode_dispatch_contig<BITS, 4>(cfg, a, s);
    default: return encode_dispatch_contig<BITS, 8>(cfg, a, s);
  }
}

template <int BITS, int LPU, bool NC, bool CONTIG>
hipError_t decode_dispatch_dtype(const tq_config& cfg, const DecodeArgs& a, tq_dtype yt, hipStream_t s) {
  dim3 grid((unsigned)grid_for(a.n_groups, LPU == 1 ? TQ_DEC_GRID_PER_CU : TQ_DEC_GRID_PER_CU_UNITS)), block(kBlock);
  const bool o32 = yt == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (cfg.flags & TQ_BLOCKS) {  // fp16 norms (checked on the host)
    if (o32)
      hipLaunchKernelGGL((decode_mfma_kernel<BITS, LPU, true, false, NC, CONTIG, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<BITS, LPU, false, false, NC, CONTIG, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (!o32 && !n32) {
    static std::atomic<int> known{-1};
    const unsigned pad = LPU == 1 && (BITS == 3 || BITS == 8)
                             ? lds_pad(known, decode_mfma_kernel<BITS, LPU, false, false, NC, CONTIG, false>,
                                       BITS == 3 ? kResident3 : kResident8, s)
                             : 0u;
    hipLaunchKernelGGL((decode_mfma_kernel<BITS, LPU, false, false, NC, CONTIG, false>), grid, block, pad, s, a);
  }
  if (!o32 && n32) hipLaunchKernelGGL((decode_mfma_kernel<BITS, LPU, false, true, NC, CONTIG, false>), grid, block, 0, s, a);
  if (o32 && !n32) hipLaunchKernelGGL((decode_mfma_kernel<BITS, LPU, true, false, NC, CONTIG, false>), grid, block, 0, s, a);
  if (o32 && n32) hipLaunchKernelGGL((decode_mfma_kernel<BITS, LPU, true, true, NC, CONTIG, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BITS, int LPU>
hipError_t decode_dispatch_nc(const tq_config& cfg, const DecodeArgs& a, bool nc, tq_dtype yt, hipStream_t s) {
  if (a.contiguous)
    return nc ? decode_dispatch_dtype<BITS, LPU, true, true>(cfg, a, yt, s)
              : decode_dispatch_dtype<BITS, LPU, false, true>(cfg, a, yt, s);
  return nc ? decode_dispatch_dtype<BITS, LPU, true, false>(cfg, a, yt, s)
            : decode_dispatch_dtype<BITS, LPU, false, false>(cfg, a, yt, s);
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
    case 4: return encode_dispatch_lpu<4>(cfg, a, s);
    default: return encode_dispatch_lpu<8>(cfg, a, s);
  }
}

hipError_t launch_decode(const tq_config& cfg, const DecodeArgs& a, bool nc, tq_dtype y_dtype, hipStream_t s) {
  switch (cfg.bits) {
    case 1: return decode_dispatch_lpu<1>(cfg, a, nc, y_dtype, s);
    case 2: return decode_dispatch_lpu<2>(cfg, a, nc, y_dtype, s);
    case 3: return decode_dispatch_lpu<3>(cfg, a, nc, y_dtype, s);
    case 4: return decode_dispatch_lpu<4>(cfg, a, nc, y_dtype, s);
    default: return decode_dispatch_lpu<8>(cfg, a, nc, y_dtype, s);
  }
}

}  // namespace tq
