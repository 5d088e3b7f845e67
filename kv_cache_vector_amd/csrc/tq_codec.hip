// Encode and decode kernels (no QJL stage) for gfx950.
//
// Work split: one lane owns one 32-coordinate group (64 contiguous bytes of
// fp16, or 128 of fp32).  A unit of dt coordinates spans LPU = dt/32
// consecutive lanes, so coordinate c of a unit lives in lane c/32, register
// c%32.  The Walsh-Hadamard butterflies of coordinate bits 0..4 run inside a
// lane's registers; bits 5.. (dt >= 64) pair lanes of the same quad with DPP
// (or a swizzle for the third lane bit).  Norms are lane reductions.
//
// Memory: each wave moves its 64 groups through a private LDS tile, so every
// global load and store instruction covers one contiguous 1 KiB span across
// the wavefront (lane l <-> bytes [16 l, 16 l + 16)); the tile re-deals the
// 16-byte chunks so that each lane ends up with its own group.  Codes and
// norms are already contiguous per lane and go straight to memory.
//
// Encode ([Scratch] §2 steps 1-3; [Fork] "How it works"):
//   n = ||x||, yhat = H_unnorm (D x); since sqrt(dt) * y = yhat / n the cell
//   of a coordinate is found by comparing |yhat| with t_k * n (t_k the N(0,1)
//   cell edges), with no per-element division.  The code bits are produced
//   most-significant first and shifted straight into the packed word, so
//   bucketize and bit-pack are one chain: per bit one compare and one
//   add-with-carry (w = 2 w + [|yhat| > t]); the sign bit is shifted in from
//   the float's sign.
// Decode: c = level(code) looked up two coordinates at a time in an LDS
//   table that already holds the first butterfly (c_a + c_b, c_a - c_b),
//   optional norm correction, x~ = n * D H_unnorm c / dt (or with norm
//   correction n * D H_unnorm c / (sqrt(dt) ||c||)).
#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

// the LDS copy statements set M0 themselves; nothing else in these kernels uses it
#pragma clang diagnostic ignored "-Winline-asm"

namespace tq {
namespace {

constexpr int kWaves = kBlock / 64;

// Streaming hints and launch widths (nontemporal loads and stores, 32 workgroups per compute unit
// for encode and 96 for the store-heavy decode measured fastest on MI355X).
#ifndef TQ_LOAD_NT
#define TQ_LOAD_NT 1
#endif
#ifndef TQ_STORE_NT
#define TQ_STORE_NT 1
#endif
#ifndef TQ_GRID_PER_CU
#define TQ_GRID_PER_CU 32
#endif
#ifndef TQ_DEC_GRID_PER_CU
#define TQ_DEC_GRID_PER_CU 96
#endif
#ifndef TQ_DEC_LGC
#define TQ_DEC_LGC 1
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

// Copy the wave's 64 groups (CH 16-byte chunks each) from global memory into
// the wave's LDS tile, group grp at tile + grp * PITCH.  Instruction k moves
// chunks 64k .. 64k+63 of the wave's span, so each instruction covers one
// contiguous 1 KiB when rows are contiguous.  Full waves issue every load
// before the first LDS write; the last, partial wave checks each chunk.
template <int CH, int PITCH, int ES, bool CONTIG>
__device__ __forceinline__ void stage_in(uint8_t* tile, const char* base, int64_t w0, int64_t n_groups, int32_t gpr,
                                         int64_t ld, int lane) {
  u32x4 t[CH];
  if (w0 + 64 <= n_groups) {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int ci = 64 * k + lane;
      const int grp = ci / CH, c = ci % CH;
      t[k] = load_stream(reinterpret_cast<const u32x4*>(base + ES * group_offset<CONTIG>(w0 + grp, gpr, ld) + 16 * c));
    }
  } else {
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int ci = 64 * k + lane;
      const int grp = ci / CH, c = ci % CH;
      t[k] = u32x4{0u, 0u, 0u, 0u};
      if (w0 + grp < n_groups)
        t[k] = load_stream(reinterpret_cast<const u32x4*>(base + ES * group_offset<CONTIG>(w0 + grp, gpr, ld) + 16 * c));
    }
  }
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int ci = 64 * k + lane;
    *reinterpret_cast<u32x4*>(tile + (ci / CH) * PITCH + 16 * (ci % CH)) = t[k];
  }
}

// stage_in in two halves, for a loop that loads one tile ahead: the loads into registers ...
template <int CH, int ES, bool CONTIG>
__device__ __forceinline__ void stage_load(u32x4* t, const char* base, int64_t w0, int64_t n_groups, int32_t gpr,
                                           int64_t ld, int lane) {
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int ci = 64 * k + lane;
    const int grp = ci / CH, c = ci % CH;
    if (w0 + 64 <= n_groups) {
      t[k] = load_stream(reinterpret_cast<const u32x4*>(base + ES * group_offset<CONTIG>(w0 + grp, gpr, ld) + 16 * c));
    } else {
      t[k] = u32x4{0u, 0u, 0u, 0u};
      if (w0 + grp < n_groups)
        t[k] = load_stream(reinterpret_cast<const u32x4*>(base + ES * group_offset<CONTIG>(w0 + grp, gpr, ld) + 16 * c));
    }
  }
}

// ... and their copy into the wave's LDS tile
template <int CH, int PITCH>
__device__ __forceinline__ void stage_put(uint8_t* tile, const u32x4* t, int lane) {
#pragma unroll
  for (int k = 0; k < CH; ++k) {
    const int ci = 64 * k + lane;
    *reinterpret_cast<u32x4*>(tile + (ci / CH) * PITCH + 16 * (ci % CH)) = t[k];
  }
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

// w = 2 w + [|y| > t]; returns the lane mask of the comparison.
__device__ __forceinline__ uint64_t shift_in_gt(uint32_t& w, float y, float t) {
  uint64_t m, carry;
  asm("v_cmp_gt_f32_e64 %1, |%3|, %4\n\t"
      "v_addc_co_u32_e64 %0, %2, %0, %0, %1"
      : "+v"(w), "=&s"(m), "=&s"(carry)
      : "v"(y), "v"(t));
  return m;
}

__device__ __forceinline__ float select_mask(uint64_t m, float if_false, float if_true) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_false), "v"(if_true), "s"(m));
  return r;
}

// w = (w << 1) | signbit(y)
__device__ __forceinline__ void shift_in_sign(uint32_t& w, float y) {
  w = __builtin_amdgcn_alignbit(w, __builtin_bit_cast(uint32_t, y), 31);
}

// Shift the code of one coordinate, most significant bit first, into the
// packed words.  Bit p of the 32-coordinate group (p = BITS*j + k) lives in
// word p/32; since the caller walks j downwards and the bits of one code
// from the top, every word receives its bits from bit 31 down to bit 0.
template <int BITS>
__device__ __forceinline__ void code_chain(uint32_t* word, int j, float y, const float* T) {
  const int p_top = BITS * j + BITS - 1;
  shift_in_sign(word[p_top >> 5], y);
  if constexpr (BITS == 2) {
    shift_in_gt(word[(p_top - 1) >> 5], y, T[0]);
  } else if constexpr (BITS == 3) {
    const uint64_t c1 = shift_in_gt(word[(p_top - 1) >> 5], y, T[1]);
    shift_in_gt(word[(p_top - 2) >> 5], y, select_mask(c1, T[0], T[2]));
  } else if constexpr (BITS == 4) {
    const uint64_t c1 = shift_in_gt(word[(p_top - 1) >> 5], y, T[3]);
    const float lo = select_mask(c1, T[0], T[4]);
    const float hi = select_mask(c1, T[2], T[6]);
    const uint64_t c2 = shift_in_gt(word[(p_top - 2) >> 5], y, select_mask(c1, T[1], T[5]));
    shift_in_gt(word[(p_top - 3) >> 5], y, select_mask(c2, lo, hi));
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

// 8-bit bucketize tables in LDS: edges t_0 = -1 (sentinel below |u|), t_1..t_127, t_128 = +inf,
// and for each bin of |u| (bins a third of the narrowest cell, so two neighbouring bins hold at
// most one edge) the number of edges below the bin's lower end, found by binary search.
__device__ __forceinline__ void setup_bins8(const EncodeArgs& a, float* edge8, uint8_t* bin8) {
  for (int i = threadIdx.x; i < 129; i += kBlock) edge8[i] = i == 0 ? -1.0f : a.thr[i - 1];
  __syncthreads();
  for (int b = threadIdx.x; b < a.n_bins; b += kBlock) {
    const float x = (float)b / a.bin_scale;
    int lo = 0, hi = 127;  // count of t_1..t_127 below x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (edge8[mid + 1] < x)
        lo = mid + 1;
      else
        hi = mid;
    }
    bin8[b] = (uint8_t)lo;
  }
  __syncthreads();
}

// 8-bit code of rotated coordinate y of a unit with norm n (kb = bins per unit of |y|):
// the bin of |u| = |y| / n (possibly one off), then the two edges around the bin's count
// give magnitude = #{t_i < |u|} exactly, compared as |y| against t n like the narrow codes.
__device__ __forceinline__ uint32_t code8(float y, float n, float kb, float top, const float* edge8,
                                          const uint8_t* bin8) {
  const float ay = __builtin_fabsf(y);
  const int m0 = bin8[(int)__builtin_fminf(ay * kb, top)];
  const float lo = edge8[m0], hi = edge8[m0 + 1];
  const uint32_t mag = (uint32_t)(m0 + (ay > hi * n ? 1 : 0) - (ay <= lo * n ? 1 : 0));
  return ((__builtin_bit_cast(uint32_t, y) >> 31) << 7) | (mag & 127u);
}

template <int BITS, int LPU, bool IN_F32, bool NORM_F32, bool CONTIG, bool AOS>
__global__ __launch_bounds__(kBlock) void encode_kernel(EncodeArgs a) {
  static_assert(!(AOS && NORM_F32), "records carry fp16 norms");
  static_assert(BITS <= 4 || BITS == 8, "1..4 or 8 bits");
  constexpr bool B8 = BITS == 8;
  __shared__ float edge8[B8 ? 132 : 1];
  __shared__ uint8_t bin8[B8 ? kMaxBins8 : 1];
  if constexpr (B8) setup_bins8(a, edge8, bin8);
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
    if constexpr (B8) {
      const float kb = n > 0.0f ? a.bin_scale / n : 0.0f;
      const float top = (float)(a.n_bins - 1);
#pragma unroll
      for (int j = 0; j < 32; ++j) word[j >> 2] |= code8(v[j], n, kb, top, edge8, bin8) << (8 * (j & 3));
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

// Copy the code record and norm of group g (lane's own) into the wave's LDS slots: records at
// rec_lds + 16 l (BITS = 3, 4) or word planes rec_lds + 256 k + 4 l (BITS = 1, 2), norms at
// n_lds + 4 l.  Returns the number of copy instructions.
template <int BITS, bool NORM_F32>
__device__ __forceinline__ void copy_rec(const uint8_t* codes, const void* norms, int64_t g, uint8_t* rec_lds,
                                         uint8_t* n_lds) {
  const uint8_t* cp = codes + g * (4 * BITS);
  if constexpr (BITS == 3 || BITS == 4) {
    lds_copy<4 * BITS>(cp, rec_lds);
  } else {
#pragma unroll
    for (int k = 0; k < BITS; ++k) lds_copy<4>(cp + 4 * k, rec_lds + 256 * k);
  }
  if constexpr (NORM_F32)
    lds_copy<4>(static_cast<const float*>(norms) + g, n_lds);
  else
    lds_copy<2>(static_cast<const uint16_t*>(norms) + g, n_lds);
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

// Block-32 encode of fp16 rows with the Walsh-Hadamard transform on MFMA.
// For a set of 32 groups, Yhat^T = M X^T with M = H_unnorm diag(D) (entries
// +-1, exact in fp16) and X the fp16 inputs: products are exact and the sums
// are accumulated in fp32, two v_mfma_f32_32x32x16_f16 per set and two sets
// per wave (the wave's 64 groups, staged through LDS as in encode_kernel).
// The rows of M are permuted so that output lane half h holds coordinates
// 16h .. 16h+15 of its group in accumulator registers 0..15; each lane
// bucketizes and packs those 16 with the same most-significant-first chain
// as encode_kernel, and one permlane32 swap per segment word hands every lane
// both halves of the record it stores.  The norm comes from the fp16 inputs
// (dot2 of the lane's 16 values plus the partner lane's).
template <int BITS, bool NORM_F32, bool CONTIG>
__global__ __launch_bounds__(kBlock) void encode32_mfma_kernel(EncodeArgs a) {
  constexpr int CH = 4, PITCH = 16 * CH + 16;
  constexpr int SEGW = (16 * BITS + 31) / 32;  // words of one lane's 16-code segment
  constexpr bool B8 = BITS == 8;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][64 * PITCH];
  __shared__ float edge8[B8 ? 132 : 1];
  __shared__ uint8_t bin8[B8 ? kMaxBins8 : 1];
  if constexpr (B8) setup_bins8(a, edge8, bin8);
  // 4 and 8 bits: the next tile's loads go out before this tile's compute and stores (measured
  // faster at 4 and 8 bits, slower at 3)
  constexpr bool PIPE = BITS == 4 || BITS == 8;
  const int lane = threadIdx.x & 63;
  const int wave = PIPE ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int n32 = lane & 31, h = lane >> 5;
  uint8_t* tile = stage[wave];
  const uint32_t dword = a.dbits[0];
  // A operand of K chunk kc: lane holds A[m][k] for row m = n32, k = 16 kc + 8 h + j, with
  // A[m][k] = H[pi(m)][k] D[k] and pi(m) the coordinate that accumulator row m should carry
  const int pm = 16 * ((n32 >> 2) & 1) + 4 * (n32 >> 3) + (n32 & 3);
  v8h_t am[2];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 16 * kc + 8 * h + j;
      const uint32_t neg = ((uint32_t)__builtin_popcount(pm & k) ^ (dword >> k)) & 1u;
      am[kc][j] = neg ? (_Float16)-1.0f : (_Float16)1.0f;
    }
  }
  float thr[7];
#pragma unroll
  for (int k = 0; k < 7; ++k) thr[k] = a.thr[k];
  const char* xbase = static_cast<const char*>(a.x);

  const int64_t stride = (int64_t)gridDim.x * kBlock;
  u32x4 pre[PIPE ? CH : 1];
  if constexpr (PIPE) {
    const int64_t f0 = (int64_t)blockIdx.x * kBlock + wave * 64;
    if (f0 < a.n_groups) stage_load<CH, 2, CONTIG>(pre, xbase, f0, a.n_groups, a.groups_per_row, a.ld_x, lane);
  }
  for (int64_t w0 = (int64_t)blockIdx.x * kBlock + wave * 64; w0 < a.n_groups; w0 += stride) {
    if constexpr (PIPE) {
      stage_put<CH, PITCH>(tile, pre, lane);
      if (w0 + stride < a.n_groups)
        stage_load<CH, 2, CONTIG>(pre, xbase, w0 + stride, a.n_groups, a.groups_per_row, a.ld_x, lane);
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
      const v8h_t b0 = *reinterpret_cast<const v8h_t*>(gp);
      const v8h_t b1 = *reinterpret_cast<const v8h_t*>(gp + 32);
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2v p0 = {b0[2 * i], b0[2 * i + 1]}, p1 = {b1[2 * i], b1[2 * i + 1]};
        ss = __builtin_amdgcn_fdot2(p0, p0, ss, false);
        ss = __builtin_amdgcn_fdot2(p1, p1, ss, false);
      }
      const v16f_t z = {};
      v16f_t y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[0], b0, z, 0, 0, 0);
      y = __builtin_amdgcn_mfma_f32_32x32x16_f16(am[1], b1, y, 0, 0, 0);
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, ss), __builtin_bit_cast(uint32_t, ss),
                                                      false, false);
      const float n = __builtin_sqrtf(__builtin_bit_cast(float, (uint32_t)r[0]) +
                                      __builtin_bit_cast(float, (uint32_t)r[1]));
      nrm[s] = n;
#pragma unroll
      for (int k = 0; k < SEGW; ++k) seg[s][k] = 0u;
      if constexpr (B8) {
        const float kb = n > 0.0f ? a.bin_scale / n : 0.0f;
        const float top = (float)(a.n_bins - 1);
#pragma unroll
        for (int j = 0; j < 16; ++j) seg[s][j >> 2] |= code8(y[j], n, kb, top, edge8, bin8) << (8 * (j & 3));
      } else {
        float T[7];
#pragma unroll
        for (int k = 0; k < 7; ++k) T[k] = thr[k] * n;
#pragma unroll
        for (int j = 15; j >= 0; --j) code_chain<BITS>(seg[s], j, y[j], T);
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
    const int64_t g = w0 + lane;
    if (PIPE ? (w0 + 64 <= a.n_groups || g < a.n_groups) : g < a.n_groups) {
      uint32_t* cp = reinterpret_cast<uint32_t*>(a.codes + g * (4 * BITS));
      if constexpr (B8) {  // 32 bytes per group: two 16-byte stores
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4 w;
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = n == 0.0f ? zero_unit_word<BITS>(4 * c + k) : join_halves<BITS>(lo, hi, 4 * c + k);
          __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(cp) + c);
        }
      } else {
#pragma unroll
        for (int k = 0; k < BITS; ++k)
          __builtin_nontemporal_store(n == 0.0f ? zero_unit_word<BITS>(k) : join_halves<BITS>(lo, hi, k), cp + k);
      }
      if constexpr (NORM_F32)
        static_cast<float*>(a.norms)[g] = n;
      else
        static_cast<__half*>(a.norms)[g] = __float2half_rn(n);
    }
  }
}

// Pair table: entry (code_a | code_b << BITS) = (c_a + c_b, c_a - c_b), N(0,1) scale.
template <int BITS>
__device__ __forceinline__ void fill_pair_table(float2* tab, const float* level) {
  constexpr int L = 1 << BITS;
  for (int e = threadIdx.x; e < L * L; e += kBlock) {
    const float ca = level[e & (L - 1)], cb = level[e >> BITS];
    tab[e] = make_float2(ca + cb, ca - cb);
  }
}

// Byte offset (8 * key) of the pair (2i, 2i+1) in the pair table.
template <int BITS>
__device__ __forceinline__ uint32_t pair_key8(const uint32_t* word, int i) {
  constexpr int PB = 2 * BITS;
  const int pos = PB * i;
  const int wi = pos >> 5, sh = pos & 31;
  uint32_t key;
  if (sh + PB <= 32)
    key = __builtin_amdgcn_ubfe(word[wi], sh, PB);
  else
    key = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(word[wi + 1], word[wi], sh), 0, PB);
  return key << 3;
}

template <int BITS, int LPU, bool OUT_F32, bool NORM_F32, bool NC, bool CONTIG, bool AOS>
__global__ __launch_bounds__(kBlock) void decode_kernel(DecodeArgs a) {
  static_assert(!(AOS && NORM_F32), "records carry fp16 norms");
  static_assert(BITS <= 4 || BITS == 8, "1..4 or 8 bits");
  constexpr bool B8 = BITS == 8;
  constexpr int L = 1 << BITS;
  constexpr int CH = OUT_F32 ? 8 : 4;
  constexpr int PITCH = 16 * CH + 16;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][64 * PITCH];
  // pair table (two codes -> first butterfly) for narrow codes; 8 bits: one level per code
  __shared__ float2 ptab[B8 ? 1 : L * L];
  __shared__ float lvl8[B8 ? 256 : 1];
  if constexpr (B8) {
    for (int e = threadIdx.x; e < 256; e += kBlock) lvl8[e] = a.level[e];
  } else {
    fill_pair_table<BITS>(ptab, a.level);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint8_t* tile = stage[wave];
  const char* tabp = reinterpret_cast<const char*>(ptab);
  const int q = lane % LPU;
  const uint32_t dword = a.dbits[q];
  char* ybase = static_cast<char*>(a.y);
  constexpr int ES = OUT_F32 ? 4 : 2;

  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t w0 = (int64_t)blockIdx.x * kBlock + wave * 64; w0 < a.n_groups; w0 += stride) {
    const int64_t g = w0 + lane;
    const bool valid = g < a.n_groups;
    uint32_t word[BITS];
    float n = 0.0f;
    if constexpr (AOS) {
      // each group is scaled by the norm its own record carries
      constexpr int R = Record<BITS>::kBytes;
      if (w0 + 64 <= a.n_groups) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.codes + w0 * R);
        u32x4 t[(Record<BITS>::kChunks + 63) / 64];
#pragma unroll
        for (int i = 0; i * 64 < Record<BITS>::kChunks; ++i)
          if (lane + 64 * i < Record<BITS>::kChunks) t[i] = load_stream(src + lane + 64 * i);
#pragma unroll
        for (int i = 0; i * 64 < Record<BITS>::kChunks; ++i)
          if (lane + 64 * i < Record<BITS>::kChunks) *reinterpret_cast<u32x4*>(tile + 16 * (lane + 64 * i)) = t[i];
        __builtin_amdgcn_wave_barrier();
        n = get_record<BITS>(reinterpret_cast<const uint16_t*>(tile + R * lane), word);
        __builtin_amdgcn_wave_barrier();
      } else if (valid) {
        n = get_record<BITS>(reinterpret_cast<const uint16_t*>(a.codes + g * R), word);
      } else {
#pragma unroll
        for (int k = 0; k < BITS; ++k) word[k] = 0u;
      }
    } else if (valid) {
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
    for (int i = 0; i < 16; ++i) {
      if constexpr (B8) {
        const uint32_t w = word[i >> 1] >> (16 * (i & 1));
        const float ca = lvl8[w & 255u], cb = lvl8[(w >> 8) & 255u];
        v[2 * i] = ca + cb;
        v[2 * i + 1] = ca - cb;
      } else {
        const float2 e = *reinterpret_cast<const float2*>(tabp + pair_key8<BITS>(word, i));
        v[2 * i] = e.x;
        v[2 * i + 1] = e.y;
      }
    }
    float scale;
    if constexpr (NC) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) ss = __builtin_fmaf(v[j], v[j], ss);
      ss = unit_sum<LPU>(ss);  // = 2 * ||c||^2: each pair contributes (a+b)^2 + (a-b)^2
      scale = n * a.inv_sqrt_dt * __builtin_sqrtf(2.0f / ss);
    } else {
      scale = n * a.inv_dt;
    }
    fwht32_from<1>(v);
    fwht_crosslane<LPU>(v, q);

    // ---- stage the group's output in LDS, then store it coalesced ----
    uint32_t o[4 * CH];
    if constexpr (!OUT_F32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const __half lo = __float2half_rn(v[2 * i] * scale);
        const __half hi = __float2half_rn(v[2 * i + 1] * scale);
        o[i] = ((uint32_t)__half_as_ushort(lo) | ((uint32_t)__half_as_ushort(hi) << 16)) ^ pair_sign_mask(dword, i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] = __builtin_bit_cast(uint32_t, v[i] * scale) ^ (((dword >> i) & 1u) << 31);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
      *reinterpret_cast<u32x4*>(tile + lane * PITCH + 16 * c) = u32x4{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
    __builtin_amdgcn_wave_barrier();
    stage_out<CH, PITCH, ES, CONTIG>(tile, ybase, w0, a.n_groups, a.groups_per_row, a.ld_y, lane);
    __builtin_amdgcn_wave_barrier();
  }
}

// Block-32 decode with the inverse transform on MFMA: for a set of 32 groups,
// Xhat^T = Minv C^T with Minv = diag(D) H_unnorm (entries +-1) and C the
// centroids in the N(0,1) scale, each split into fp16 hi + lo parts.  The pair
// table yields, per lookup of two codes, (hi pair, lo pair); two lookups form
// one B operand [hi hi lo lo hi hi lo lo] of four coordinates, and the A
// operand repeats each Minv entry on the hi and lo slot, so Minv (c_hi + c_lo)
// is summed in fp32 by four v_mfma_f32_32x32x16_f16 per set.  Output rows are
// permuted as in encode32_mfma_kernel (lane half h: coordinates 16h..16h+15),
// scaled by n / 32 (or n / ||Xhat|| with norm correction, ||Xhat||^2 =
// 32 ||c||^2), staged in LDS and stored coalesced.
template <int BITS, bool OUT_F32, bool NORM_F32, bool NC, bool CONTIG>
__global__ __launch_bounds__(kBlock) void decode32_mfma_kernel(DecodeArgs a) {
  constexpr int L = 1 << BITS;
  constexpr int CH = OUT_F32 ? 8 : 4, PITCH = 16 * CH + 16, ES = OUT_F32 ? 4 : 2;
  constexpr int LGC = TQ_DEC_LGC, NCOPY = 1 << LGC;  // pair-table copies (lane l reads copy l % NCOPY)
  __shared__ __attribute__((aligned(16))) uint8_t stage[kWaves][64 * PITCH];
  __shared__ __attribute__((aligned(16))) uint2 ptab[L * L * NCOPY];
  __shared__ __attribute__((aligned(16))) uint8_t pre_rec[kWaves][1024];
  __shared__ __attribute__((aligned(16))) uint8_t pre_norm[kWaves][256];
  for (int x = threadIdx.x; x < L * L * NCOPY; x += kBlock) {
    const int e = x >> LGC;
    const float ca = a.level[e & (L - 1)], cb = a.level[e >> BITS];
    const _Float16 ha = (_Float16)ca, hb = (_Float16)cb;
    const _Float16 la = (_Float16)(ca - (float)ha), lb = (_Float16)(cb - (float)hb);
    ptab[x] = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16),
                         (uint32_t)__builtin_bit_cast(uint16_t, la) | ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n32 = lane & 31, h = lane >> 5;
  uint8_t* tile = stage[wave];
  const char* tabp = reinterpret_cast<const char*>(ptab);
  const uint32_t toff = (uint32_t)(lane & (NCOPY - 1)) * 8u;
  const uint32_t dword = a.dbits[0];
  // A operand of MFMA f: row m = n32 carries output coordinate pm; slot 8h + j is code
  // coordinate 8f + 4h + {0,1,0,1,2,3,2,3}[j] (hi parts on slots 0,1,4,5, lo parts on 2,3,6,7)
  const int pm = 16 * ((n32 >> 2) & 1) + 4 * (n32 >> 3) + (n32 & 3);
  v8h_t am[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 8 * f + 4 * h + ((j >> 2) << 1) + (j & 1);
      const uint32_t neg = ((uint32_t)__builtin_popcount(pm & c) ^ (dword >> pm)) & 1u;
      am[f][j] = neg ? (_Float16)-1.0f : (_Float16)1.0f;
    }
  }
  char* ybase = static_cast<char*>(a.y);

  // The record and norm of the next iteration are copied into LDS before this iteration's stores
  // are issued, so the wait for them at the top of an iteration leaves the previous iteration's
  // stores (4 for a full wave) in flight.
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  uint8_t* rec_lds = pre_rec[wave];
  uint8_t* n_lds = pre_norm[wave];
  const int64_t first = (int64_t)blockIdx.x * kBlock + wave * 64;
  copy_rec<BITS, NORM_F32>(a.codes, a.norms, first + lane < a.n_groups ? first + lane : a.n_groups - 1, rec_lds, n_lds);
  bool prev_full = false;
  for (int64_t w0 = first; w0 < a.n_groups; w0 += stride) {
    if (prev_full)
      wait_vm<4>();
    else
      wait_vm<0>();
    const int64_t g = w0 + lane;
    uint32_t rec[BITS];
    float n = 0.0f;
    {
      uint32_t pr[BITS], pn;
      if constexpr (BITS == 3 || BITS == 4) {
#pragma unroll
        for (int k = 0; k < BITS; ++k) pr[k] = reinterpret_cast<const uint32_t*>(rec_lds)[4 * lane + k];
      } else {
#pragma unroll
        for (int k = 0; k < BITS; ++k) pr[k] = reinterpret_cast<const uint32_t*>(rec_lds + 256 * k)[lane];
      }
      pn = reinterpret_cast<const uint32_t*>(n_lds)[lane];
      const bool live = g < a.n_groups;
#pragma unroll
      for (int k = 0; k < BITS; ++k) rec[k] = live ? pr[k] : 0u;
      const float nf = NORM_F32 ? __builtin_bit_cast(float, pn) : __half2float(__ushort_as_half((uint16_t)pn));
      n = live ? nf : 0.0f;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slots read before the next copy lands
    {
      const int64_t gn = w0 + stride + lane;
      copy_rec<BITS, NORM_F32>(a.codes, a.norms, gn < a.n_groups ? gn : a.n_groups - 1, rec_lds, n_lds);
    }
    prev_full = w0 + 64 <= a.n_groups;
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
      // this lane's codes start at coordinate 4h of each 8-coordinate chunk: shift the record by 4h codes
      uint32_t w[BITS];
#pragma unroll
      for (int k = 0; k < BITS; ++k)
        w[k] = __builtin_amdgcn_alignbit(k + 1 < BITS ? rs[s][k + 1] : 0u, rs[s][k], 4 * BITS * h);
      v16f_t y = {};
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
      float scale;
      if constexpr (NC) {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss = __builtin_fmaf(y[i], y[i], ss);
        const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, ss), __builtin_bit_cast(uint32_t, ss),
                                                        false, false);
        scale = ns[s] / __builtin_sqrtf(__builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]));
      } else {
        scale = ns[s] * a.inv_dt;
      }
      uint8_t* dst = tile + (32 * s + n32) * PITCH + ES * 16 * h;
      if constexpr (!OUT_F32) {
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const __half lo = __float2half_rn(y[2 * i] * scale), hi = __float2half_rn(y[2 * i + 1] * scale);
          o[i] = (uint32_t)__half_as_ushort(lo) | ((uint32_t)__half_as_ushort(hi) << 16);
        }
        reinterpret_cast<u32x4*>(dst)[0] = u32x4{o[0], o[1], o[2], o[3]};
        reinterpret_cast<u32x4*>(dst)[1] = u32x4{o[4], o[5], o[6], o[7]};
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          reinterpret_cast<u32x4*>(dst)[c] =
              u32x4{__builtin_bit_cast(uint32_t, y[4 * c] * scale), __builtin_bit_cast(uint32_t, y[4 * c + 1] * scale),
                    __builtin_bit_cast(uint32_t, y[4 * c + 2] * scale), __builtin_bit_cast(uint32_t, y[4 * c + 3] * scale)};
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
int64_t grid_for(int64_t n_groups, int per_cu) {
  const int cus = device_cu_count();
  int64_t need = (n_groups + kBlock - 1) / kBlock;
  int64_t cap = (int64_t)cus * per_cu;
  return need < cap ? need : cap;
}

template <int BITS, int LPU, bool CONTIG>
hipError_t encode_dispatch_dtype(const tq_config& cfg, const EncodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)grid_for(a.n_groups, TQ_GRID_PER_CU)), block(kBlock);
  const bool in32 = cfg.x_dtype == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (cfg.flags & TQ_BLOCKS) {  // fp16 norms (checked on the host)
    if (in32)
      hipLaunchKernelGGL((encode_kernel<BITS, LPU, true, false, CONTIG, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((encode_kernel<BITS, LPU, false, false, CONTIG, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if constexpr (LPU == 1) {
    if (!in32) {
      if (n32)
        hipLaunchKernelGGL((encode32_mfma_kernel<BITS, true, CONTIG>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((encode32_mfma_kernel<BITS, false, CONTIG>), grid, block, 0, s, a);
      return hipGetLastError();
    }
  }
  if (!in32 && !n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, false, false, CONTIG, false>), grid, block, 0, s, a);
  if (!in32 && n32) hipLaunchKernelGGL((encode_kernel<BITS, LPU, false, true, CONTIG, false>), grid, block, 0, s, a);
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
  dim3 grid((unsigned)grid_for(a.n_groups, LPU == 1 ? TQ_DEC_GRID_PER_CU : TQ_GRID_PER_CU)), block(kBlock);
  const bool o32 = yt == TQ_F32, n32 = cfg.norm_dtype == TQ_F32;
  if (cfg.flags & TQ_BLOCKS) {  // fp16 norms (checked on the host)
    if (o32)
      hipLaunchKernelGGL((decode_kernel<BITS, LPU, true, false, NC, CONTIG, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<BITS, LPU, false, false, NC, CONTIG, true>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if constexpr (LPU == 1 && BITS <= 4) {
    if (!o32 && !n32) hipLaunchKernelGGL((decode32_mfma_kernel<BITS, false, false, NC, CONTIG>), grid, block, 0, s, a);
    if (!o32 && n32) hipLaunchKernelGGL((decode32_mfma_kernel<BITS, false, true, NC, CONTIG>), grid, block, 0, s, a);
    if (o32 && !n32) hipLaunchKernelGGL((decode32_mfma_kernel<BITS, true, false, NC, CONTIG>), grid, block, 0, s, a);
    if (o32 && n32) hipLaunchKernelGGL((decode32_mfma_kernel<BITS, true, true, NC, CONTIG>), grid, block, 0, s, a);
    return hipGetLastError();
  }
  if (!o32 && !n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, false, false, NC, CONTIG, false>), grid, block, 0, s, a);
  if (!o32 && n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, false, true, NC, CONTIG, false>), grid, block, 0, s, a);
  if (o32 && !n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, true, false, NC, CONTIG, false>), grid, block, 0, s, a);
  if (o32 && n32) hipLaunchKernelGGL((decode_kernel<BITS, LPU, true, true, NC, CONTIG, false>), grid, block, 0, s, a);
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
