// QJL inner-product scores on gfx950 ([README] combined estimator):
//
//   score[i][j] = n_j * ( <q_i, D H c_j> + rho_j * sqrt(pi/2)/m * <S q_i, sign_j> )
//
// Both contractions over all (query, key) pairs run on int8 MFMA
// (v_mfma_i32_32x32x32_i8, the shape that reaches the int8 matrix peak on
// gfx950) with exact integer accumulation:
//   * key side, exact small integers: the reconstruction c_j = sgn * C[mag]
//     is split over the magnitude bits, c = sum_t w_t * T_t with
//     T_t[d] = sgn_d * [mag_d contains the bits of t] in {0, +-1} and weights
//     w_t from the Moebius inversion of the positive centroids; the sign
//     sketch is a +-1 plane.
//   * query side, fixed point: the plane-weighted copies w_t qhat of qhat =
//     H D q, and p = S q = S~ qhat (fp32 MFMA), are scaled per query to
//     16-bit integers and split into two int8 limbs, hi * 256 + lo; since the
//     weights ride on the query, all planes add into one integer accumulator,
//     which is shifted by 8 between the limb passes.
// <q, D H c> = <H D q, c> (H, D symmetric involutions), so keys are never
// rotated back.  The rounding error is that of 16-bit fixed point for qhat
// and p (about 1e-5 of ||q|| per element), far inside the 1e-4 tolerance.
//
// Kernels: prep_queries (one workgroup per 16 queries: rotation in registers,
// S~ projection on fp32 MFMA, fixed-point limbs written as MFMA operand
// fragments), scores (each wave builds the operand planes of 32*CB keys in
// registers from their codes and sign bits, keeps them, and streams 32-query
// blocks through an LDS ring shared by the workgroup's waves).
#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kQB = 32;         // queries per block (the MFMA's M)
#ifndef TQ_SCORES_WG_PER_CU
#define TQ_SCORES_WG_PER_CU 2
#endif
// the queries are cut into as few chunks (one workgroup row each) as give this many workgroups per compute unit
constexpr int kScoresWgPerCu = TQ_SCORES_WG_PER_CU;
#ifndef TQ_SCORES_WAVES
#define TQ_SCORES_WAVES 8
#endif
#ifndef TQ_SCORES_CB2
#define TQ_SCORES_CB2 1
#endif
constexpr int kSW = TQ_SCORES_WAVES;  // waves per scores workgroup, each with its own keys
// 32-key tiles held by one scores wave: TQ_SCORES_CB2 for 1- and 2-plane keys, one for 4 planes
constexpr int scores_cb(int np) { return np <= 2 ? TQ_SCORES_CB2 : 1; }
constexpr float kFixed = 32000.0f;
constexpr int kStoreNT = 2;  // cache-policy operand of the buffer stores: nontemporal (streaming)

// Byte offset of element idx (of a Kd- or Km-long int8 vector) of query r inside its block's
// fragment f0 + idx / 32: fragment = 1 KiB, lane 32 h + r holds bytes 16 h .. 16 h + 15 of the
// 32-byte chunk, which is the operand layout of v_mfma_i32_32x32x32_i8.
__device__ __forceinline__ int frag_offset(int f0, int r, int idx) {
  return (f0 + (idx >> 5)) * 1024 + ((((idx >> 4) & 1) * 32 + r) * 16) + (idx & 15);
}

// ---------------------------------------------------------------------------
// query preparation: one workgroup per 16 queries (half of a 32-query block).
// Thread t owns 8 consecutive coordinates (and 8 projections) of query t / 16:
// the rotation runs 3 butterfly stages in registers and 4 across the 16 lanes
// of the query, the maxima are 16-lane reductions, and each thread writes its
// 8 limbs as 8-byte pieces of the block's operand fragments.  dt, m <= 128.
// ---------------------------------------------------------------------------
template <bool Q_F32, int NP>
__global__ __launch_bounds__(256) void prep_queries(ScoreArgs a) {
  __shared__ float qhat[16][128 + 4];
  __shared__ float pbuf[16][128 + 4];
  const int dt = a.dt, m = a.m, Kd = a.kd, Km = a.km, RQ = 2 * (NP * Kd + Km);
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = tid >> 4, c8 = (tid & 15) * 8;  // query r of the 16, coordinates c8 .. c8 + 7
  const int64_t row = row0 + r;

  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = c8 + i;
    float x = 0.0f;
    if (row < a.n_q && d < dt) {
      if constexpr (Q_F32)
        x = static_cast<const float*>(a.q)[row * a.ld_q + d];
      else
        x = __half2float(static_cast<const __half*>(a.q)[row * a.ld_q + d]);
    }
    v[i] = ((a.dbits[(d >> 5) & 7] >> (d & 31)) & 1u) ? -x : x;
  }
  // unnormalised FWHT over dt coordinates: bits 0..2 in registers, bits 3..6 across lanes 1, 2, 4, 8 apart
#pragma unroll
  for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & bit)) {
        const float x = v[i], y = v[i | bit];
        v[i] = x + y;
        v[i | bit] = x - y;
      }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((8 << k) >= dt) break;
    const bool upper = (tid >> k) & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float o = __shfl_xor(v[i], 1 << k);
      v[i] = upper ? o - v[i] : v[i] + o;
    }
  }
  const float inv_sqrt_dt = a.inv_sqrt_dt;
  float ma = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = c8 + i < dt ? v[i] * inv_sqrt_dt : 0.0f;
    ma = fmaxf(ma, fabsf(v[i]));
    qhat[r][c8 + i] = v[i];
  }
  __syncthreads();

  // p = S~ qhat on fp32 MFMA: the 16 queries x 16 projections of tile ct.  K step s of lane group
  // q = lane / 16 takes coordinate q dt/4 + s, so each lane's S~ operands are dt/4 contiguous floats
  // (loaded up front as 16-byte pieces) and its qhat operands a contiguous LDS run.
  const int q4 = lane >> 4, kq = dt / 4;
  for (int ct = wave; ct < m / 16; ct += 4) {
    const float4* srow = reinterpret_cast<const float4*>(a.s_rot32 + (int64_t)(16 * ct + (lane & 15)) * dt + kq * q4);
    float4 sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (4 * i < kq) sv[i] = srow[i];
    const float* qrow = &qhat[lane & 15][kq * q4];
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (4 * i < kq) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qrow[4 * i], sv[i].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qrow[4 * i + 1], sv[i].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qrow[4 * i + 2], sv[i].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qrow[4 * i + 3], sv[i].w, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pbuf[4 * q4 + i][16 * ct + (lane & 15)] = acc[i];
  }
  __syncthreads();
  float pv[8], mp = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pv[i] = c8 + i < m ? pbuf[r][c8 + i] : 0.0f;
    mp = fmaxf(mp, fabsf(pv[i]));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ma = fmaxf(ma, __shfl_xor(ma, 1 << k));
    mp = fmaxf(mp, __shfl_xor(mp, 1 << k));
  }

  // fixed-point limbs: Q = rint(x * kFixed / max), hi = floor((Q + 128) / 256), lo = Q - 256 hi
  int8_t* blk = a.qrec + (row0 & ~(int64_t)(kQB - 1)) * RQ;
  const int rb = (int)(row0 & (kQB - 1)) + r;  // row within the 32-query block
  auto put = [&](const float* x, float mx, int idx, int f0, int nks) {
    uint32_t hw[2] = {0u, 0u}, lw[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int Q = mx > 0.0f ? (int)rintf(x[i] * (kFixed / mx)) : 0;
      Q = Q > 32000 ? 32000 : (Q < -32000 ? -32000 : Q);
      const int hi = (Q + 128) >> 8, lo = Q - 256 * hi;
      hw[i >> 2] |= (uint32_t)(hi & 0xFF) << (8 * (i & 3));
      lw[i >> 2] |= (uint32_t)(lo & 0xFF) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(blk + frag_offset(f0, rb, idx)) = make_uint2(hw[0], hw[1]);
    *reinterpret_cast<uint2*>(blk + frag_offset(f0 + nks, rb, idx)) = make_uint2(lw[0], lw[1]);
  };
  // plane t carries w_t qhat; one fixed-point scale over all planes lets them share an accumulator
  float wmax = 0.0f;
#pragma unroll
  for (int t = 0; t < NP; ++t) wmax = fmaxf(wmax, fabsf(a.plane_w[t]));
  const float mq = ma * wmax;
  if (c8 < Kd) {
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = v[i] * a.plane_w[t];
      put(x, mq, c8, 2 * t * (Kd / 32), Kd / 32);
    }
  }
  if (c8 < Km) put(pv, mp, c8, 2 * NP * (Kd / 32), Km / 32);
  if ((tid & 15) == 0) {
    a.qscale[row * 2] = (mq > 0.0f ? mq / kFixed : 0.0f) * inv_sqrt_dt;
    a.qscale[row * 2 + 1] = (mp > 0.0f ? mp / kFixed : 0.0f) * a.qjl_const;
  }
}

// Ternary plane t of 16 consecutive codes (the low 16 * BITS bits of `bits`): byte i is +1 or -1 (the
// code's sign) where the code's magnitude contains the bits of t, else 0.
template <int BITS>
__device__ __forceinline__ v4i ternary_piece(uint64_t bits, int t) {
  uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t code = (uint32_t)(bits >> (BITS * i)) & ((1u << BITS) - 1);
    const uint32_t mag = code & ((1u << (BITS - 1)) - 1);
    const uint32_t v = ((mag & (uint32_t)t) == (uint32_t)t) ? ((code >> (BITS - 1)) ? 0xFFu : 0x01u) : 0u;
    b[i >> 2] |= v << (8 * (i & 3));
  }
  return v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// The +-1 sign plane of 16 projections (bit set: +1).
__device__ __forceinline__ v4i sign_piece(uint32_t sb) {
  uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) b[i >> 2] |= (((sb >> i) & 1u) ? 0x01u : 0xFFu) << (8 * (i & 3));
  return v4i{(int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

// ---------------------------------------------------------------------------
// scores: workgroup = kSW waves x (32*CB keys each), loops over 32-query blocks
//
// Queries are the MFMA's A operand (rows) and keys its B operand (columns):
// lane l's accumulator holds, for key l % 32 of each tile, the queries
// 8 g + 4 (l / 32) + i (i = 0..3) of each group g.  So the key scales are two
// registers per tile, and one 4-byte store per accumulator writes a whole
// 128-byte row piece per 32 lanes: each store instruction fills two cache
// lines, where the transposed layout would touch 32 lines with 32 bytes each.
// Query records are copied straight into a ring of three LDS buffers
// (global_load_lds) two blocks ahead.  vmcnt counts stores and copies
// together, in issue order, so the wait that makes block b + 1 resident
// skips the two youngest blocks of stores: a wave never waits for stores
// younger than two blocks, and the write stream stays deep enough to keep
// HBM busy.
// ---------------------------------------------------------------------------
// Dynamic LDS of one scores workgroup: a ring of three query blocks and their scales.
template <int NP, int KD, int KM, int CB>
struct ScoresLds {
  static constexpr int RQ = 2 * (NP * 32 * KD + 32 * KM);  // bytes per query record
  static constexpr int KIB = kQB * RQ / 1024;               // 1 KiB copies per block
  static constexpr int KPW = (KIB + kSW - 1) / kSW;         // 1 KiB copies per wave and block
  static constexpr int KEYS = 32 * CB * kSW;                // keys per workgroup
  static constexpr int QS = 3 * kQB * RQ;
  static constexpr int TOTAL = QS + 3 * kQB * 2 * 4;
  static_assert(TOTAL <= 160 * 1024, "fits the LDS of one compute unit");
  // vmcnt (6 bits) must hold two blocks of stores plus one block of copies
  static_assert(2 * 16 * CB + KPW + 1 <= 63, "outstanding memory operations fit vmcnt");
};

template <int NP, int KD, int KM, int CB, bool NORM_F32>
__global__ __launch_bounds__(64 * kSW, kSW == 8 ? 2 : 1) void scores_kernel(ScoreArgs a) {
  using LY = ScoresLds<NP, KD, KM, CB>;
  constexpr int RQ = LY::RQ;
  constexpr int KIB = LY::KIB;
  constexpr int KEYS = LY::KEYS;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int8_t (*qblk)[kQB * RQ] = reinterpret_cast<int8_t (*)[kQB * RQ]>(smem);
  float (*qs)[kQB * 2] = reinterpret_cast<float (*)[kQB * 2]>(smem + LY::QS);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int64_t wg_key0 = (int64_t)blockIdx.x * KEYS;
  const int64_t key0 = wg_key0 + wave * (32 * CB);

  // this wave's key-side operands (column col of each 32-key tile), built in registers from the codes and
  // sign bits and kept for the whole query loop: lane (col, half) holds coordinates (projections)
  // 32 ks + 16 half .. + 15 of its key, as NP ternary planes and the sign plane
  constexpr int BITS = NP == 1 ? 1 : NP == 2 ? 2 : 3;
  const int dt = a.dt, m = a.m;
  v4i bT[CB][NP][KD], bS[CB][KM];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t j = key0 + 32 * cb + col;
    const bool live = j < a.n_k;
#pragma unroll
    for (int ks = 0; ks < KD; ++ks) {
      const int d0 = 32 * ks + 16 * half;
      uint64_t bits = 0;
      const bool on = live && d0 < dt;
      if (on) {  // the key's codes are one little-endian bitstream of dt * BITS bits
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(a.codes + j * (dt * BITS / 8));
        const int pos = BITS * d0, w0 = pos >> 5;
        bits = wp[w0];
        if (((pos + 16 * BITS - 1) >> 5) > w0) bits |= (uint64_t)wp[w0 + 1] << 32;
        bits >>= (pos & 31);
      }
#pragma unroll
      for (int t = 0; t < NP; ++t) bT[cb][t][ks] = on ? ternary_piece<BITS>(bits, t) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int ks = 0; ks < KM; ++ks) {
      const int p0 = 32 * ks + 16 * half;
      const bool on = live && p0 < m;
      const uint32_t sb = on ? reinterpret_cast<const uint16_t*>(a.qjl_bits + j * (m / 8))[p0 >> 4] : 0u;
      bS[cb][ks] = on ? sign_piece(sb) : v4i{0, 0, 0, 0};
    }
  }
  // key scales n_j and n_j rho_j of this lane's key in each tile (0 past the last key)
  float kn[CB], knr[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t j = key0 + 32 * cb + col;
    float n = 0.0f, rho = 0.0f;
    if (j < a.n_k) {
      if constexpr (NORM_F32)
        n = static_cast<const float*>(a.norms)[j];
      else
        n = __half2float(static_cast<const __half*>(a.norms)[j]);
      rho = __half2float(__ushort_as_half(a.rnorm[j]));
    }
    kn[cb] = n;
    knr[cb] = n * rho;
  }

  // byte offsets from a 32-query block's first score: this lane's (4 rows further for half 1) and one row's;
  // 32 bits hold every offset within a block when rows are shorter than 2^24 floats
  const bool narrow = a.ld_s < (int64_t(1) << 24);
  const int lane_boff = (int)(4 * half * a.ld_s + col) * 4;
  const int row_bytes = (int)a.ld_s * 4;

  const int64_t q_begin = (int64_t)blockIdx.y * a.q_chunk;
  const int64_t q_end = q_begin + a.q_chunk < a.n_q_pad ? q_begin + a.q_chunk : a.n_q_pad;
  // copy the records (KIB pieces of 1 KiB) and scales (wave 0) of block r0 into buffer buf; every wave
  // issues KPW copies (past the last piece a wave copies the last one again: the same bytes to the same
  // place), so the vmcnt bookkeeping below is the same for all waves
  auto fetch = [&](int64_t r0, int buf) {
    const char* src = reinterpret_cast<const char*>(a.qrec) + r0 * RQ;
#pragma unroll
    for (int i = 0; i < LY::KPW; ++i) {
      const int k = wave + kSW * i < KIB ? wave + kSW * i : KIB - 1;
      lds_copy<16>(src + 1024 * k + 16 * lane, qblk[buf] + 1024 * k);
    }
    if (wave == 0) lds_copy<4>(a.qscale + r0 * 2 + lane, qs[buf]);
  };
  // blocks b and b + 1 are resident when block b starts; block b + 2 is copied during it
  fetch(q_begin, 0);
  if (q_begin + kQB < q_end) fetch(q_begin + kQB, 1);
  wait_vm<0>();
  __syncthreads();

  int cur = 0;
  for (int64_t r0 = q_begin; r0 < q_end; r0 += kQB, cur = cur == 2 ? 0 : cur + 1) {
    const bool ahead = r0 + 2 * kQB < q_end;
    if (ahead) fetch(r0 + 2 * kQB, cur == 0 ? 2 : cur - 1);

    v16i accT[CB], accS[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) accT[cb] = accS[cb] = v16i{};
    const int8_t* qfrag = qblk[cur] + 16 * lane;
#pragma unroll
    for (int limb = 0; limb < 2; ++limb) {
      if (limb == 1) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          accT[cb] <<= 8;
          accS[cb] <<= 8;
        }
      }
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
#pragma unroll
        for (int t = 0; t < NP; ++t) {
          const v4i bq = *reinterpret_cast<const v4i*>(qfrag + 1024 * ((2 * t + limb) * KD + ks));
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            accT[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bq, bT[cb][t][ks], accT[cb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int ks = 0; ks < KM; ++ks) {
        const v4i bp = *reinterpret_cast<const v4i*>(qfrag + 1024 * (2 * NP * KD + limb * KM + ks));
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) accS[cb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bp, bS[cb][ks], accS[cb], 0, 0, 0);
      }
    }

    // epilogue: key key0 + 32 cb + col, queries r0 + 8 g + 4 half + i
    float val[CB][16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int q0 = 8 * g + 4 * half;
      const v4f ab01 = *reinterpret_cast<const v4f*>(&qs[cur][2 * q0]);  // alpha, beta of queries q0, q0 + 1
      const v4f ab23 = *reinterpret_cast<const v4f*>(&qs[cur][2 * q0 + 4]);
      const float alpha[4] = {ab01[0], ab01[2], ab23[0], ab23[2]};
      const float beta[4] = {ab01[1], ab01[3], ab23[1], ab23[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          val[cb][4 * g + i] = (kn[cb] * alpha[i]) * (float)accT[cb][4 * g + i] +
                               (knr[cb] * beta[i]) * (float)accS[cb][4 * g + i];
    }
    const bool fast = narrow && key0 + 32 * CB <= a.n_k && r0 + kQB <= a.n_q;  // wave-uniform
    if (fast) {
      // buffer stores: the block's base and each row's offset in scalar registers, the lane's offset in
      // one vector register, so a store is a single instruction; nontemporal, since no kernel of this
      // call reads the scores back
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(a.scores + r0 * a.ld_s + key0, (short)0, -1, 0x00020000);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(val[cb][4 * g + i]), rs, lane_boff + 128 * cb,
                                                  (8 * g + i) * row_bytes, kStoreNT);
    } else {
      int64_t ld = a.ld_s;
      asm volatile("" : "+s"(ld));  // keeps the addresses of this rare path out of the loop's registers
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = r0 + 8 * g + 4 * half + i;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            if (row < a.n_q && key0 + 32 * cb + col < a.n_k) a.scores[row * ld + key0 + 32 * cb + col] = val[cb][4 * g + i];
        }
    }
    if (fast) {
      // the copy of block b + 1 (issued one block ago) must land; younger than it are the previous block's
      // 16 CB stores, this block's copies and this block's 16 CB stores, none of which are waited for
      if (!ahead)
        wait_vm<32 * CB>();
      else if (wave == 0)
        wait_vm<32 * CB + LY::KPW + 1>();
      else
        wait_vm<32 * CB + LY::KPW>();
    } else {
      wait_vm<0>();  // also completes the copy of block b + 1, whatever follows
    }
    lds_barrier();
  }
  wait_vm<0>();
}

template <int NP, int KD, int KM, bool NORM_F32>
hipError_t launch_scores_t(const ScoreArgs& a, hipStream_t s) {
  constexpr int CB = scores_cb(NP);
  constexpr int lds = ScoresLds<NP, KD, KM, CB>::TOTAL;
  // more than the default 64 KiB of dynamic LDS for the larger records; setting it twice from
  // racing first calls is harmless
  static std::atomic<bool> ready{false};
  if (!ready.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scores_kernel<NP, KD, KM, CB, NORM_F32>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    ready.store(true, std::memory_order_release);
  }
  // query chunks: enough workgroups for kScoresWgPerCu per compute unit, each chunk as long as possible (every
  // workgroup rebuilds its key operands once)
  const int64_t key_wgs = a.n_k_pad / (32 * CB * kSW), blocks = a.n_q_pad / kQB;
  int64_t chunks = ((int64_t)kScoresWgPerCu * device_cu_count() + key_wgs - 1) / key_wgs;
  chunks = chunks < 1 ? 1 : (chunks > blocks ? blocks : chunks);
  const int64_t chunk_blocks = (blocks + chunks - 1) / chunks;
  ScoreArgs b = a;
  b.q_chunk = chunk_blocks * kQB;
  dim3 grid((unsigned)key_wgs, (unsigned)((blocks + chunk_blocks - 1) / chunk_blocks));
  hipLaunchKernelGGL((scores_kernel<NP, KD, KM, CB, NORM_F32>), grid, dim3(64 * kSW), lds, s, b);
  return hipGetLastError();
}

template <int NP, bool NORM_F32>
hipError_t launch_scores_np(const ScoreArgs& a, hipStream_t s) {
  const int kd = a.kd / 64, km = a.km / 64;
  if (kd == 1 && km == 1) return launch_scores_t<NP, 2, 2, NORM_F32>(a, s);
  if (kd == 1 && km == 2) return launch_scores_t<NP, 2, 4, NORM_F32>(a, s);
  if (kd == 2 && km == 1) return launch_scores_t<NP, 4, 2, NORM_F32>(a, s);
  return launch_scores_t<NP, 4, 4, NORM_F32>(a, s);
}

template <bool NORM_F32>
hipError_t launch_scores_norm(const tq_config& cfg, const ScoreArgs& a, hipStream_t s) {
  switch (cfg.bits) {
    case 1: return launch_scores_np<1, NORM_F32>(a, s);
    case 2: return launch_scores_np<2, NORM_F32>(a, s);
    default: return launch_scores_np<4, NORM_F32>(a, s);
  }
}

}  // namespace

int64_t scores_key_tile(int bits) { return 32 * scores_cb(1 << (bits - 1)) * kSW; }
int64_t scores_query_block() { return kQB; }

hipError_t launch_qjl_scores(const tq_config& cfg, const ScoreArgs& a, hipStream_t s) {
  dim3 gq((unsigned)(a.n_q_pad / 16));
  const int np = 1 << (cfg.bits - 1);
  if (a.q_f32) {
    if (np == 1) hipLaunchKernelGGL((prep_queries<true, 1>), gq, dim3(256), 0, s, a);
    if (np == 2) hipLaunchKernelGGL((prep_queries<true, 2>), gq, dim3(256), 0, s, a);
    if (np == 4) hipLaunchKernelGGL((prep_queries<true, 4>), gq, dim3(256), 0, s, a);
  } else {
    if (np == 1) hipLaunchKernelGGL((prep_queries<false, 1>), gq, dim3(256), 0, s, a);
    if (np == 2) hipLaunchKernelGGL((prep_queries<false, 2>), gq, dim3(256), 0, s, a);
    if (np == 4) hipLaunchKernelGGL((prep_queries<false, 4>), gq, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return cfg.norm_dtype == TQ_F32 ? launch_scores_norm<true>(cfg, a, s) : launch_scores_norm<false>(cfg, a, s);
}

}  // namespace tq
