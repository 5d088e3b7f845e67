// QJL inner-product scores on gfx950 ([README] combined estimator):
//
//   score[i][j] = n_j * ( <q_i, D H c_j> + rho_j * sqrt(pi/2)/m * <S q_i, sign_j> )
//
// Both contractions over all (query, key) pairs run on int8 MFMA
// (v_mfma_i32_16x16x64_i8) with exact integer accumulation:
//   * key side, exact small integers: the reconstruction c_j = sgn * C[mag]
//     is split over the magnitude bits, c = sum_t w_t * T_t with
//     T_t[d] = sgn_d * [mag_d contains the bits of t] in {0, +-1} and weights
//     w_t from the Moebius inversion of the positive centroids; the sign
//     sketch is a +-1 plane.
//   * query side, fixed point: qhat = H D q and p = S q = S~ qhat (fp32 MFMA)
//     are scaled per query to 16-bit integers and split into two int8 limbs,
//     hi * 256 + lo; the accumulator is shifted by 8 between the limb passes.
// <q, D H c> = <H D q, c> (H, D symmetric involutions), so keys are never
// rotated back.  The rounding error is that of 16-bit fixed point for qhat
// and p (about 1e-5 of ||q|| per element), far inside the 1e-4 tolerance.
//
// Kernels: prep_queries (one workgroup per 16 queries: rotation in LDS, S~
// projection on fp32 MFMA, fixed-point limbs), prep_keys (one lane per key:
// ternary planes and per-key scalars), scores (each wave keeps the operand
// planes of 64 keys in registers and streams 16-query blocks through LDS).
#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kQB = 16;         // queries per row block
constexpr int kQChunk = 512;    // queries per scores workgroup
constexpr float kFixed = 32000.0f;

// ---------------------------------------------------------------------------
// query preparation
// ---------------------------------------------------------------------------
template <bool Q_F32>
__global__ __launch_bounds__(256) void prep_queries(ScoreArgs a) {
  extern __shared__ float smem[];
  const int dt = a.dt, m = a.m;
  float* qhat = smem;                // [kQB][dt]
  float* pbuf = smem + kQB * dt;     // [kQB][m]
  __shared__ float red[kQB][2];
  const int row0 = blockIdx.x * kQB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int e = tid; e < kQB * dt; e += 256) {
    const int r = e / dt, d = e % dt;
    float v = 0.0f;
    if (row0 + r < a.n_q) {
      if constexpr (Q_F32)
        v = static_cast<const float*>(a.q)[(int64_t)(row0 + r) * a.ld_q + d];
      else
        v = __half2float(static_cast<const __half*>(a.q)[(int64_t)(row0 + r) * a.ld_q + d]);
    }
    qhat[e] = ((a.dbits[d >> 5] >> (d & 31)) & 1u) ? -v : v;
  }
  __syncthreads();
  for (int h = 1; h < dt; h <<= 1) {  // unnormalised butterflies, one index bit per pass
    for (int e = tid; e < kQB * dt / 2; e += 256) {
      const int r = e / (dt / 2), pidx = e % (dt / 2);
      const int i = (pidx / h) * 2 * h + (pidx % h);
      float* row = qhat + r * dt;
      const float x = row[i], y = row[i + h];
      row[i] = x + y;
      row[i + h] = x - y;
    }
    __syncthreads();
  }
  const float inv_sqrt_dt = a.inv_sqrt_dt;
  for (int e = tid; e < kQB * dt; e += 256) qhat[e] *= inv_sqrt_dt;
  __syncthreads();

  // p = S~ qhat on fp32 MFMA: 16 queries x 16 projections per tile, K = 4 per step
  for (int t = wave; t < m / 16; t += 4) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* srow = a.s_rot32 + (int64_t)(16 * t + (lane & 15)) * dt;
    for (int k0 = 0; k0 < dt; k0 += 4) {
      const float av = qhat[(lane & 15) * dt + k0 + (lane >> 4)];
      const float bv = srow[k0 + (lane >> 4)];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) pbuf[(4 * (lane >> 4) + i) * m + 16 * t + (lane & 15)] = acc[i];
  }
  __syncthreads();

  // per-query maxima (wave w handles queries 4w .. 4w+3)
  for (int r = 4 * wave; r < 4 * wave + 4; ++r) {
    float ma = 0.0f, mp = 0.0f;
    for (int d = lane; d < dt; d += 64) ma = fmaxf(ma, fabsf(qhat[r * dt + d]));
    for (int j = lane; j < m; j += 64) mp = fmaxf(mp, fabsf(pbuf[r * m + j]));
    for (int off = 32; off >= 1; off >>= 1) {
      ma = fmaxf(ma, __shfl_xor(ma, off));
      mp = fmaxf(mp, __shfl_xor(mp, off));
    }
    if (lane == 0) {
      red[r][0] = ma;
      red[r][1] = mp;
    }
  }
  __syncthreads();

  // fixed-point limbs: Q = rint(x * kFixed / max), hi = floor((Q + 128) / 256), lo = Q - 256 hi
  const int Kd = a.kd, Km = a.km, RQ = 2 * (Kd + Km);
  for (int e = tid; e < kQB * (Kd + Km); e += 256) {
    const int r = e / (Kd + Km), c = e % (Kd + Km);
    const bool is_p = c >= Kd;
    const int idx = is_p ? c - Kd : c;
    const int lim = is_p ? m : dt;
    const float mx = red[r][is_p ? 1 : 0];
    float x = 0.0f;
    if (idx < lim) x = is_p ? pbuf[r * m + idx] : qhat[r * dt + idx];
    int Q = mx > 0.0f ? (int)rintf(x * (kFixed / mx)) : 0;
    Q = Q > 32000 ? 32000 : (Q < -32000 ? -32000 : Q);
    const int hi = (Q + 128) >> 8, lo = Q - 256 * hi;
    int8_t* rec = a.qrec + (int64_t)(row0 + r) * RQ;
    const int base = is_p ? 2 * Kd : 0, width = is_p ? Km : Kd;
    rec[base + idx] = (int8_t)hi;
    rec[base + width + idx] = (int8_t)lo;
  }
  if (tid < kQB) {
    const float sa = red[tid][0] > 0.0f ? red[tid][0] / kFixed : 0.0f;
    const float sp = red[tid][1] > 0.0f ? red[tid][1] / kFixed : 0.0f;
    a.qscale[(row0 + tid) * 2] = sa * inv_sqrt_dt;
    a.qscale[(row0 + tid) * 2 + 1] = sp * a.qjl_const;
  }
}

// ---------------------------------------------------------------------------
// key preparation: one lane per key
// ---------------------------------------------------------------------------
template <int BITS, bool NORM_F32>
__global__ __launch_bounds__(256) void prep_keys(ScoreArgs a) {
  constexpr int NP = 1 << (BITS - 1);
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= a.n_k_pad) return;
  const int dt = a.dt, m = a.m, Kd = a.kd, Km = a.km;
  const int RK = NP * Kd + Km;
  uint32_t* rec = reinterpret_cast<uint32_t*>(a.krec + j * RK);
  const bool live = j < a.n_k;
  // ternary planes, 4 coordinates per dword
  for (int d4 = 0; d4 < Kd; d4 += 4) {
    uint32_t planes[NP];
#pragma unroll
    for (int t = 0; t < NP; ++t) planes[t] = 0u;
    if (live) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d = d4 + k;
        if (d >= dt) break;
        const int pos = BITS * d;  // coordinate d of the unit: group d/32, bit BITS*(d%32) -> same as BITS*d
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(a.codes + j * (dt * BITS / 8));
        uint32_t c = wp[pos >> 5] >> (pos & 31);
        if ((pos & 31) + BITS > 32) c |= wp[(pos >> 5) + 1] << (32 - (pos & 31));
        c &= (1u << BITS) - 1;
        const uint32_t mag = c & ((1u << (BITS - 1)) - 1);
        const uint32_t sgn_byte = (c >> (BITS - 1)) ? 0xFFu : 0x01u;
#pragma unroll
        for (int t = 0; t < NP; ++t)
          if ((mag & (uint32_t)t) == (uint32_t)t) planes[t] |= sgn_byte << (8 * k);
      }
    }
#pragma unroll
    for (int t = 0; t < NP; ++t) rec[(t * Kd + d4) / 4] = planes[t];
  }
  // sign plane: +1 where the bit is set, -1 where clear
  for (int p4 = 0; p4 < Km; p4 += 4) {
    uint32_t w = 0u;
    if (live) {
      const uint8_t* sb = a.qjl_bits + j * (m / 8);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int p = p4 + k;
        if (p >= m) break;
        const uint32_t bit = (sb[p >> 3] >> (p & 7)) & 1u;
        w |= (bit ? 0x01u : 0xFFu) << (8 * k);
      }
    }
    rec[(NP * Kd + p4) / 4] = w;
  }
  float n = 0.0f, rho = 0.0f;
  if (live) {
    if constexpr (NORM_F32)
      n = static_cast<const float*>(a.norms)[j];
    else
      n = __half2float(static_cast<const __half*>(a.norms)[j]);
    rho = __half2float(__ushort_as_half(a.rnorm[j]));
  }
  a.kscale[2 * j] = n;
  a.kscale[2 * j + 1] = n * rho;
}

// ---------------------------------------------------------------------------
// scores: workgroup = 4 waves x (16*CB keys each), loops over 16-query blocks
//
// Keys are the MFMA's A operand and queries its B operand, so each lane's
// accumulator holds 4 consecutive keys of one query: one 16-byte store per
// 16-key tile writes them.  The next block's query records are fetched into
// registers before this block's MFMAs and parked in the other LDS buffer
// after them, so one barrier per block suffices and the L2 latency of the
// fetch hides behind the contraction.
// ---------------------------------------------------------------------------
template <int NP, int KD, int KM, int CB>
__global__ __launch_bounds__(256) void scores_kernel(ScoreArgs a) {
  constexpr int Kd = 64 * KD, Km = 64 * KM, RQ = 2 * (Kd + Km), RK = NP * Kd + Km;
  constexpr int QV = kQB * RQ / 16;  // 16-byte vectors per query block
  constexpr int PER = (QV + 255) / 256;
  __shared__ __attribute__((aligned(16))) int8_t qblk[2][kQB * RQ];
  __shared__ float qs[2][kQB * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col_l = lane & 15, slot = lane >> 4;
  const int64_t key0 = (int64_t)blockIdx.x * (64 * CB) + wave * (16 * CB);

  // this wave's key-side operands (row col_l of each 16-key tile), kept in registers
  v4i bT[CB][NP][KD], bS[CB][KM];
  float nk[CB][4], nrk[CB][4];  // scales of the 4 keys 16 cb + 4 slot + i whose scores this lane writes
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int64_t key = key0 + 16 * cb + col_l;
    const int8_t* rec = a.krec + key * RK;
#pragma unroll
    for (int t = 0; t < NP; ++t)
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) bT[cb][t][ks] = *reinterpret_cast<const v4i*>(rec + t * Kd + 64 * ks + 16 * slot);
#pragma unroll
    for (int ks = 0; ks < KM; ++ks) bS[cb][ks] = *reinterpret_cast<const v4i*>(rec + NP * Kd + 64 * ks + 16 * slot);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t kk = key0 + 16 * cb + 4 * slot + i;
      nk[cb][i] = a.kscale[2 * kk];
      nrk[cb][i] = a.kscale[2 * kk + 1];
    }
  }
  float w[NP];
#pragma unroll
  for (int t = 0; t < NP; ++t) w[t] = a.plane_w[t];
  // 16-byte stores need 16-byte aligned rows
  const bool vec = ((a.ld_s & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.scores) & 15) == 0);

  const int64_t q_begin = (int64_t)blockIdx.y * kQChunk;
  const int64_t q_end = q_begin + kQChunk < a.n_q_pad ? q_begin + kQChunk : a.n_q_pad;
  const v4i* qrec_v = reinterpret_cast<const v4i*>(a.qrec);
  v4i pre[PER];
  float pqs = 0.0f;
  auto fetch = [&](int64_t r0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = tid + 256 * p;
      if (e < QV) pre[p] = qrec_v[r0 * (RQ / 16) + e];
    }
    if (tid < kQB * 2) pqs = a.qscale[r0 * 2 + tid];
  };
  auto park = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int e = tid + 256 * p;
      if (e < QV) reinterpret_cast<v4i*>(qblk[buf])[e] = pre[p];
    }
    if (tid < kQB * 2) qs[buf][tid] = pqs;
  };
  fetch(q_begin);
  park(0);
  __syncthreads();

  int cur = 0;
  for (int64_t r0 = q_begin; r0 < q_end; r0 += kQB, cur ^= 1) {
    const bool more = r0 + kQB < q_end;
    if (more) fetch(r0 + kQB);

    v4i accT[CB][NP], accS[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int t = 0; t < NP; ++t) accT[cb][t] = v4i{0, 0, 0, 0};
      accS[cb] = v4i{0, 0, 0, 0};
    }
    const int8_t* qrow = qblk[cur] + col_l * RQ + 16 * slot;
#pragma unroll
    for (int limb = 0; limb < 2; ++limb) {
      if (limb == 1) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
          for (int t = 0; t < NP; ++t) accT[cb][t] <<= 8;
          accS[cb] <<= 8;
        }
      }
#pragma unroll
      for (int ks = 0; ks < KD; ++ks) {
        const v4i bq = *reinterpret_cast<const v4i*>(qrow + limb * Kd + 64 * ks);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int t = 0; t < NP; ++t)
            accT[cb][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bT[cb][t][ks], bq, accT[cb][t], 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < KM; ++ks) {
        const v4i bp = *reinterpret_cast<const v4i*>(qrow + 2 * Kd + limb * Km + 64 * ks);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) accS[cb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bS[cb][ks], bp, accS[cb], 0, 0, 0);
      }
    }
    if (more) park(cur ^ 1);

    // epilogue: lane holds keys 16 cb + 4 slot + i of query r0 + col_l
    const float alpha = qs[cur][2 * col_l], beta = qs[cur][2 * col_l + 1];
    v4f val[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sum = 0.0f;
#pragma unroll
        for (int t = 0; t < NP; ++t) sum = __builtin_fmaf(w[t], (float)accT[cb][t][i], sum);
        val[cb][i] = nk[cb][i] * (alpha * sum) + nrk[cb][i] * (beta * (float)accS[cb][i]);
      }
    const int64_t row = r0 + col_l;
    float* out = a.scores + row * a.ld_s + key0 + 4 * slot;
    if (vec && key0 + 16 * CB <= a.n_k && r0 + kQB <= a.n_q) {  // whole tile inside the matrix (wave-uniform)
      // plain (cached) stores: L2 merges the 64-byte row pieces of the 16 queries into whole lines
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) *reinterpret_cast<v4f*>(out + 16 * cb) = val[cb];
    } else if (row < a.n_q) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + 16 * cb + 4 * slot + i < a.n_k) out[16 * cb + i] = val[cb][i];
    }
    __syncthreads();
  }
}

template <int NP, int KD, int KM>
hipError_t launch_scores_t(const ScoreArgs& a, hipStream_t s) {
  constexpr int CB = NP <= 2 ? 4 : 2;
  dim3 grid((unsigned)(a.n_k_pad / (64 * CB)), (unsigned)((a.n_q_pad + kQChunk - 1) / kQChunk));
  hipLaunchKernelGGL((scores_kernel<NP, KD, KM, CB>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int NP>
hipError_t launch_scores_np(const ScoreArgs& a, hipStream_t s) {
  const int kd = a.kd / 64, km = a.km / 64;
  if (kd == 1 && km == 1) return launch_scores_t<NP, 1, 1>(a, s);
  if (kd == 1 && km == 2) return launch_scores_t<NP, 1, 2>(a, s);
  if (kd == 2 && km == 1) return launch_scores_t<NP, 2, 1>(a, s);
  return launch_scores_t<NP, 2, 2>(a, s);
}

}  // namespace

int64_t scores_key_tile(int bits) { return bits <= 2 ? 256 : 128; }

hipError_t launch_qjl_scores(const tq_config& cfg, const ScoreArgs& a, hipStream_t s) {
  const size_t lds = (size_t)kQB * (a.dt + a.m) * sizeof(float);
  dim3 gq((unsigned)(a.n_q_pad / kQB));
  if (a.q_f32)
    hipLaunchKernelGGL((prep_queries<true>), gq, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((prep_queries<false>), gq, dim3(256), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 gk((unsigned)((a.n_k_pad + 255) / 256));
  const bool n32 = cfg.norm_dtype == TQ_F32;
  switch (cfg.bits) {
    case 1:
      if (n32) hipLaunchKernelGGL((prep_keys<1, true>), gk, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((prep_keys<1, false>), gk, dim3(256), 0, s, a);
      break;
    case 2:
      if (n32) hipLaunchKernelGGL((prep_keys<2, true>), gk, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((prep_keys<2, false>), gk, dim3(256), 0, s, a);
      break;
    default:
      if (n32) hipLaunchKernelGGL((prep_keys<3, true>), gk, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((prep_keys<3, false>), gk, dim3(256), 0, s, a);
      break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (cfg.bits) {
    case 1: return launch_scores_np<1>(a, s);
    case 2: return launch_scores_np<2>(a, s);
    default: return launch_scores_np<4>(a, s);
  }
}

}  // namespace tq
