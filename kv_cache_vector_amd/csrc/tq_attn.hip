// Single-token decode attention over a block-32 quantized KV cache (gfx950).
//
// [Fork] "Fused tile path: K and V decoded inside attention": work in the
// Hadamard domain so that no per-token inverse transform is needed.
//   keys:   <q_b, D H c_b> = <H D q_b, c_b>, so each query block is rotated
//           once (H, D symmetric) and scored directly against the centroids;
//   values: sum_j p_j D H c_j = D H sum_j p_j c_j, so the weighted sum stays
//           in the rotated domain and one inverse transform per output block
//           runs at the very end.
// All query heads of one KV head share every K and V read ([Fork] GQA note:
// the decode kernel must serve the whole query group per KV read).
//
// Per workgroup: one KV head, a range of tokens, 4 waves of 256 tokens each,
// 32-token tiles:
//   K side   each lane expands the 3/4-bit codes of 8 coordinates of one token
//            through an LDS pair table into fp16 hi/lo operands; three
//            v_mfma_f32_16x16x32_f16 per 32-block (q_hi c_hi + q_lo c_hi +
//            q_hi c_lo) give the block dot products to ~2^-22, each scaled by
//            the block norm in fp32 and summed over blocks.
//   softmax  online (running max and sum) per query head over 16-lane rows.
//   V side   codes expanded token-major into a wave-private LDS tile (16-dim
//            chunks XOR-swizzled by token); ds_read_b64_tr_b16 returns four
//            tokens of one coordinate per lane, the operand layout of the
//            value MFMA (K = 32 tokens); the block norms of V are folded into
//            the softmax weights (A operand, fp16).
// Each wave writes its partial (acc, max, sum); a merge kernel rescales and
// adds the partials, then applies D_V H once per 32-block.
#include <hip/hip_fp16.h>

#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) short lds_short;

constexpr int kAttnWaves = 4;
constexpr int kTile = 32;                       // tokens per tile (K of the value MFMA)
constexpr int kTokPerWave = 256;
constexpr int kTokPerWG = kAttnWaves * kTokPerWave;

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__device__ __forceinline__ float row16_max(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// bits [pos, pos + width) of a little-endian multi-word code record
__device__ __forceinline__ uint32_t bits_at(const uint32_t* w, int pos, int width) {
  const int wi = pos >> 5, sh = pos & 31;
  if (sh + width <= 32) return __builtin_amdgcn_ubfe(w[wi], sh, width);
  return __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh), 0, width);
}

template <int NB, int KB, int VB, int GM>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  constexpr int HD = NB * 32;
  constexpr int KL = 1 << KB, VL = 1 << VB;
  __shared__ uint2 ktab[KL * KL];      // pair of K codes -> (fp16 hi pair, fp16 lo pair)
  __shared__ uint32_t vtab[VL * VL];   // pair of V codes -> fp16 pair
  __shared__ __attribute__((aligned(16))) _Float16 qh[GM * HD];
  __shared__ __attribute__((aligned(16))) _Float16 ql[GM * HD];
  __shared__ __attribute__((aligned(16))) _Float16 vt[kAttnWaves][kTile * HD];
  __shared__ _Float16 vn[kAttnWaves][kTile * NB];
  __shared__ float pt[kAttnWaves][GM * kTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.y;
  const int G = a.group;

  for (int e = tid; e < KL * KL; e += 256) {
    const float ca = a.klevel[e & (KL - 1)], cb = a.klevel[e >> KB];
    const _Float16 ha = (_Float16)ca, hb = (_Float16)cb;
    const _Float16 la = (_Float16)(ca - (float)ha), lb = (_Float16)(cb - (float)hb);
    ktab[e] = make_uint2(pack_h2(ha, hb), pack_h2(la, lb));
  }
  for (int e = tid; e < VL * VL; e += 256)
    vtab[e] = pack_h2((_Float16)a.vlevel[e & (VL - 1)], (_Float16)a.vlevel[e >> VB]);

  // rotated query blocks of this KV head's group: qhat_b = H D_K q_b / sqrt(32), split fp16 hi + lo
  float* qf = reinterpret_cast<float*>(&vt[0][0]);  // GM * HD floats, staging only
  for (int e = tid; e < GM * HD; e += 256) {
    const int r = e / HD, d = e % HD;
    float v = 0.0f;
    if (r < G) {
      const int64_t off = (int64_t)(kvh * G + r) * HD + d;
      v = a.q_f32 ? static_cast<const float*>(a.q)[off] : __half2float(static_cast<const __half*>(a.q)[off]);
    }
    qf[e] = ((a.kdbits >> (d & 31)) & 1u) ? -v : v;
  }
  __syncthreads();
  for (int hb = 1; hb < 32; hb <<= 1) {
    for (int e = tid; e < GM * HD / 2; e += 256) {
      const int r = e / (HD / 2), rem = e % (HD / 2), b = rem / 16, p = rem % 16;
      const int i = (p / hb) * 2 * hb + (p % hb);
      float* blk = qf + r * HD + 32 * b;
      const float x = blk[i], y = blk[i + hb];
      blk[i] = x + y;
      blk[i + hb] = x - y;
    }
    __syncthreads();
  }
  for (int e = tid; e < GM * HD; e += 256) {
    const float v = qf[e] * 0.17677669529663688f;  // 1/sqrt(32)
    const _Float16 h = (_Float16)v;
    qh[e] = h;
    ql[e] = (_Float16)(v - (float)h);
  }
  __syncthreads();

  // this lane's query operands (read per block from LDS): row = query head of the group,
  // coordinates 8g..8g+7 of the block; rows >= GM multiply zeros
  const int qrow = row < GM ? row : 0;
  const bool qlive = row < GM;

  const int64_t T = a.n_tokens;
  const uint8_t* kbase = a.k_codes + (int64_t)kvh * T * NB * (4 * KB);
  const uint8_t* vbase = a.v_codes + (int64_t)kvh * T * NB * (4 * VB);
  const uint16_t* knb = a.k_norms + (int64_t)kvh * T * NB;
  const uint16_t* vnb = a.v_norms + (int64_t)kvh * T * NB;
  _Float16* vtile = vt[wave];
  float m_run[4], lsum[4];
  v4f acc[NB][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    lsum[i] = 0.0f;
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b][0] = acc[b][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t t_begin = (int64_t)blockIdx.x * a.tokens_per_wg + (int64_t)wave * kTokPerWave;
  const int64_t t_end = t_begin + kTokPerWave < T ? t_begin + kTokPerWave : T;
  for (int64_t tb = t_begin; tb < t_end; tb += kTile) {
    // ---- value tile: decode token-major into LDS (chunk c of token t at chunk c ^ (t & 7))
#pragma unroll
    for (int k = 0; k < NB / 2; ++k) {
      const int u = lane + 64 * k, t = u / NB, b = u % NB;
      const int64_t tok = tb + t;
      uint32_t w[VB] = {};
      _Float16 nv = (_Float16)0.0f;
      const bool live = tok < T;
      if (live) {
        const uint32_t* rp = reinterpret_cast<const uint32_t*>(vbase + (tok * NB + b) * (4 * VB));
#pragma unroll
        for (int q = 0; q < VB; ++q) w[q] = rp[q];
        nv = __builtin_bit_cast(_Float16, vnb[tok * NB + b]);
      }
      vn[wave][t * NB + b] = nv;
      uint32_t o[16];
#pragma unroll
      for (int pp = 0; pp < 16; ++pp) o[pp] = live ? vtab[bits_at(w, 2 * VB * pp, 2 * VB)] : 0u;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = 2 * b + half;
        _Float16* dst = vtile + t * HD + 16 * (c ^ (t & 7));
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(o[8 * half], o[8 * half + 1], o[8 * half + 2], o[8 * half + 3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(o[8 * half + 4], o[8 * half + 5], o[8 * half + 6], o[8 * half + 7]);
      }
    }

    // ---- key side: scores of 2 x 16 tokens for the group's query heads
    float s[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int64_t tok = tb + 16 * st + row;
      const bool live = tok < T;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[st][i] = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // this lane's 8 coordinates 8g..8g+7 of block b: 8*KB bits from bit 8*g*KB of the record
        uint32_t win = 0u;
        float nk = 0.0f;
        if (live) {
          const uint32_t* rp = reinterpret_cast<const uint32_t*>(kbase + (tok * NB + b) * (4 * KB));
          const int pos = 8 * KB * g, i0 = pos >> 5, i1 = i0 + 1 < KB ? i0 + 1 : KB - 1;
          win = __builtin_amdgcn_alignbit(rp[i1], rp[i0], pos & 31);
          nk = __half2float(__ushort_as_half(knb[tok * NB + b]));
        }
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint2 e = ktab[__builtin_amdgcn_ubfe(win, 2 * KB * pp, 2 * KB)];
          bh[pp] = e.x;
          bl[pp] = e.y;
        }
        const v8h bhi = __builtin_bit_cast(v8h, make_uint4(bh[0], bh[1], bh[2], bh[3]));
        const v8h blo = __builtin_bit_cast(v8h, make_uint4(bl[0], bl[1], bl[2], bl[3]));
        v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
        const v8h zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
        const v8h aqh = qlive ? *reinterpret_cast<const v8h*>(&qh[qrow * HD + 32 * b + 8 * g]) : zero8;
        const v8h aql = qlive ? *reinterpret_cast<const v8h*>(&ql[qrow * HD + 32 * b + 8 * g]) : zero8;
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqh, bhi, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(aql, bhi, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqh, blo, c, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[st][i] = __builtin_fmaf(nk, c[i], s[st][i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) s[st][i] = live ? s[st][i] * a.kscale : -INFINITY;
    }

    // ---- online softmax: row 4g + i of the tile, reduced over the 16 token lanes
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mt = row16_max(fmaxf(s[0][i], s[1][i]));
      const float m_new = fmaxf(m_run[i], mt);
      const bool none = m_new == -INFINITY;
      const float alpha = (none || m_run[i] == -INFINITY) ? 0.0f : __expf(m_run[i] - m_new);
      const float p0 = none ? 0.0f : __expf(s[0][i] - m_new);
      const float p1 = none ? 0.0f : __expf(s[1][i] - m_new);
      lsum[i] = lsum[i] * alpha + row16_sum(p0 + p1);
      m_run[i] = m_new;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        acc[b][0][i] *= alpha;
        acc[b][1][i] *= alpha;
      }
      const int r = 4 * g + i;
      if (r < GM) {
        pt[wave][r * kTile + row] = p0;
        pt[wave][r * kTile + 16 + row] = p1;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- value side: A = softmax weight * value norm (fp16), B = 4 tokens x 1 coordinate per tr read
    float pa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pa[j] = (row < G && row < GM) ? pt[wave][row * kTile + 8 * g + j] : 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      v8h av;
#pragma unroll
      for (int j = 0; j < 8; ++j) av[j] = (_Float16)(pa[j] * (float)vn[wave][(8 * g + j) * NB + b]);
#pragma unroll
      for (int nh = 0; nh < 2; ++nh) {
        const int c = 2 * b + nh;
        const int t1 = 8 * g + (row >> 2), t2 = t1 + 4;
        lds_short* base = (lds_short*)vtile;
        const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(base + t1 * HD + 16 * (c ^ (t1 & 7)) + 4 * (row & 3)));
        const v4s r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(base + t2 * HD + 16 * (c ^ (t2 & 7)) + 4 * (row & 3)));
        const v4h h1 = __builtin_bit_cast(v4h, r1), h2 = __builtin_bit_cast(v4h, r2);
        const v8h bv = {h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
        acc[b][nh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[b][nh], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- this wave's partial: acc rows = query heads 4g + i, columns = coordinates
  const int64_t pw = ((int64_t)kvh * a.wg_per_head + blockIdx.x) * kAttnWaves + wave;
  float* pbase = a.part + pw * G * (HD + 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    if (r >= G) continue;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      pbase[r * (HD + 2) + 32 * b + row] = acc[b][0][i];
      pbase[r * (HD + 2) + 32 * b + 16 + row] = acc[b][1][i];
    }
    if (row == 0) {
      pbase[r * (HD + 2) + HD] = m_run[i];
      pbase[r * (HD + 2) + HD + 1] = lsum[i];
    }
  }
}

// Merge: one workgroup per (query head, 32-block); threads (part lane pl, coordinate dl).
__global__ __launch_bounds__(256) void attn_merge(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, HD = a.head_dim, G = a.group;
  const int kvh = h / G, r = h % G;
  const int tid = threadIdx.x, pl = tid >> 5, dl = tid & 31;
  const int n_part = a.wg_per_head * kAttnWaves;
  const float* base = a.part + (int64_t)kvh * n_part * G * (HD + 2);
  __shared__ float red[8][33];
  __shared__ float mx;
  // global max over the partials' running maxima
  float m = -INFINITY;
  for (int p = tid; p < n_part; p += 256) m = fmaxf(m, base[((int64_t)p * G + r) * (HD + 2) + HD]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6][32] = m;
  __syncthreads();
  if (tid == 0) {
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red[w][32]);
    mx = mm;
  }
  __syncthreads();
  const float M = mx;
  float acc = 0.0f, l = 0.0f;
  for (int p = pl; p < n_part; p += 8) {
    const float* pb = base + ((int64_t)p * G + r) * (HD + 2);
    const float mp = pb[HD];
    if (mp == -INFINITY) continue;
    const float f = __expf(mp - M);
    acc = __builtin_fmaf(pb[32 * b + dl], f, acc);
    l = __builtin_fmaf(pb[HD + 1], f, l);
  }
  __syncthreads();
  red[pl][dl] = acc;
  if (dl == 0) red[pl][32] = l;
  __syncthreads();
  if (pl == 0) {
    float s = 0.0f, ls = 0.0f;
    for (int q = 0; q < 8; ++q) {
      s += red[q][dl];
      ls += red[q][32];
    }
    // out = D_V * H_unnorm(acc) / (32 * l): butterflies across the 32 lanes of the first wave
    float v = s;
    for (int hb = 1; hb < 32; hb <<= 1) {
      const float o = __shfl_xor(v, hb);
      v = (dl & hb) ? o - v : v + o;
    }
    v = v / (32.0f * ls);
    if ((a.vdbits >> dl) & 1u) v = -v;
    a.out[(int64_t)h * HD + 32 * b + dl] = v;
  }
}

template <int NB, int KB, int VB>
hipError_t launch_nb(const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.wg_per_head, (unsigned)a.n_kv_heads);
  if (a.group <= 4)
    hipLaunchKernelGGL((attn_kernel<NB, KB, VB, 4>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<NB, KB, VB, 16>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge, dim3((unsigned)a.n_q_heads, (unsigned)(a.head_dim / 32)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_bits(const AttnArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_nb<4, KB, VB>(a, s) : launch_nb<8, KB, VB>(a, s);
}

}  // namespace

int attn_tokens_per_wg() { return kTokPerWG; }

hipError_t launch_decode_attn(int kbits, int vbits, const AttnArgs& a, hipStream_t s) {
  if (kbits == 3 && vbits == 3) return launch_bits<3, 3>(a, s);
  if (kbits == 4 && vbits == 4) return launch_bits<4, 4>(a, s);
  if (kbits == 3 && vbits == 4) return launch_bits<3, 4>(a, s);
  return launch_bits<4, 3>(a, s);
}

}  // namespace tq
