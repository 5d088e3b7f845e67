// Attention of many query rows over a block-32 quantized KV cache (gfx950): the
// prefill-chunk kernel behind tq_multi_attn when a KV head has more than 16
// (query token, head) rows.  Built without the VGPR-form MFMA option, so its
// value accumulators can sit in the accumulation registers.
#include <hip/hip_fp16.h>

#include "tq_attn_common.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

using namespace attn;

// ---------------------------------------------------------------------------------------------
// Several query tokens (a prefill chunk): a workgroup of 8 waves takes 128 rows of one KV head
// ((query token, head) pairs, 16 per wave) and a token range.  Per
// 64-token tile the whole workgroup decodes K (fp16 hi and lo parts of the unit-scale centroids)
// and V (fp16 centroids times the block norm) once into LDS, one (token, block) unit per thread;
// each wave then scores its rows against the decoded keys (split-fp16 16x16x32 MFMAs, block
// norms applied per block in fp32), runs the online
// softmax of its rows and adds p V with the value MFMA.  Decoding is shared by 128 rows instead
// of the 16 of the decode kernel.  The partials and the merge are the decode kernel's.
constexpr int kPWaves = 8;
constexpr int kPRT = 1;                       // 16-row tiles per wave
constexpr int kPRows = 16 * kPRT * kPWaves;   // rows per workgroup

template <int NB, int KB, int VB>
__global__ __launch_bounds__(64 * kPWaves, 1) void prefill_kernel(AttnArgs a) {
  constexpr int HD = NB * 32;
  constexpr bool K8 = KB == 8;
  constexpr int KL = 1 << KB, VL = 1 << VB;
  constexpr int LGCK = K8 ? 4 : (KB == 3 ? 5 : 3), LGCV = VB == 3 ? 5 : 3;
  constexpr int CK = 1 << LGCK, CV = 1 << LGCV;
  constexpr int SLOTS = HD / 8;  // 16-byte slots per decoded token row
  constexpr int NCT = HD / 16;   // 16-coordinate output tiles
  constexpr int PSTR = kTile + 8;  // fp16 per weight row (144 bytes: rows 4 apart land 64 banks apart)
  constexpr int NT = 64 * kPWaves;
  struct Smem {
    uint32_t ktab[K8 ? KL * CK : 2 * KL * KL * CK + 1];
    uint32_t vtab[VL * VL * CV];
    float kn[kTile][NB + 1];  // +1: the 16 tokens of a subtile read distinct banks
    __attribute__((aligned(16))) _Float16 khi[kTile * HD];
    __attribute__((aligned(16))) _Float16 klo[kTile * HD];
    __attribute__((aligned(16))) _Float16 vt[kTile * HD];
    __attribute__((aligned(16))) _Float16 pt[kPWaves][kPRT * 16 * PSTR];
  };
  __shared__ Smem sm;
  uint32_t* kth = sm.ktab;
  uint32_t* ktl = sm.ktab + (K8 ? 0 : KL * KL * CK + 1);
  // K rows: slot 4b + g (8 coordinates) of token t at slot ^ (t & 15), so the 16 tokens of a
  // subtile read one slot each from distinct banks, and 16 consecutive tokens written by 16
  // lanes (one block each) do too.  V rows: slot 2c + k (half k of 16-coordinate chunk c) at
  // slot ^ vsw(t), distinct over the 16 tokens one transposing load reads.
  auto kslot = [](int t, int slot) { return t * HD + 8 * (slot ^ (t & 15)); };
  auto vsw = [](int t) { return (2 * ((((t >> 3) & 3) << 2) | (t & 3))) & (SLOTS - 1); };
  auto vslot = [&](int t, int c, int k) { return t * HD + 8 * ((2 * c + k) ^ vsw(t)); };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.y / a.n_rg, rg = blockIdx.y % a.n_rg;
  const int G = a.group;
  const int64_t T = a.n_tokens;
  const int64_t row0 = (int64_t)rg * kPRows + 16 * kPRT * wave;  // first row of this wave
  const uint32_t koff = (uint32_t)(lane & (CK - 1)) * 4u, voff = (uint32_t)(lane & (CV - 1)) * 4u;

  // (token, block) units of a tile: unit tid + NT * k of this thread, k < UPT
  constexpr int UNITS = kTile * NB;
  constexpr int UPT = UNITS >= NT ? UNITS / NT : 1;
  static_assert(UNITS % NT == 0 || NT % UNITS == 0, "whole units per thread");
  const bool decoder = tid < UNITS;
  const uint8_t* kbase = a.k_codes + (int64_t)kvh * T * NB * (4 * KB);
  const uint8_t* vbase = a.v_codes + (int64_t)kvh * T * NB * (4 * VB);
  const uint16_t* knb = a.k_norms + (int64_t)kvh * T * NB;
  const uint16_t* vnb = a.v_norms + (int64_t)kvh * T * NB;
  struct Raw {
    uint32_t kw[UPT][KB], vw[UPT][VB];
    uint32_t kn[UPT], vn[UPT];
  };
  auto load = [&](Raw& r, int64_t tb) {
    const int64_t rem = T - 1 - tb;
    const uint32_t last = rem < kTile ? (uint32_t)rem : (uint32_t)(kTile - 1);
    const uint32_t* kp0 = reinterpret_cast<const uint32_t*>(kbase + tb * NB * (4 * KB));
    const uint32_t* vp0 = reinterpret_cast<const uint32_t*>(vbase + tb * NB * (4 * VB));
#pragma unroll
    for (int k = 0; k < UPT; ++k) {
      const int u0 = tid + NT * k;
      const uint32_t t = min((uint32_t)(u0 % kTile), last);
      const uint32_t u = t * NB + (uint32_t)(u0 / kTile);
#pragma unroll
      for (int q = 0; q < KB; ++q) r.kw[k][q] = kp0[u * KB + q];
#pragma unroll
      for (int q = 0; q < VB; ++q) r.vw[k][q] = vp0[u * VB + q];
      r.kn[k] = knb[tb * NB + u];
      r.vn[k] = vnb[tb * NB + u];
    }
  };
  const int64_t t_begin = (int64_t)blockIdx.x * kTile;
  const int64_t t_step = (int64_t)a.wg_per_head * kTile;
  Raw raw;  // raw words of the next tile to decode
  if (decoder && t_begin < T) load(raw, t_begin);

  // Set-up reads from global memory in one round trip: the levels, staged in the K norm tile (which
  // the first tile is the first to write), and the query elements, all issued before any is used.
  float* lv = &sm.kn[0][0];
  static_assert(sizeof(sm.kn) >= sizeof(float) * (KL + VL), "levels fit the K norm tile");
  for (int x = tid; x < KL; x += NT) lv[x] = a.klevel[x];
  if (tid < VL) lv[KL + tid] = a.vlevel[tid];

  // query operands: row `row` of each row tile, coordinates 8g .. 8g + 7 of each block, rotated
  // by H D_K (butterflies in registers, then across the lanes 16 and 32 apart) and split into fp16
  // hi + lo parts of qhat / sqrt(32).  Rows past the live ones read row 0's query and are zeroed.
  v8h qh8[kPRT][NB], ql8[kPRT][NB];
#pragma unroll
  for (int rt = 0; rt < kPRT; ++rt) {
    const int64_t rr = row0 + 16 * rt + row;
    const bool live = rr < a.rows;
    const int64_t i = live ? rr / G : 0;
    const int64_t qoff = (i * a.n_q_heads + (int64_t)kvh * G + (live ? rr % G : 0)) * HD;
    float qx[NB][8];
    if (a.q_f32) {
      const float* q32 = static_cast<const float*>(a.q) + qoff;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) qx[b][j] = q32[32 * b + 8 * g + j];
    } else {
      const _Float16* q16 = static_cast<const _Float16*>(a.q) + qoff;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) qx[b][j] = (float)q16[32 * b + 8 * g + j];
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 32 * b + 8 * g + j;
        const float x = live ? qx[b][j] : 0.0f;
        v[j] = ((a.kdbits >> (d & 31)) & 1u) ? -x : x;
      }
#pragma unroll
      for (int hb = 1; hb < 8; hb <<= 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (!(j & hb)) {
            const float x = v[j], y = v[j | hb];
            v[j] = x + y;
            v[j | hb] = x - y;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = v[j];
        float o = __shfl_xor(x, 16);
        x = (g & 1) ? o - x : x + o;
        o = __shfl_xor(x, 32);
        x = (g & 2) ? o - x : x + o;
        x *= 0.17677669529663688f;  // 1/sqrt(32)
        qh8[rt][b][j] = (_Float16)x;
        ql8[rt][b][j] = (_Float16)(x - (float)qh8[rt][b][j]);
      }
    }
  }
  __syncthreads();  // levels

  if constexpr (K8) {
    for (int x = tid; x < KL * CK; x += NT) {
      const float c = lv[x / CK];
      const _Float16 h = (_Float16)c;
      kth[x] = pack_h2(h, (_Float16)(c - (float)h));
    }
  } else {
    for (int x = tid; x < KL * KL * CK; x += NT) {
      const int e = x / CK;
      const float ca = lv[e & (KL - 1)], cb = lv[e >> KB];
      const _Float16 ha = (_Float16)ca, hb = (_Float16)cb;
      kth[x] = pack_h2(ha, hb);
      ktl[x] = pack_h2((_Float16)(ca - (float)ha), (_Float16)(cb - (float)hb));
    }
  }
  for (int x = tid; x < VL * VL * CV; x += NT) {
    const int e = x / CV;
    sm.vtab[x] = pack_h2((_Float16)lv[KL + (e & (VL - 1))], (_Float16)lv[KL + (e >> VB)]);
  }

  const int64_t all_live = T - (a.causal ? a.n_q : 1);  // last token every row sees
  float m_run[kPRT][4], lsum[kPRT][4];
  v4f acc[kPRT][NCT];
#pragma unroll
  for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_run[rt][i] = kNoRef;
      lsum[rt][i] = 0.0f;
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) acc[rt][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }
  _Float16* ptile = sm.pt[wave];
  __syncthreads();  // tables

  auto tile = [&](Raw& cur, int64_t tb) {
    // ---- decode this thread's units: K hi/lo (unit scale), K norm, V x norm; one 16-byte slot
    // (8 coordinates) at a time, which keeps few decoded words live
#pragma unroll
    for (int k = 0; k < (decoder ? UPT : 0); ++k) {
      const int u0 = tid + NT * k, ut = u0 % kTile, ub = u0 / kTile;  // a wave decodes one block of all 64 tokens
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int pp = 4 * q + m;
          if constexpr (K8) {
            const uint32_t w = cur.kw[k][pp >> 1];
            const uint32_t e0 = lut_word(kth, w, 16 * (pp & 1), 8, LGCK, koff);
            const uint32_t e1 = lut_word(kth, w, 16 * (pp & 1) + 8, 8, LGCK, koff);
            hi[m] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
            lo[m] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
          } else {
            const int pos = 2 * KB * pp, wi = pos >> 5, sh = pos & 31;
            const uint32_t w =
                sh + 2 * KB <= 32 ? cur.kw[k][wi] : __builtin_amdgcn_alignbit(cur.kw[k][wi + 1], cur.kw[k][wi], sh);
            const int s2 = sh + 2 * KB <= 32 ? sh : 0;
            hi[m] = lut_word(kth, w, s2, 2 * KB, LGCK, koff);
            lo[m] = lut_word(ktl, w, s2, 2 * KB, LGCK, koff);
          }
        }
        *reinterpret_cast<uint4*>(sm.khi + kslot(ut, 4 * ub + q)) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4*>(sm.klo + kslot(ut, 4 * ub + q)) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
      sm.kn[ut][ub] = __half2float(__ushort_as_half((uint16_t)cur.kn[k]));
      const _Float16 nv = __builtin_bit_cast(_Float16, (uint16_t)cur.vn[k]);
      const v2h nv2 = {nv, nv};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int pp = 4 * q + m;
          const int pos = 2 * VB * pp, wi = pos >> 5, sh = pos & 31;
          const uint32_t w =
              sh + 2 * VB <= 32 ? cur.vw[k][wi] : __builtin_amdgcn_alignbit(cur.vw[k][wi + 1], cur.vw[k][wi], sh);
          const int s2 = sh + 2 * VB <= 32 ? sh : 0;
          const v2h c = __builtin_bit_cast(v2h, lut_word(sm.vtab, w, s2, 2 * VB, LGCV, voff));
          o[m] = __builtin_bit_cast(uint32_t, c * nv2);
        }
        *reinterpret_cast<uint4*>(sm.vt + vslot(ut, 2 * ub + (q >> 1), q & 1)) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    // the raw words are dead once decoded: the same registers take the next tile's loads, which
    // stay in flight through this tile's scores and values
    const int64_t tn = tb + t_step;
    if (decoder) load(cur, tn < T ? tn : tb);
    __syncthreads();

    // ---- scores of the wave's rows against the 64 tokens (4 subtiles of 16)
    float s[kPRT][4][4];
#pragma unroll
    for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[rt][st][i] = 0.0f;
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int t = 16 * st + row;
        const v8h bhi = *reinterpret_cast<const v8h*>(sm.khi + kslot(t, 4 * b + g));
        const v8h blo = *reinterpret_cast<const v8h*>(sm.klo + kslot(t, 4 * b + g));
        const float nk = sm.kn[t][b];
#pragma unroll
        for (int rt = 0; rt < kPRT; ++rt) {
          v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh8[rt][b], bhi, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql8[rt][b], bhi, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(qh8[rt][b], blo, c, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) s[rt][st][i] = __builtin_fmaf(nk, c[i], s[rt][st][i]);
        }
      }
      // keep the key operands of one block live at a time (the scheduler would otherwise hoist
      // the LDS reads of every block and run out of registers)
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane (row, g) holds rows 16 rt + 4g + i of token 16 st + row
    if (tb + kTile - 1 <= all_live) {  // every row sees the whole tile
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[rt][st][i] *= a.kscale;
        }
      }
    } else {  // the last token of row rr is n_tokens - n_q + rr / group (causal) or n_tokens - 1
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t rr = row0 + 16 * rt + 4 * g + i;
          const int64_t lim = a.causal && rr < a.rows ? T - a.n_q + rr / G : T - 1;
#pragma unroll
          for (int st = 0; st < 4; ++st)
            s[rt][st][i] = tb + 16 * st + row <= lim ? s[rt][st][i] * a.kscale : -INFINITY;
        }
      }
    }

    // ---- online softmax of the wave's rows (reference moved lazily, as in the decode kernel)
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int st = 0; st < 4; ++st) grow |= s[rt][st][i] > m_run[rt][i] + kSlack;
      }
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float mt = fmaxf(fmaxf(s[rt][0][i], s[rt][1][i]), fmaxf(s[rt][2][i], s[rt][3][i]));
          mt = head_reduce<1, true>(mt);
          const float m_new = fmaxf(m_run[rt][i], mt);
          const float alpha = __expf(m_run[rt][i] - m_new);
          lsum[rt][i] *= alpha;
          m_run[rt][i] = m_new;
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) acc[rt][ct][i] *= alpha;
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const float p = __expf(s[rt][st][i] - m_run[rt][i]);
          lsum[rt][i] += p;
          ptile[(16 * rt + 4 * g + i) * PSTR + 16 * st + row] = (_Float16)p;
        }
      }
    }
    wave_sync();

    // ---- value side: acc[row][coordinate] += p[row][token] * (nV c)[token][coordinate]
#pragma unroll
    for (int half = 0; half < kTile / 32; ++half) {
      v8h av[kPRT];
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt)
        av[rt] = *reinterpret_cast<const v8h*>(ptile + (16 * rt + row) * PSTR + 32 * half + 8 * g);
      const int t1 = 32 * half + 8 * g + (row >> 2), t2 = t1 + 4;
      lds_short* base = (lds_short*)sm.vt;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(base + vslot(t1, ct, (row & 3) >> 1) + 4 * (row & 1)));
        const v4s r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)(base + vslot(t2, ct, (row & 3) >> 1) + 4 * (row & 1)));
        const v4h h1 = __builtin_bit_cast(v4h, r1), h2 = __builtin_bit_cast(v4h, r2);
        const v8h bv = {h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
#pragma unroll
        for (int rt = 0; rt < kPRT; ++rt)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[rt], bv, acc[rt][ct], 0, 0, 0);
        if (ct % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // the next tile's decode overwrites the tiles
  };

  for (int64_t tb = t_begin; tb < T; tb += t_step) tile(raw, tb);

  // ---- partials of the wave's rows: part[kvh][rg][wg][row][HD coordinates, reference, sum]
  float* pbase = a.part + ((int64_t)blockIdx.y * a.wg_per_head + blockIdx.x) * kPRows * (HD + 2);
#pragma unroll
  for (int rt = 0; rt < kPRT; ++rt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float l = head_reduce<1, false>(lsum[rt][i]);
      const int r = 16 * kPRT * wave + 16 * rt + 4 * g + i;
      if (row0 + 16 * rt + 4 * g + i >= a.rows) continue;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) pbase[r * (HD + 2) + 16 * ct + row] = acc[rt][ct][i];
      if (row == 0) {
        pbase[r * (HD + 2) + HD] = m_run[rt][i];
        pbase[r * (HD + 2) + HD + 1] = l;
      }
    }
  }
}

template <int NB, int KB, int VB>
hipError_t launch_nb(const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.wg_per_head, (unsigned)(a.n_kv_heads * a.n_rg));
  hipLaunchKernelGGL((prefill_kernel<NB, KB, VB>), grid, dim3(64 * kPWaves), 0, s, a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_bits(const AttnArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_nb<4, KB, VB>(a, s) : launch_nb<8, KB, VB>(a, s);
}

}  // namespace

int attn_prefill_rows() { return kPRows; }

hipError_t launch_prefill(int kbits, int vbits, const AttnArgs& a, hipStream_t s) {
  if (kbits == 3 && vbits == 3) return launch_bits<3, 3>(a, s);
  if (kbits == 4 && vbits == 4) return launch_bits<4, 4>(a, s);
  if (kbits == 3 && vbits == 4) return launch_bits<3, 4>(a, s);
  if (kbits == 4 && vbits == 3) return launch_bits<4, 3>(a, s);
  if (kbits == 8 && vbits == 3) return launch_bits<8, 3>(a, s);
  return launch_bits<8, 4>(a, s);
}

}  // namespace tq
