// Single-token decode attention over a block-32 quantized KV cache (gfx950).
//
// [Fork] "Fused tile path: K and V decoded inside attention": work in the
// Hadamard domain so that no per-token inverse transform is needed.
//   keys:   <q_b, D H c_b> = <H D q_b, c_b>, so each query block is rotated
//           once (H, D symmetric) and scored directly against the centroids;
//   values: sum_j p_j D H c_j = D H sum_j p_j c_j, so the weighted sum stays
//           in the rotated domain and one inverse transform per output block
//           runs at the very end.
// All query heads of one KV head share every K and V read (same page, "Fused
// kernel": without that GQA amortization a fused kernel loses to f16).
//
// Work split.  A workgroup owns one KV head and a token range and walks it in
// 64-token tiles; its 4 waves split the head's 32-blocks (wave w owns blocks
// w*NB/4 ..), so each wave reads only its blocks' codes and keeps only their
// accumulators.  Per tile:
//   loads    next tile's K windows, K/V norms and V records go straight to
//            registers one tile ahead (two register sets, no staging buffer);
//   K side   per owned block, the 64 tokens form 4 subtiles of 16; each lane
//            expands 8 coordinates of one token through an LDS pair table
//            (8-bit keys: a one-code table, two lookups per pair) into fp16
//            hi/lo operands, and three v_mfma_f32_16x16x32_f16
//            (q_hi c_hi + q_lo c_hi + q_hi c_lo) give the block dot products
//            to ~2^-22.  Row r of the query operand is head r % GP (GP = query
//            heads padded to 4, 8 or 16), so each subtile's 16x16 product
//            repeats its scores 16/GP times; lane group g keeps the product of
//            subtile slot 4g/GP, and every lane holds live scores of a distinct
//            (head, token); block norms scale them in fp32;
//   exchange the waves' partial scores (over their own blocks) are summed
//            through LDS, after which every wave holds the full scores;
//   softmax  online per query head against a running reference that only
//            moves when a score passes it by more than kSlack;
//   V side   one 32-token half of the tile at a time: each lane expands one
//            (token, block) record (pair table, scaled by the block norm with
//            one packed fp16 multiply per pair; at head_dim 128 two lanes split
//            a block) into a wave-private LDS tile of 32 rows;
//            ds_read_b64_tr_b16 returns four tokens of one coordinate per lane,
//            the B layout of the value MFMA (K = 32 tokens); the softmax
//            weights are the fp16 A operand.  Halving the tile keeps every
//            workgroup within half of the LDS: two share a compute unit, and
//            each wave may use up to 256 VGPRs.
// Each workgroup writes one partial (acc, max, sum) per query head; a merge
// kernel rescales and adds the partials, then applies D_V H once per block.
#include <hip/hip_fp16.h>

#include "tq_attn_common.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

using namespace attn;

constexpr int kWaves = 4;
constexpr int kMergeLanes = 8;


// One tile's worth of this lane's global data, loaded a tile ahead.
template <int NBW, int KB, int VB, int NC>
struct TileRegs {
  uint32_t kw[NBW][4][2];  // K: 2 words covering this lane's 8 coordinates, per owned block and subtile
  uint32_t kn[NC];         // K norms (fp16) of the token this lane scales, per accumulator; NBW halves
  uint32_t vw[2][VB];      // V: per 32-token half, the whole record of this lane's (token, block)
  uint32_t vn[2];          // V norms (fp16) of those two (token, block) units
};

template <int NB, int KB, int VB, int GP>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  constexpr int HD = NB * 32;
  constexpr int NBW = NB / kWaves;  // blocks per wave
  constexpr int S = 16 / GP;        // subtiles whose products one lane group picks from (slot 4g / GP)
  constexpr int NC = 4 / S;         // accumulators per block for the 4 subtiles
  constexpr int KL = 1 << KB, VL = 1 << VB;
  constexpr int VROW = NBW * 32;    // fp16 per V tile row (one token, the wave's blocks)
  constexpr int VT = kTile / 2;     // tokens per V tile: the value side runs in two 32-token halves
  constexpr int NXS = GP == 16 ? 1 : 2;  // score exchange buffers (one at 16 rows, saving LDS)
  constexpr int NCH = 2 * NBW;      // 16-coordinate chunks per V tile row
  // fp16 offset of 16-byte half k of chunk c in V tile row t.  Chunks are permuted by token bits
  // above the rows that share 256 bytes of banks, and the halves by bit 3, so the 16 rows written
  // by 16 consecutive lanes, and the rows read together by the transposing loads, use distinct banks.
  constexpr int RB = NBW == 2 ? 1 : 2;
  auto vslot = [](int t, int c, int k) {
    return t * VROW + 8 * (2 * (c ^ ((t >> RB) & (NCH - 1))) + (k ^ ((t >> 3) & 1)));
  };
  static_assert(NBW == 1 || NBW == 2, "head_dim 128 or 256");

  // Pair tables (two codes -> two fp16 levels, N(0,1) scale): K hi part, K lo part, V.  Each
  // entry is replicated in CK / CV copies interleaved at word granularity; lane l reads copy
  // l % C, so the random lookups of one instruction fall in distinct LDS banks.
  constexpr bool K8 = KB == 8;  // 8-bit keys: one-code table of (hi, lo) pairs instead of pair tables
  constexpr int LGCK = K8 ? 4 : (KB == 3 ? 5 : 3), LGCV = VB == 3 ? 5 : 3;
  constexpr int CK = 1 << LGCK, CV = 1 << LGCV;
  // hi and lo tables one word apart from a 256-byte multiple: their lookups at the same entry stay
  // two ds_read_b32 into the operand registers instead of one ds_read2st64 into a register pair
  constexpr int XSTR = kWaves * NC * 4 + 4;  // per-lane row of the score exchange (+4 breaks bank aliasing)
  // One LDS block with the lookup tables first, so that their addresses fit the 16-bit immediate
  // offset of ds_read and a lookup address is one and-or of the shifted code bits with the copy offset.
  struct Smem {
    uint32_t ktab[K8 ? KL * CK : 2 * KL * KL * CK + 1];
    uint32_t vtab[VL * VL * CV];
    __attribute__((aligned(16))) _Float16 vt[kWaves][VT * VROW];
    __attribute__((aligned(16))) _Float16 pt[kWaves][GP * kTile];
    __attribute__((aligned(16))) float xs[NXS][64][XSTR];
  };
  __shared__ Smem sm;
  uint32_t* ktab = sm.ktab;
  uint32_t* kth = ktab;
  uint32_t* ktl = ktab + (K8 ? 0 : KL * KL * CK + 1);
  uint32_t* vtab = sm.vtab;
  auto& vt = sm.vt;
  auto& pt = sm.pt;
  auto& xs = sm.xs;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.y / a.n_rg, rg = blockIdx.y % a.n_rg;
  const int G = a.group;
  const int64_t row0 = (int64_t)rg * a.grp;                                 // first row of the group
  const int grows = (int)(a.rows - row0 < a.grp ? a.rows - row0 : a.grp);  // live rows in the group
  const uint32_t koff = (uint32_t)(lane & (CK - 1)) * 4u, voff = (uint32_t)(lane & (CV - 1)) * 4u;

  const int64_t T = a.n_tokens;
  const uint8_t* kbase = a.k_codes + (int64_t)kvh * T * NB * (4 * KB);
  const uint8_t* vbase = a.v_codes + (int64_t)kvh * T * NB * (4 * VB);
  const uint16_t* knb = a.k_norms + (int64_t)kvh * T * NB;
  const uint16_t* vnb = a.v_norms + (int64_t)kvh * T * NB;
  const int b0 = NBW * wave;  // first owned block

  // this lane's K window: bits [24g, 24g + 24) of a 3-bit record, from the 8 bytes at word
  // kword (0, 0, 1, 1 for g = 0..3) shifted right by 0, 24, 16 or 40 bits; word g of a 4-bit
  // record; words 2g, 2g + 1 (one byte per code) of an 8-bit record
  const int kword = KB == 8 ? 2 * g : KB == 4 ? g : (g >= 2 ? 1 : 0);
  const int kshift = KB == 3 ? 24 * g - 32 * kword : 0;
  // token (within the tile) whose K norm scales accumulator cc in this lane
  auto ktok = [&](int cc) { return 16 * (cc * S + (4 * g) / GP) + row; };

  // tiles are dealt round-robin: workgroup x takes tiles x, x + W, x + 2W, ... (W workgroups per
  // KV head), so the workgroups in flight stream one contiguous stretch of the cache together
  const int64_t t_begin = (int64_t)blockIdx.x * kTile;
  const int64_t t_step = (int64_t)a.wg_per_head * kTile;

  using Regs = TileRegs<NBW, KB, VB, NC>;
  // Loads address a tile through uniform base pointers plus 32-bit per-lane offsets; the token of
  // an offset is clamped to the last token of the head (only the final tile has tokens past it).
  constexpr uint32_t KREC = NB * 4 * KB, VREC = NB * 4 * VB;  // bytes per token
  auto load = [&](Regs& r, int64_t tb) {
    const int64_t rem = T - 1 - tb;
    const uint32_t last = rem < kTile ? (uint32_t)rem : (uint32_t)(kTile - 1);
    const uint8_t* kt = kbase + tb * KREC;
    const uint8_t* vt8 = vbase + tb * VREC;
    const uint16_t* knt = knb + tb * NB;
    const uint16_t* vnt = vnb + tb * NB;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint32_t t = min((uint32_t)(16 * st + row), last);
#pragma unroll
      for (int bl = 0; bl < NBW; ++bl) {
        const uint32_t off = t * KREC + (uint32_t)((b0 + bl) * 4 * KB + 4 * kword);
        if constexpr (KB == 4) {
          r.kw[bl][st][0] = *reinterpret_cast<const uint32_t*>(kt + off);
          r.kw[bl][st][1] = 0u;
        } else {
          const uint2 w = *reinterpret_cast<const uint2*>(kt + off);
          r.kw[bl][st][0] = w.x;  // raw words: nothing computed from a load before its use
          r.kw[bl][st][1] = w.y;
        }
      }
    }
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const uint32_t t = min((uint32_t)ktok(cc), last);
      r.kn[cc] = NBW == 2 ? *reinterpret_cast<const uint32_t*>(knt + t * NB + b0) : (uint32_t)knt[t * NB + b0];
    }
    // V: in half hh, lane l holds token 32 hh + l % 32 and block b0 + l / 32 (head_dim 128: block b0,
    // whose coordinates lanes l and l + 32 split)
    const uint32_t vblk = (uint32_t)(b0 + (NBW == 2 ? (lane >> 5) : 0));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t t = min((uint32_t)(32 * hh + (lane & 31)), last);
      const uint8_t* rp = vt8 + t * VREC + vblk * (4 * VB);
      if constexpr (VB == 4) {  // 16-byte records
        const uint4 w = *reinterpret_cast<const uint4*>(rp);
        r.vw[hh][0] = w.x;
        r.vw[hh][1] = w.y;
        r.vw[hh][2] = w.z;
        r.vw[hh][3] = w.w;
      } else {
#pragma unroll
        for (int q = 0; q < VB; ++q) r.vw[hh][q] = reinterpret_cast<const uint32_t*>(rp)[q];
      }
      r.vn[hh] = (uint32_t)vnt[t * NB + vblk];
    }
  };

  // the first tile's loads go out before the tables and the query are set up, hiding their latency
  Regs rs[2];
  if (t_begin < T) load(rs[0], t_begin);

  // Set-up reads from global memory in one round trip: the levels (staged in the score-exchange
  // area, which the first tile's exchange is the first to use) and this thread's EPT consecutive
  // query elements, all of one row and one 32-block.
  constexpr int EPT = GP * HD / 256;  // query elements per thread (2 .. 16)
  constexpr int TPB = 32 / EPT;       // threads per 32-block, consecutive lanes of one wave
  static_assert(GP * HD % 256 == 0 && EPT >= 2 && EPT <= 32, "query staging splits evenly");
  float* lv = &xs[0][0][0];
  static_assert(sizeof(xs) >= sizeof(float) * (KL + VL), "levels fit the exchange area");
  for (int x = tid; x < KL; x += 256) lv[x] = a.klevel[x];
  if (tid < VL) lv[KL + tid] = a.vlevel[tid];
  const int qe0 = tid * EPT, qr = qe0 / HD, qd0 = qe0 % HD;
  float qv[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) qv[k] = 0.0f;
  if (qr < grows) {
    const int64_t rr = row0 + qr, i = rr / G;  // query token and head of the row
    const int64_t off = (i * a.n_q_heads + (int64_t)kvh * G + rr % G) * HD + qd0;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      qv[k] = a.q_f32 ? static_cast<const float*>(a.q)[off + k] : __half2float(static_cast<const __half*>(a.q)[off + k]);
  }

  // rotated query blocks qhat_b = H D_K q_b / sqrt(32) of the group's rows (rows past the live
  // ones zero): the sign flips, then the butterflies over coordinate bits from the lowest up, the
  // first log2 EPT inside the thread and the rest between the TPB threads of the block (the same
  // additions in the same order as a textbook FWHT); staged in fp32 over the V tile area
#pragma unroll
  for (int k = 0; k < EPT; ++k) qv[k] = ((a.kdbits >> ((qd0 + k) & 31)) & 1u) ? -qv[k] : qv[k];
#pragma unroll
  for (int hb = 1; hb < EPT; hb <<= 1) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      if (!(k & hb)) {
        const float x = qv[k], y = qv[k | hb];
        qv[k] = x + y;
        qv[k | hb] = x - y;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < TPB; m <<= 1) {
    const bool upper = (lane & m) != 0;  // this thread holds the coordinates with the bit set
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const float o = __shfl_xor(qv[k], m);
      qv[k] = upper ? o - qv[k] : qv[k] + o;
    }
  }
  float* qf = reinterpret_cast<float*>(&vt[0][0]);
  static_assert(sizeof(vt) >= sizeof(float) * GP * HD, "query staging fits the V tiles");
  if constexpr (EPT == 2) {
    *reinterpret_cast<float2*>(qf + qe0) = make_float2(qv[0], qv[1]);
  } else {
#pragma unroll
    for (int k = 0; k < EPT; k += 4)
      *reinterpret_cast<float4*>(qf + qe0 + k) = make_float4(qv[k], qv[k + 1], qv[k + 2], qv[k + 3]);
  }
  __syncthreads();  // levels and the rotated query are in LDS

  if constexpr (K8) {
    for (int x = tid; x < KL * CK; x += 256) {  // code -> (fp16 hi part, fp16 lo part)
      const float c = lv[x / CK];
      const _Float16 h = (_Float16)c;
      kth[x] = pack_h2(h, (_Float16)(c - (float)h));
    }
  } else {
    for (int x = tid; x < KL * KL * CK; x += 256) {
      const int e = x / CK;
      const float ca = lv[e & (KL - 1)], cb = lv[e >> KB];
      const _Float16 ha = (_Float16)ca, hb = (_Float16)cb;
      kth[x] = pack_h2(ha, hb);
      ktl[x] = pack_h2((_Float16)(ca - (float)ha), (_Float16)(cb - (float)hb));
    }
  }
  for (int x = tid; x < VL * VL * CV; x += 256) {
    const int e = x / CV;
    vtab[x] = pack_h2((_Float16)lv[KL + (e & (VL - 1))], (_Float16)lv[KL + (e >> VB)]);
  }

  // query operands of this lane: row `row` of the A operand is head row % GP (every row live, so
  // each subtile's product holds its scores in all 16 rows; a lane keeps the one of its own slot)
  v8h qh8[NBW], ql8[NBW];
#pragma unroll
  for (int bl = 0; bl < NBW; ++bl) {
    const int b = NBW * wave + bl;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = qf[(row % GP) * HD + 32 * b + 8 * g + j] * 0.17677669529663688f;  // 1/sqrt(32)
      const _Float16 h = (_Float16)v, l = (_Float16)(v - (float)h);
      qh8[bl][j] = h;
      ql8[bl][j] = l;
    }
  }
  const int slot = (4 * g) / GP;  // the subtile of a stack whose scores this lane's registers hold
  __syncthreads();  // query staging is overwritten by the V tiles below

  // last token each register's row may see: all tokens, or with a causal mask the row's query
  // position n_tokens - n_q + i (register i of this lane holds row (4g + i) % GP of the group)
  int64_t lim[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t rr = row0 + (4 * g + i) % GP;
    lim[i] = a.causal && rr < a.rows ? T - a.n_q + rr / G : T - 1;
  }
  const int64_t all_live = T - (a.causal ? a.n_q : 1);  // last token every row sees
  float m_run[4], lsum[4];
  v4f acc[NBW][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = kNoRef;
    lsum[i] = 0.0f;
  }
#pragma unroll
  for (int bl = 0; bl < NBW; ++bl) acc[bl][0] = acc[bl][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  _Float16* vtile = vt[wave];
  _Float16* ptile = pt[wave];
  int parity = 0;
  // ---- value records of half hh -> V tile rows 0..31 (norm folded in, chunks swizzled): lane l
  // expands its (token, block) record: a whole block (head_dim 256; chunks 2 (l / 32), +1) or half a
  // block (head_dim 128; lanes l and l + 32 take coordinates 0..15 and 16..31, chunk l / 32)
  auto write_v = [&](const Regs& cur, int hh) {
    constexpr int NP = NBW == 2 ? 16 : 8;  // code pairs this lane expands
    const int tl = lane & 31, up = lane >> 5;
    uint32_t win[VB];  // this lane's codes from bit 0
    if constexpr (NBW == 2) {
#pragma unroll
      for (int k = 0; k < VB; ++k) win[k] = cur.vw[hh][k];
    } else {
      constexpr int WO = (16 * VB) / 32, SH = (16 * VB) % 32;  // codes 16.. start at word WO, bit SH
#pragma unroll
      for (int k = 0; k < VB; ++k) {
        const uint32_t lo = k + WO < VB ? cur.vw[hh][k + WO] : 0u;
        const uint32_t hi = k + WO + 1 < VB ? cur.vw[hh][k + WO + 1] : 0u;
        const uint32_t sw = SH ? __builtin_amdgcn_alignbit(hi, lo, SH) : lo;
        win[k] = up ? sw : cur.vw[hh][k];
      }
    }
    const _Float16 nv = __builtin_bit_cast(_Float16, (uint16_t)cur.vn[hh]);
    const v2h nv2 = {nv, nv};
    uint32_t o[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
      const int pos = 2 * VB * pp, wi = pos >> 5, sh = pos & 31;
      const uint32_t w = sh + 2 * VB <= 32 ? win[wi] : __builtin_amdgcn_alignbit(win[wi + 1], win[wi], sh);
      const int s2 = sh + 2 * VB <= 32 ? sh : 0;
      const v2h c = __builtin_bit_cast(v2h, lut_word(vtab, w, s2, 2 * VB, LGCV, voff));
      o[pp] = __builtin_bit_cast(uint32_t, c * nv2);
    }
#pragma unroll
    for (int ch = 0; ch < NP / 8; ++ch) {
      const int c = NBW == 2 ? 2 * up + ch : up;
      *reinterpret_cast<uint4*>(vtile + vslot(tl, c, 0)) = make_uint4(o[8 * ch], o[8 * ch + 1], o[8 * ch + 2], o[8 * ch + 3]);
      *reinterpret_cast<uint4*>(vtile + vslot(tl, c, 1)) =
          make_uint4(o[8 * ch + 4], o[8 * ch + 5], o[8 * ch + 6], o[8 * ch + 7]);
    }
  };

  auto tile = [&](const Regs& cur, int64_t tb) {
    write_v(cur, 0);

    // ---- key side: partial scores over the owned blocks
    float s[NC][4];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[cc][i] = 0.0f;
    }
#pragma unroll
    for (int bl = 0; bl < NBW; ++bl) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        v4f cs[S];
#pragma unroll
        for (int sv = 0; sv < S; ++sv) {
          const int st = cc * S + sv;
          cs[sv] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
          uint32_t bh[4], bo[4];
          if constexpr (K8) {
            // two one-code lookups per pair; byte permutes gather the two hi and the two lo halves
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              const uint32_t w = cur.kw[bl][st][pp >> 1];
              const uint32_t e0 = lut_word(kth, w, 16 * (pp & 1), 8, LGCK, koff);
              const uint32_t e1 = lut_word(kth, w, 16 * (pp & 1) + 8, 8, LGCK, koff);
              bh[pp] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);
              bo[pp] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);
            }
          } else {
            const uint32_t win =
                KB == 4 ? cur.kw[bl][st][0]
                        : (uint32_t)((((uint64_t)cur.kw[bl][st][1] << 32) | cur.kw[bl][st][0]) >> kshift);
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              bh[pp] = lut_word(kth, win, 2 * KB * pp, 2 * KB, LGCK, koff);
              bo[pp] = lut_word(ktl, win, 2 * KB * pp, 2 * KB, LGCK, koff);
            }
          }
          const v8h bhi = __builtin_bit_cast(v8h, make_uint4(bh[0], bh[1], bh[2], bh[3]));
          const v8h blo = __builtin_bit_cast(v8h, make_uint4(bo[0], bo[1], bo[2], bo[3]));
          const v8h ah = qh8[bl], al = ql8[bl];
          cs[sv] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bhi, cs[sv], 0, 0, 0);
          cs[sv] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bhi, cs[sv], 0, 0, 0);
          cs[sv] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, blo, cs[sv], 0, 0, 0);
        }
        v4f c = cs[0];
#pragma unroll
        for (int sv = 1; sv < S; ++sv) {
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] = slot == sv ? cs[sv][i] : c[i];
        }
        const float nk = __half2float(__ushort_as_half((uint16_t)(cur.kn[cc] >> (16 * bl))));
#pragma unroll
        for (int i = 0; i < 4; ++i) s[cc][i] = __builtin_fmaf(nk, c[i], s[cc][i]);
      }
    }

    // ---- sum the waves' partial scores
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      *reinterpret_cast<float4*>(&xs[parity % NXS][lane][(wave * NC + cc) * 4]) =
          make_float4(s[cc][0], s[cc][1], s[cc][2], s[cc][3]);
    lds_barrier();
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int64_t tok = tb + ktok(cc);
      float4 v = *reinterpret_cast<const float4*>(&xs[parity % NXS][lane][cc * 4]);
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const float4 u = *reinterpret_cast<const float4*>(&xs[parity % NXS][lane][(w * NC + cc) * 4]);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      if (tb + kTile - 1 <= all_live) {  // every row sees the whole tile: no per-row test
        s[cc][0] = v.x * a.kscale;
        s[cc][1] = v.y * a.kscale;
        s[cc][2] = v.z * a.kscale;
        s[cc][3] = v.w * a.kscale;
      } else {
        s[cc][0] = tok <= lim[0] ? v.x * a.kscale : -INFINITY;
        s[cc][1] = tok <= lim[1] ? v.y * a.kscale : -INFINITY;
        s[cc][2] = tok <= lim[2] ? v.z * a.kscale : -INFINITY;
        s[cc][3] = tok <= lim[3] ? v.w * a.kscale : -INFINITY;
      }
    }
    if constexpr (NXS == 1) lds_barrier();  // one exchange buffer: every wave has read it before the next tile's writes

    // ---- online softmax; register i of this lane belongs to head (4g + i) % GP.  The reference
    // m_run of a head only moves when some score of the tile exceeds it by more than kSlack (always
    // on the first tile): the weights exp(s - m_run) then stay below e^kSlack, well inside fp16, and
    // most tiles skip the cross-lane maximum and the rescaling.  lsum holds this lane's share of the
    // weight sum; the lanes of a head are summed once, after the last tile.
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) grow |= s[cc][i] > m_run[i] + kSlack;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float mt = s[0][i];
#pragma unroll
        for (int cc = 1; cc < NC; ++cc) mt = fmaxf(mt, s[cc][i]);
        mt = head_reduce<S, true>(mt);
        const float m_new = fmaxf(m_run[i], mt);  // >= kNoRef, so alpha below is never NaN
        const float alpha = __expf(m_run[i] - m_new);
        lsum[i] *= alpha;
        m_run[i] = m_new;
#pragma unroll
        for (int bl = 0; bl < NBW; ++bl) {
          acc[bl][0][i] *= alpha;
          acc[bl][1][i] *= alpha;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i, h = r % GP, sub = r / GP;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const float p = __expf(s[cc][i] - m_run[i]);
        lsum[i] += p;
        ptile[h * kTile + 16 * (cc * S + sub) + row] = (_Float16)p;
      }
    }
    wave_sync();

    // ---- value side: acc[head][coordinate] += p[head][token] * (nV c)[token][coordinate], one 32-token
    // half of the tile at a time (the V tile holds one half; the second is expanded once the first is read)
#pragma unroll
    for (int half = 0; half < kTile / VT; ++half) {
      if (half > 0) {
        wave_sync();  // the previous half's transposing reads are issued before its rows are overwritten
        write_v(cur, half);
        wave_sync();
      }
      const v8h z = {0, 0, 0, 0, 0, 0, 0, 0};
      const v8h av = row < grows ? *reinterpret_cast<const v8h*>(ptile + (row % GP) * kTile + VT * half + 8 * g) : z;
      const int t1 = 8 * g + (row >> 2), t2 = t1 + 4;
#pragma unroll
      for (int bl = 0; bl < NBW; ++bl) {
#pragma unroll
        for (int nh = 0; nh < 2; ++nh) {
          const int c = 2 * bl + nh;
          lds_short* base = (lds_short*)vtile;
          const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4s*)(base + vslot(t1, c, (row & 3) >> 1) + 4 * (row & 1)));
          const v4s r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4s*)(base + vslot(t2, c, (row & 3) >> 1) + 4 * (row & 1)));
          const v4h h1 = __builtin_bit_cast(v4h, r1), h2 = __builtin_bit_cast(v4h, r2);
          const v8h bv = {h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
          acc[bl][nh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[bl][nh], 0, 0, 0);
        }
      }
    }
    wave_sync();
    parity ^= 1;
  };
  // Tiles go in pairs with no exit between them: a workgroup with an odd number of tiles ends on a
  // tile past the end, whose tokens are all masked.  The prefetch is unconditional (a load aimed
  // past the end reloads an earlier tile), so the same loads are in flight on every path into a
  // tile and the wait for the current register set leaves the next one pending.
  for (int64_t tb = t_begin; tb < T; tb += 2 * t_step) {
    const int64_t t1 = tb + t_step, t2 = tb + 2 * t_step;
    load(rs[1], t1 < T ? t1 : tb);
    tile(rs[0], tb);
    load(rs[0], t2 < T ? t2 : tb);
    tile(rs[1], t1);
  }

  // ---- partial of this workgroup: part[kvh][rg][wg][row][HD coordinates, reference, sum]
  float* pbase = a.part + ((int64_t)blockIdx.y * a.wg_per_head + blockIdx.x) * a.grp * (HD + 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;  // accumulator row = row of the group
    if (h >= grows) continue;
#pragma unroll
    for (int bl = 0; bl < NBW; ++bl) {
      pbase[h * (HD + 2) + 32 * (b0 + bl) + row] = acc[bl][0][i];
      pbase[h * (HD + 2) + 32 * (b0 + bl) + 16 + row] = acc[bl][1][i];
    }
  }
  // running max / sum of head h are held in register h % 4 of the lanes whose row group maps to h
#pragma unroll
  for (int i = 0; i < 4; ++i) lsum[i] = head_reduce<S, false>(lsum[i]);
  if (wave == 0 && row == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * g + i, h = r % GP;
      if (r < GP && h < grows) {
        pbase[h * (HD + 2) + HD] = m_run[i];
        pbase[h * (HD + 2) + HD + 1] = lsum[i];
      }
    }
  }
}

// Merge: one workgroup per (output row, 32-block); kMergeLanes x 32 threads (partial lane, coordinate).
// Output row o = (query token i, query head h) reads row i * group + h % group of KV head h / group.
__global__ __launch_bounds__(256) void attn_merge(AttnArgs a) {
  const int64_t o = blockIdx.x;
  const int b = blockIdx.y, HD = a.head_dim, G = a.group;
  const int64_t i = o / a.n_q_heads;
  const int h = (int)(o % a.n_q_heads), kvh = h / G;
  const int64_t rr = i * G + h % G, rg = rr / a.grp, r = rr % a.grp;
  const int tid = threadIdx.x, pl = tid >> 5, dl = tid & 31;
  const int n_part = a.wg_per_head;
  const int64_t stride = (int64_t)a.grp * (HD + 2);
  const float* base = a.part + ((int64_t)kvh * a.n_rg + rg) * n_part * stride + r * (HD + 2);
  __shared__ float red[kMergeLanes][34];
  // one pass over this lane's partials with a running reference (the partials' own references
  // differ; a larger one rescales what was summed so far)
  float m = -INFINITY, acc = 0.0f, l = 0.0f;
#pragma unroll 16
  for (int p = pl; p < n_part; p += kMergeLanes) {
    const float* pb = base + p * stride;
    const float mp = pb[HD], lp = pb[HD + 1], xp = pb[32 * b + dl];
    // branch-free, so the loads of the unrolled iterations go out together (every partial has a
    // finite reference; a row with no live token in a workgroup has reference kNoRef and sum 0)
    const float m_new = fmaxf(m, mp);
    const float f_old = m == -INFINITY ? 0.0f : __expf(m - m_new), f_new = __expf(mp - m_new);
    acc = __builtin_fmaf(xp, f_new, acc * f_old);
    l = __builtin_fmaf(lp, f_new, l * f_old);
    m = m_new;
  }
  red[pl][dl] = acc;
  if (dl == 0) {
    red[pl][32] = l;
    red[pl][33] = m;
  }
  __syncthreads();
  if (pl == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kMergeLanes; ++q) M = fmaxf(M, red[q][33]);
    float s = 0.0f, ls = 0.0f;
#pragma unroll
    for (int q = 0; q < kMergeLanes; ++q) {
      const float mq = red[q][33];
      const float f = mq == -INFINITY ? 0.0f : __expf(mq - M);
      s = __builtin_fmaf(red[q][dl], f, s);
      ls = __builtin_fmaf(red[q][32], f, ls);
    }
    // out = D_V * H_unnorm(acc) / (32 * l): butterflies across the 32 lanes of the first wave
    float v = s;
#pragma unroll
    for (int hb = 1; hb < 32; hb <<= 1) {
      const float o = __shfl_xor(v, hb);
      v = (dl & hb) ? o - v : v + o;
    }
    v = v / (32.0f * ls);
    if ((a.vdbits >> dl) & 1u) v = -v;
    a.out[o * HD + 32 * b + dl] = v;
  }
}

template <int NB, int KB, int VB>
hipError_t launch_nb(const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.wg_per_head, (unsigned)(a.n_kv_heads * a.n_rg));
  if (a.grp == attn_prefill_rows()) {
    hipError_t e = launch_prefill(KB, VB, a, s);
    if (e != hipSuccess) return e;
  } else if (a.grp <= 4)
    hipLaunchKernelGGL((attn_kernel<NB, KB, VB, 4>), grid, dim3(256), 0, s, a);
  else if (a.grp <= 8)
    hipLaunchKernelGGL((attn_kernel<NB, KB, VB, 8>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_kernel<NB, KB, VB, 16>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge, dim3((unsigned)(a.n_q * a.n_q_heads), (unsigned)(a.head_dim / 32)), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

template <int KB, int VB>
hipError_t launch_bits(const AttnArgs& a, hipStream_t s) {
  return a.head_dim == 128 ? launch_nb<4, KB, VB>(a, s) : launch_nb<8, KB, VB>(a, s);
}

}  // namespace

// Token range per workgroup: a multiple of two 64-token tiles (the decode kernel walks its tiles in
// pairs) that spreads the cache over about 512 workgroups (two per compute unit; 256 for the 8-wave
// prefill workgroups, one per compute unit), 128 .. 8192 tokens; `columns` = KV heads x row groups,
// the workgroup columns that each walk it, `grp` = rows per group.  (Groups of up to 4 rows would fit
// three workgroups per compute unit, but spreading them over 768 measured slower: 62 against 60 us
// for the 131072-token decode; the kernel is built for two, with the registers that leaves.)
#ifndef TQ_ATTN_WG_TARGET4
#define TQ_ATTN_WG_TARGET4 512
#endif
int64_t attn_tokens_per_wg(int64_t columns, int64_t n_tokens, int64_t grp) {
  const int64_t target = grp > 16 ? 256 : grp <= 4 ? TQ_ATTN_WG_TARGET4 : 512;
  int64_t per = (n_tokens * columns + target - 1) / target;
  per = (per + 2 * kTile - 1) / (2 * kTile) * (2 * kTile);
  if (per < 2 * kTile) per = 2 * kTile;
  if (per > 8192) per = 8192;
  return per;
}

// Scratch of tq_decode_attn_noalloc: the softmax partials of a decode call live in this array instead
// of a caller workspace.  Every device the library runs on holds its own copy, at its own address, for
// the life of the process; in host code `scratch` names a host-side stand-in, so kernels only ever get
// the device address resolved here.  No kernel needs it cleared: each workgroup writes its whole
// partial before the merge reads it.
static __device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

hipError_t attn_scratch(void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {  // first call on this device (concurrent first calls resolve the same address)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_attn(int kbits, int vbits, const AttnArgs& a, hipStream_t s) {
  if (kbits == 3 && vbits == 3) return launch_bits<3, 3>(a, s);
  if (kbits == 4 && vbits == 4) return launch_bits<4, 4>(a, s);
  if (kbits == 3 && vbits == 4) return launch_bits<3, 4>(a, s);
  if (kbits == 4 && vbits == 3) return launch_bits<4, 3>(a, s);
  if (kbits == 8 && vbits == 3) return launch_bits<8, 3>(a, s);
  return launch_bits<8, 4>(a, s);
}

}  // namespace tq
