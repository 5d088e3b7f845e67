// Internal declarations shared by the host dispatcher and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "tq.h"

namespace tq {

constexpr int kMaxDt = 256;
constexpr int kBlock = 256;  // threads per workgroup for the streaming kernels

// Arguments of the encode kernel (one 32-coordinate group per lane).
struct EncodeArgs {
  const void* x;
  int64_t ld_x;            // row stride in elements
  uint8_t* codes;
  void* norms;
  int64_t n_groups;        // rows * head_dim / 32
  int32_t groups_per_row;  // head_dim / 32
  int32_t contiguous;      // ld_x == head_dim
  uint32_t dbits[8];       // D: bit c%32 of word c/32 set when D_c = -1
  float thr[128];          // positive N(0,1) cell edges t_1 < t_2 < ... (the edge at 0 is implicit), then +inf
  float bin_scale;         // 4 and 8 bits: bucket-table bins per unit of |u| (N(0,1) scale)
  int32_t n_bins;          // 4 and 8 bits: bucket-table entries in use (<= kLutEntries4, kMaxBins8)
};

constexpr int kLutEntries4 = 256;  // 4-bit bucket table: every index of a saturating byte conversion
constexpr int kMaxBins8 = 1024;

// Arguments of the decode kernel.
struct DecodeArgs {
  const uint8_t* codes;
  const void* norms;
  void* y;
  int64_t ld_y;
  int64_t n_groups;
  int32_t groups_per_row;
  int32_t contiguous;
  uint32_t dbits[8];
  float level[256];  // N(0,1) centroid of each stored code (sign-magnitude order)
  float inv_dt;      // 1 / dt
  float inv_sqrt_dt; // 1 / sqrt(dt)
};

// QJL arguments (dt == head_dim, one unit per row).
struct QjlEncodeArgs {
  const void* x;
  int64_t ld_x;
  uint8_t* codes;
  void* norms;
  uint8_t* qjl_bits;
  uint16_t* rnorm;
  int64_t n_units;
  const double* s_rot;  // S~ = S D H, [m][dt] float64
  uint32_t dbits[8];
  double thr[8];        // positive N(0,1) cell edges
  double level[16];     // N(0,1) centroid by stored code
  int32_t m;
};

struct QjlDecodeArgs {
  const uint8_t* codes;
  const void* norms;
  const uint8_t* qjl_bits;
  const uint16_t* rnorm;
  const float* s_rot;   // S~ [m][dt] float32
  void* y;
  int64_t ld_y;
  int64_t n_units;
  uint32_t dbits[8];
  float level[16];
  int32_t m;
  float qjl_scale;      // sqrt(dt) * sqrt(pi/2) / m
  float inv_dt;
  float inv_sqrt_dt;
};

// QJL scores (tq_qjl_scores): workspace-resident operands for the int8 MFMA kernel.
struct ScoreArgs {
  const void* q;
  int64_t ld_q;
  int64_t n_q, n_q_pad;      // queries, padded to a multiple of 32
  const uint8_t* codes;
  const void* norms;
  const uint8_t* qjl_bits;
  const uint16_t* rnorm;
  int64_t n_k, n_k_pad;      // keys, padded to the scores key tile
  int64_t q_chunk;           // queries per scores workgroup (a multiple of 32; set by the launcher)
  float* scores;
  int64_t ld_s;
  int8_t* qrec;              // [n_q_pad / 32] blocks of 32 queries x 2*(planes*kd+km) int8 limbs (per plane
                             // w_t qhat hi, lo; then p hi, lo), each block laid out as 1 KiB MFMA fragments
  float* qscale;             // [n_q_pad][2]: fixed-point scale of qhat / sqrt(dt), of p * sqrt(pi/2)/m
  const float* s_rot32;      // S~ [m][dt] float32
  uint32_t dbits[8];
  float plane_w[8];          // weight of each ternary plane (N(0,1) scale)
  int32_t dt, m, kd, km;     // kd, km: dt and m rounded up to 64
  int32_t q_f32;
  float inv_sqrt_dt, qjl_const;
};

// Attention over a block-32 K/V cache with fp16 norms (tq_decode_attn, tq_multi_attn).  The
// rows of a KV head are its (query token, query head) pairs, row = token * group + head in group;
// they are cut into row groups of at most 16, one workgroup column per (KV head, row group).
struct AttnArgs {
  const void* q;             // [n_q][n_q_heads][head_dim]
  int32_t q_f32;
  int32_t n_q_heads, n_kv_heads, group;  // group = n_q_heads / n_kv_heads
  int32_t head_dim;
  int64_t n_tokens;
  int64_t n_q;               // query tokens (1 for decode)
  int64_t rows;              // n_q * group rows per KV head
  int32_t grp;               // rows per row group: rows if rows <= 16, else the prefill kernel's 128
  int32_t n_rg;              // row groups per KV head
  int32_t causal;            // row of query token i sees tokens j <= n_tokens - n_q + i
  const uint8_t* k_codes;
  const uint16_t* k_norms;
  const uint8_t* v_codes;
  const uint16_t* v_norms;
  float* out;                // [n_q][n_q_heads][head_dim]
  float* part;               // [n_kv_heads][n_rg][wg_per_head][grp][head_dim + 2] partial (acc, ref, sum)
  int32_t wg_per_head;
  int64_t tokens_per_wg;
  uint32_t kdbits, vdbits;   // D_K, D_V of the 32-long blocks
  float klevel[256], vlevel[16];
  float kscale;              // softmax scale / sqrt(32): score = kscale * sum_b n_b <H D q_b, c_b>
};

// Compute units of the current device, cached per device (relaxed atomics: concurrent first calls
// store the same value).  Launch sizing only; 256 if the query fails.
inline int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  hipDeviceProp_t prop;
  int cus = 256;
  if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0) cus = prop.multiProcessorCount;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// launchers (return hipGetLastError() of the launch)
hipError_t launch_encode(const tq_config& cfg, const EncodeArgs& a, hipStream_t s);
hipError_t launch_decode(const tq_config& cfg, const DecodeArgs& a, bool nc, tq_dtype y_dtype, hipStream_t s);
hipError_t launch_qjl_encode(const tq_config& cfg, const QjlEncodeArgs& a, hipStream_t s);
hipError_t launch_qjl_decode(const tq_config& cfg, const QjlDecodeArgs& a, bool nc, tq_dtype y_dtype, hipStream_t s);
hipError_t launch_qjl_scores(const tq_config& cfg, const ScoreArgs& a, hipStream_t s);
int64_t scores_key_tile(int bits);
int64_t scores_query_block();
hipError_t launch_decode_attn(int kbits, int vbits, const AttnArgs& a, hipStream_t s);
// Device address of the library's static decode-attention scratch on the current device (resolved on
// the first call per device), kAttnScratchBytes long.
constexpr size_t kAttnScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
hipError_t attn_scratch(void** ptr);
int64_t attn_tokens_per_wg(int64_t columns, int64_t n_tokens, int64_t grp);
int attn_prefill_rows();  // rows per workgroup of the many-row (prefill) attention kernel
hipError_t launch_prefill(int kbits, int vbits, const AttnArgs& a, hipStream_t s);  // its main kernel (no merge)

}  // namespace tq
