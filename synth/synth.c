/*
 * Seeded synthetic inputs shared by the HIP path's tests/benchmark and by the
 * CPU oracle.  It holds none of the quantizer's arithmetic: only a
 * counter-based uniform generator, the Box-Muller transform, the KV-cache
 * shaping (per-channel log-normal scales, outlier channels) and an exact
 * float64 -> binary16 rounding.
 *
 * Uniforms: splitmix64's output function (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) applied to a
 * counter.  For a (seed, stream) pair the key is
 *     key = fin(fin(seed) ^ ((stream + 1) * G2))
 * and the 64-bit draw at index i is
 *     r_i = fin(key + (i + 1) * G)
 * with G the golden-ratio increment of splitmix64 and fin its finalizer.
 * U_i = (r_i >> 11) * 2^-53 lies in [0, 1).
 *
 * Normals: Box-Muller (1958) on the pair p = i / 2,
 *     R = sqrt(-2 ln(1 - U_{2p})),  theta = 2 pi U_{2p+1},
 *     Z_{2p} = R cos(theta),  Z_{2p+1} = R sin(theta).
 *
 * Every function is a pure function of its arguments: the value at a given
 * index does not depend on how the range is split into calls or threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define G1 0x9E3779B97F4A7C15ull
#define G2 0xD1B54A32D192ED03ull

static inline uint64_t fin(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return fin(fin(seed) ^ ((stream + 1ull) * G2));
}

static inline double unif(uint64_t key, uint64_t i) {
  return (double)(fin(key + (i + 1ull) * G1) >> 11) * 0x1.0p-53;
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = unif(key, 2 * p), u2 = unif(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(1.0 - u1));
  double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

/* Round a float64 to binary16, round-to-nearest-even, IEEE overflow to inf. */
static uint16_t f64_to_f16(double x) {
  uint64_t b;
  memcpy(&b, &x, 8);
  uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  uint64_t mag = b & 0x7FFFFFFFFFFFFFFFull;
  if (mag >= 0x7FF0000000000000ull)
    return sign | (mag > 0x7FF0000000000000ull ? 0x7E00u : 0x7C00u);
  int e = (int)(mag >> 52) - 1023;
  if (e > 15) return sign | 0x7C00u;
  if (e < -25) return sign;
  uint64_t m = (mag & ((1ull << 52) - 1)) | (1ull << 52);
  int shift = (e >= -14) ? 42 : 28 - e;
  uint64_t q = m >> shift;
  uint64_t rem = m & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q++;
  if (e >= -14) {
    uint32_t he = (uint32_t)(e + 15);
    if (q == (1u << 11)) { q >>= 1; he++; }
    if (he >= 31) return sign | 0x7C00u;
    return (uint16_t)(sign | (he << 10) | (q & 0x3FFu));
  }
  return (uint16_t)(sign | q);
}

void synth_uniform(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, double* out) {
  uint64_t key = stream_key(seed, stream);
  for (uint64_t k = 0; k < n; ++k) out[k] = unif(key, start + k);
}

void synth_normal(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n, double* out) {
  uint64_t key = stream_key(seed, stream);
  for (uint64_t k = 0; k < n; ++k) out[k] = normal_at(key, start + k);
}

void synth_f64_to_f16(const double* in, uint64_t n, uint16_t* out) {
  for (uint64_t k = 0; k < n; ++k) out[k] = f64_to_f16(in[k]);
}

/* ---- KV-cache shaped tensors -------------------------------------------
 * One tensor of shape [layers][heads][tokens][head_dim] holding either the
 * K (kv = 0) or the V (kv = 1) half of a cache laid out conceptually as
 * [layer][head][K|V][token][head_dim].
 *   entry  = Z * s_c            (Z from stream `data_stream`, index = flat
 *                                position in the conceptual K|V layout)
 *   s_c    = exp(sigma * Z')    (stream 4, one per (layer, head, kv, channel))
 *            * outlier_mult     for the n_outliers channels chosen per
 *                                (layer, head, kv) from stream 5
 * The result is rounded to binary16 (out16) or returned as float64 (out64).
 */
typedef struct {
  uint64_t seed;
  int layers, heads, kv;
  int64_t tokens;
  int head_dim;
  double sigma;
  int n_outliers;
  double outlier_mult;
  int data_stream;
  uint16_t* out16;
  double* out64;
  int64_t slab_begin, slab_end; /* range of (layer, head) slabs */
} kv_job;

static void channel_scales(const kv_job* j, int64_t slab, double* scale) {
  uint64_t kscale = stream_key(j->seed, 4), kout = stream_key(j->seed, 5);
  int64_t base = (slab * 2 + j->kv) * (int64_t)j->head_dim;
  for (int c = 0; c < j->head_dim; ++c) scale[c] = exp(j->sigma * normal_at(kscale, (uint64_t)(base + c)));
  /* outlier channels: distinct, uniform over the remaining channels */
  int chosen[16];
  int n_ch = j->n_outliers < 16 ? j->n_outliers : 16;
  for (int o = 0; o < n_ch; ++o) {
    double u = unif(kout, (uint64_t)((slab * 2 + j->kv) * 16 + o));
    int pick = (int)(u * (double)(j->head_dim - o));
    /* map pick-th free channel to a channel index (skip already chosen ones, in increasing order) */
    int c = -1, free_seen = -1;
    while (free_seen < pick) {
      ++c;
      int taken = 0;
      for (int q = 0; q < o; ++q) taken |= (chosen[q] == c);
      if (!taken) ++free_seen;
    }
    chosen[o] = c;
    scale[c] *= j->outlier_mult;
  }
}

static void* kv_worker(void* arg) {
  const kv_job* j = (const kv_job*)arg;
  uint64_t kdata = stream_key(j->seed, (uint64_t)j->data_stream);
  double scale[1024];
  for (int64_t slab = j->slab_begin; slab < j->slab_end; ++slab) {
    channel_scales(j, slab, scale);
    int64_t src0 = (slab * 2 + j->kv) * j->tokens * j->head_dim; /* conceptual K|V index */
    int64_t dst0 = slab * j->tokens * j->head_dim;
    int64_t n = j->tokens * j->head_dim;
    for (int64_t k = 0; k < n; ++k) {
      double v = normal_at(kdata, (uint64_t)(src0 + k)) * scale[k % j->head_dim];
      if (j->out16) j->out16[dst0 + k] = f64_to_f16(v);
      else j->out64[dst0 + k] = v;
    }
  }
  return 0;
}

/* Returns 0 on success, -1 on bad arguments. */
int synth_kv(uint64_t seed, int layers, int heads, int kv, int64_t tokens, int head_dim, double sigma,
             int n_outliers, double outlier_mult, int data_stream, uint16_t* out16, double* out64, int nthreads) {
  if (layers <= 0 || heads <= 0 || tokens <= 0 || head_dim <= 0 || head_dim > 1024 || (kv != 0 && kv != 1) ||
      n_outliers < 0 || n_outliers > 16 || n_outliers > head_dim || (!out16 && !out64))
    return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  int64_t slabs = (int64_t)layers * heads;
  kv_job jobs[256];
  pthread_t th[256];
  int used = 0;
  /* split slabs when there are enough; otherwise one thread per slab range */
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = slabs * t / nthreads, e = slabs * (t + 1) / nthreads;
    if (b == e) continue;
    kv_job jb = {seed, layers, heads, kv, tokens, head_dim, sigma, n_outliers, outlier_mult, data_stream,
                 out16, out64, b, e};
    jobs[used] = jb;
    ++used;
  }
  for (int t = 0; t < used; ++t) pthread_create(&th[t], 0, kv_worker, &jobs[t]);
  for (int t = 0; t < used; ++t) pthread_join(th[t], 0);
  return 0;
}

/* Parallel fill of N(0,1) rounded to binary16 or binary32 (for query / fp32 inputs). */
typedef struct {
  uint64_t key;
  uint64_t begin, end;
  uint16_t* out16;
  float* out32;
} nrm_job;

static void* nrm_worker(void* arg) {
  const nrm_job* j = (const nrm_job*)arg;
  for (uint64_t i = j->begin; i < j->end; ++i) {
    double v = normal_at(j->key, i);
    if (j->out16) j->out16[i] = f64_to_f16(v);
    else j->out32[i] = (float)v; /* C conversion double->float rounds to nearest even */
  }
  return 0;
}

void synth_normal_rounded(uint64_t seed, uint64_t stream, uint64_t n, uint16_t* out16, float* out32, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  nrm_job jobs[256];
  pthread_t th[256];
  uint64_t key = stream_key(seed, stream);
  for (int t = 0; t < nthreads; ++t) {
    nrm_job jb = {key, n * (uint64_t)t / (uint64_t)nthreads, n * (uint64_t)(t + 1) / (uint64_t)nthreads, out16, out32};
    jobs[t] = jb;
  }
  for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], 0, nrm_worker, &jobs[t]);
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], 0);
}
