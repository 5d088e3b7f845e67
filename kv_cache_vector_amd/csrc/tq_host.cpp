// Host side of libtq: codebook solver, QJL parameter preparation, argument
// validation and kernel dispatch for the C ABI declared in include/tq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace {

thread_local std::string g_last_error;

tq_status fail(tq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tq_status fail(tq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tq_status ok() {
  g_last_error.clear();
  return TQ_OK;
}

tq_status hip_fail(hipError_t e, const char* where) {
  return fail(TQ_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Lloyd-Max for N(0,1) ([Scratch] §2 step 3; [README]: solved once per bit
// width by numerical integration).  Jacobi iteration of the two optimality
// conditions (edges at midpoints, levels at conditional means) from a uniform
// grid on [-3, 3]; the Gaussian is log-concave so the fixed point is unique.
// ---------------------------------------------------------------------------
double std_pdf(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * 0.39894228040143267794; }

// P(a < X < b) computed from the tail on the far side of zero to avoid cancellation
double std_mass(double a, double b) {
  if (a >= 0.0) return 0.5 * (std::erfc(a * M_SQRT1_2) - std::erfc(b * M_SQRT1_2));
  if (b <= 0.0) return 0.5 * (std::erfc(-b * M_SQRT1_2) - std::erfc(-a * M_SQRT1_2));
  return 1.0 - 0.5 * std::erfc(-a * M_SQRT1_2) - 0.5 * std::erfc(b * M_SQRT1_2);
}

// Lloyd-Max for N(0,1) at many levels (5..8 bits).  Lloyd's iteration contracts
// ever more slowly as L grows, so the fixed point of the non-negative half is
// found by Newton's method on G_i(c) = c_i - E[X | e_i < X < e_{i+1}], with
// e_0 = 0, e_i = (c_{i-1} + c_i)/2 and e_h = +inf.  The Jacobian is
// tridiagonal: with m_i the conditional mean and P_i the cell mass,
//   dm_i/de_i = phi(e_i)(m_i - e_i)/P_i,  dm_i/de_{i+1} = phi(e_{i+1})(e_{i+1} - m_i)/P_i.
// Start: the high-resolution point density, proportional to phi^(1/3), i.e.
// edges at the quantiles of N(0, 3) (inverse normal CDF by bisection on erfc).
// Steps are halved while they would break the ordering or raise the residual.
bool solve_lloyd_max_newton(int bits, double* levels, double* edges, double* distortion) {
  const int h = 1 << (bits - 1), L = 2 * h;
  auto upper_tail = [](double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x * M_SQRT1_2); };
  auto inv_upper_tail = [&](double p) {  // x >= 0 with P(X > x) = p, p in (0, 1/2]
    double lo = 0.0, hi = 40.0;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      (upper_tail(mid) > p ? lo : hi) = mid;
    }
    return 0.5 * (lo + hi);
  };
  std::vector<double> c(h), e(h + 1), m(h), P(h), G(h), a(h), b(h), d(h), rhs(h), nc(h);
  auto edges_of = [&](const std::vector<double>& cc) {
    e[0] = 0.0;
    for (int i = 1; i < h; ++i) e[i] = 0.5 * (cc[i - 1] + cc[i]);
    e[h] = INFINITY;
  };
  auto residual = [&](const std::vector<double>& cc) {
    edges_of(cc);
    double worst = 0.0;
    for (int i = 0; i < h; ++i) {
      P[i] = upper_tail(e[i]) - upper_tail(e[i + 1]);
      m[i] = (std_pdf(e[i]) - std_pdf(e[i + 1])) / P[i];
      G[i] = cc[i] - m[i];
      worst = std::max(worst, std::fabs(G[i]));
    }
    return worst;
  };
  for (int i = 0; i <= h; ++i) e[i] = i == h ? INFINITY : std::sqrt(3.0) * inv_upper_tail(0.5 * (1.0 - (double)i / h));
  for (int i = 0; i < h; ++i) c[i] = (std_pdf(e[i]) - std_pdf(e[i + 1])) / (upper_tail(e[i]) - upper_tail(e[i + 1]));
  double res = residual(c);
  for (int it = 0; it < 100 && res > 1e-15; ++it) {
    // tridiagonal J: sub a[i] = dG_i/dc_{i-1}, diag d[i], super b[i] = dG_i/dc_{i+1}
    for (int i = 0; i < h; ++i) {
      const double dlo = i >= 1 ? std_pdf(e[i]) * (m[i] - e[i]) / P[i] : 0.0;
      const double dhi = i + 1 < h ? std_pdf(e[i + 1]) * (e[i + 1] - m[i]) / P[i] : 0.0;
      a[i] = -0.5 * dlo;
      b[i] = -0.5 * dhi;
      d[i] = 1.0 - 0.5 * dlo - 0.5 * dhi;
      rhs[i] = -G[i];
    }
    for (int i = 1; i < h; ++i) {  // Thomas algorithm
      const double w = a[i] / d[i - 1];
      d[i] -= w * b[i - 1];
      rhs[i] -= w * rhs[i - 1];
    }
    std::vector<double> delta(h);
    delta[h - 1] = rhs[h - 1] / d[h - 1];
    for (int i = h - 2; i >= 0; --i) delta[i] = (rhs[i] - b[i] * delta[i + 1]) / d[i];
    double step = 1.0, new_res = INFINITY;
    for (int tries = 0; tries < 60; ++tries, step *= 0.5) {
      bool ordered = true;
      for (int i = 0; i < h; ++i) {
        nc[i] = c[i] + step * delta[i];
        if (nc[i] <= (i ? nc[i - 1] : 0.0)) ordered = false;
      }
      if (!ordered) continue;
      new_res = residual(nc);
      if (new_res < res || new_res <= 1e-15) break;
    }
    if (!(new_res < INFINITY)) return false;
    const bool progress = new_res < res;
    c = nc;
    res = residual(c);
    if (!progress) break;  // at the rounding floor
  }
  if (!(res < 1e-12)) return false;
  edges_of(c);
  double sum = 0.0;
  for (int i = 0; i < h; ++i) {
    levels[h + i] = c[i];
    levels[h - 1 - i] = -c[i];
    sum += 2.0 * (upper_tail(e[i]) - upper_tail(e[i + 1])) * c[i] * c[i];
  }
  for (int k = 0; k + 1 < L; ++k) edges[k] = 0.5 * (levels[k] + levels[k + 1]);
  edges[h - 1] = 0.0;
  *distortion = 1.0 - sum;
  return true;
}

struct GaussCell {
  // mass and first moment of N(0,1) over (a, b)
  void operator()(double a, double b, double* m0, double* m1) const {
    *m0 = std_mass(a, b);
    *m1 = std_pdf(a) - std_pdf(b);
  }
};

// ---------------------------------------------------------------------------
// Exact marginal of a rotated unit vector ([Fork] "How it works": the
// codebook is solved for Beta((d-1)/2, (d-1)/2); [README], stage 1: the Gaussian
// is its large-d limit).  A coordinate T of a uniform unit vector in d
// dimensions has density proportional to (1 - t^2)^((d-3)/2) on [-1, 1].
// With t = sin(theta) the mass element becomes cos^(d-2)(theta) d theta, a
// smooth bell of width about 1/sqrt(d) with no end-point singularity, which
// composite 16-point Gauss-Legendre integrates to rounding.  Cells are given
// in the unit-variance scale u = sqrt(d) t; the first moment is returned in
// that scale too.  Masses are not normalised (the Lloyd step only needs
// ratios; the distortion divides by their sum).
// ---------------------------------------------------------------------------
struct GaussLegendre16 {
  double x[16], w[16];
  GaussLegendre16() {
    const int n = 16;
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));  // Newton on P_16 from the usual initial guess
      double dp = 1.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          double p2 = ((2 * k - 1) * z * p1 - (k - 1) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-17) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

struct SphereCell {
  int dim;
  void operator()(double a, double b, double* m0, double* m1) const {
    static const GaussLegendre16 gl;
    const double sd = std::sqrt((double)dim), n = dim - 2;
    // beyond |theta| = acos(exp(-745/n)) the integrand is below the smallest double
    const double lim = std::acos(std::exp(-745.0 / n));
    double lo = std::max(-lim, std::asin(std::max(-1.0, std::min(1.0, a / sd))));
    double hi = std::min(lim, std::asin(std::max(-1.0, std::min(1.0, b / sd))));
    double s0 = 0.0, s1 = 0.0;
    if (hi > lo) {
      const double h = 1.0 / std::sqrt(n);  // panel no wider than the bell
      const int panels = std::min(100000, std::max(1, (int)std::ceil((hi - lo) / h)));
      const double pw = (hi - lo) / panels;
      for (int p = 0; p < panels; ++p) {
        const double mid = lo + (p + 0.5) * pw;
        for (int k = 0; k < 16; ++k) {
          const double th = mid + 0.5 * pw * gl.x[k];
          const double sn = std::sin(th);
          const double f = 0.5 * pw * gl.w[k] * std::exp(0.5 * n * std::log1p(-sn * sn));  // cos^n, cos >= 0
          s0 += f;
          s1 += f * sn;
        }
      }
    }
    *m0 = s0;
    *m1 = sd * s1;
  }
};

// Jacobi iteration of Lloyd's two conditions for the symmetric law whose
// cell moments `cell` returns, starting from a uniform grid on [-r, r].
template <typename Cell>
void solve_lloyd_max(int bits, const Cell& cell, double r, double* levels, double* edges, double* distortion) {
  const int L = 1 << bits;
  std::vector<double> c(L), t(L - 1), nc(L);
  for (int i = 0; i < L; ++i) c[i] = -r + 2.0 * r * (i + 0.5) / L;
  for (int it = 0; it < 1000000; ++it) {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    double moved = 0.0;
    for (int i = 0; i < L; ++i) {
      double a = i == 0 ? -INFINITY : t[i - 1];
      double b = i == L - 1 ? INFINITY : t[i];
      double m0, m1;
      cell(a, b, &m0, &m1);
      nc[i] = m1 / m0;
      moved = std::max(moved, std::fabs(nc[i] - c[i]));
    }
    c = nc;
    if (moved <= 1e-15) break;
  }
  for (int i = 0; i < L / 2; ++i) {  // exact symmetry
    double m = 0.5 * (c[L - 1 - i] - c[i]);
    c[i] = -m;
    c[L - 1 - i] = m;
  }
  double sum = 0.0, total = 0.0;
  for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  t[L / 2 - 1] = 0.0;
  for (int i = 0; i < L; ++i) {
    double a = i == 0 ? -INFINITY : t[i - 1];
    double b = i == L - 1 ? INFINITY : t[i];
    double m0, m1;
    cell(a, b, &m0, &m1);
    sum += m0 * c[i] * c[i];
    total += m0;
  }
  for (int i = 0; i < L; ++i) levels[i] = c[i];
  for (int k = 0; k + 1 < L; ++k) edges[k] = t[k];
  // E[(X - Q X)^2] = E[X^2] - sum_i P_i c_i^2 at a Lloyd fixed point, E[X^2] = 1
  *distortion = 1.0 - sum / total;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
size_t esize(tq_dtype t) { return t == TQ_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tq_status check_config(const tq_config* cfg, const char* who) {
  if (!cfg) return fail(TQ_ERR_INVALID_ARG, "%s: cfg is NULL", who);
  if (cfg->dt != 32 && cfg->dt != 64 && cfg->dt != 128 && cfg->dt != 256)
    return fail(TQ_ERR_INVALID_ARG, "%s: dt must be 32, 64, 128 or 256 (got %d)", who, cfg->dt);
  if (cfg->head_dim <= 0 || cfg->head_dim % cfg->dt || cfg->head_dim > 65536)
    return fail(TQ_ERR_INVALID_ARG, "%s: head_dim (%d) must be a positive multiple of dt (%d), <= 65536", who,
                cfg->head_dim, cfg->dt);
  if ((cfg->bits < 1 || cfg->bits > 4) && cfg->bits != 8)
    return fail(TQ_ERR_UNSUPPORTED, "%s: bits must be 1..4 or 8 (got %d)", who, cfg->bits);
  if (!cfg->cb) return fail(TQ_ERR_INVALID_ARG, "%s: codebook is NULL", who);
  if (cfg->cb->bits != cfg->bits || cfg->cb->dim != cfg->dt)
    return fail(TQ_ERR_INVALID_ARG, "%s: codebook (bits %d, dim %d) does not match config (bits %d, dt %d)", who,
                cfg->cb->bits, cfg->cb->dim, cfg->bits, cfg->dt);
  if (!cfg->signs) return fail(TQ_ERR_INVALID_ARG, "%s: signs is NULL", who);
  for (int i = 0; i < cfg->dt; ++i)
    if (cfg->signs[i] != 1.0f && cfg->signs[i] != -1.0f)
      return fail(TQ_ERR_INVALID_ARG, "%s: signs[%d] = %g is not +1 or -1", who, i, (double)cfg->signs[i]);
  if (cfg->flags & ~(unsigned)(TQ_NORM_CORRECT | TQ_QJL | TQ_BLOCKS))
    return fail(TQ_ERR_INVALID_ARG, "%s: unknown flag bits 0x%x", who, cfg->flags);
  if ((cfg->x_dtype != TQ_F16 && cfg->x_dtype != TQ_F32) || (cfg->norm_dtype != TQ_F16 && cfg->norm_dtype != TQ_F32))
    return fail(TQ_ERR_INVALID_ARG, "%s: dtype must be TQ_F16 or TQ_F32", who);
  if (cfg->flags & TQ_BLOCKS) {
    if (cfg->norm_dtype != TQ_F16)
      return fail(TQ_ERR_INVALID_ARG, "%s: TQ_BLOCKS records carry fp16 norms (norm_dtype must be TQ_F16)", who);
    if (cfg->flags & TQ_QJL) return fail(TQ_ERR_UNSUPPORTED, "%s: TQ_BLOCKS does not combine with TQ_QJL", who);
  }
  if (cfg->flags & TQ_QJL) {
    if (cfg->bits > 4) return fail(TQ_ERR_UNSUPPORTED, "%s: QJL takes a 1..4-bit MSE stage (got %d)", who, cfg->bits);
    if (cfg->head_dim != cfg->dt)
      return fail(TQ_ERR_UNSUPPORTED, "%s: QJL needs one unit per row (dt == head_dim)", who);
    if (cfg->qjl_m < 32 || cfg->qjl_m > 256 || cfg->qjl_m % 32)
      return fail(TQ_ERR_INVALID_ARG, "%s: qjl_m must be a multiple of 32 in 32..256 (got %d)", who, cfg->qjl_m);
    if (cfg->qjl_m * cfg->dt > 16384)
      return fail(TQ_ERR_UNSUPPORTED, "%s: QJL needs qjl_m * dt <= 16384 (the projection is staged in 64 KiB of LDS)",
                  who);
  }
  return TQ_OK;
}

tq_status check_params(const tq_config* cfg, const char* who) {
  if (!cfg->qjl_params) return fail(TQ_ERR_INVALID_ARG, "%s: qjl_params is NULL (call tq_qjl_prepare)", who);
  if (!aligned(cfg->qjl_params, 16)) return fail(TQ_ERR_INVALID_ARG, "%s: qjl_params must be 16-byte aligned", who);
  return TQ_OK;
}

tq_status check_rows(const char* who, const char* name, const void* p, int64_t n_rows, int64_t ld, int head_dim,
                     size_t es) {
  if (!p) return fail(TQ_ERR_INVALID_ARG, "%s: %s is NULL", who, name);
  if (ld < head_dim) return fail(TQ_ERR_INVALID_ARG, "%s: ld of %s (%lld) < head_dim (%d)", who, name, (long long)ld,
                                 head_dim);
  if (!aligned(p, 16) || (ld * (int64_t)es) % 16)
    return fail(TQ_ERR_INVALID_ARG, "%s: %s must be 16-byte aligned with a row stride that is a multiple of 16 bytes",
                who, name);
  if (n_rows > (int64_t)(INT64_MAX / 4) / (ld * (int64_t)es))
    return fail(TQ_ERR_INVALID_ARG, "%s: %s size overflows", who, name);
  return TQ_OK;
}

// codes / norms of tq_quantize and tq_dequantize: two planes, or records (TQ_BLOCKS)
tq_status check_code_planes(const tq_config* cfg, const char* who, const void* codes, const void* norms) {
  if (cfg->flags & TQ_BLOCKS) {
    if (!codes || !aligned(codes, 16))
      return fail(TQ_ERR_INVALID_ARG, "%s: TQ_BLOCKS records (codes) must be non-NULL, 16-byte aligned", who);
    if (norms) return fail(TQ_ERR_INVALID_ARG, "%s: with TQ_BLOCKS the norms live in the records; pass NULL", who);
    return TQ_OK;
  }
  if (!codes || !aligned(codes, 4)) return fail(TQ_ERR_INVALID_ARG, "%s: codes must be non-NULL, 4-byte aligned", who);
  if (!norms || !aligned(norms, esize(cfg->norm_dtype)))
    return fail(TQ_ERR_INVALID_ARG, "%s: norms must be non-NULL and aligned to its element size", who);
  return TQ_OK;
}

void fill_dbits(const tq_config& cfg, uint32_t* dbits) {
  for (int w = 0; w < 8; ++w) dbits[w] = 0;
  for (int c = 0; c < cfg.dt; ++c)
    if (cfg.signs[c] < 0.0f) dbits[c / 32] |= 1u << (c % 32);
}

// N(0,1) centroid of each stored code: code = s << (b-1) | m, with the
// positive half's m-th level for s = 0 and its negative for s = 1.
template <typename T, int N>
void fill_levels(const tq_codebook& cb, T (&level)[N]) {
  const int L = 1 << cb.bits, h = L / 2;
  for (int code = 0; code < N; ++code) level[code] = 0;
  for (int code = 0; code < L && code < N; ++code) {
    int s = code >> (cb.bits - 1), m = code & (h - 1);
    int idx = s ? h - 1 - m : h + m;
    level[code] = (T)cb.unit_centroids[idx];
  }
}

template <typename T, int N>
void fill_thr(const tq_codebook& cb, T (&thr)[N]) {
  const int L = 1 << cb.bits, h = L / 2;
  for (int k = 0; k < N; ++k) thr[k] = (T)INFINITY;
  for (int k = 0; k + 1 < h && k < N; ++k) thr[k] = (T)cb.unit_bounds[h + k];  // edges above 0, ascending
}

// Bins of the 4- and 8-bit encoders' bucket tables: consecutive edges (the
// first one and 0 too) lie at least 1.6 bins apart, so any window of 1.52 bins
// holds at most one edge; the last entry is the first bin whose window (from
// 0.51 below it) starts at or above the top edge.
void fill_bins(const tq_codebook& cb, tq::EncodeArgs& a) {
  a.bin_scale = 0.0f;
  a.n_bins = 0;
  if (cb.bits != 4 && cb.bits != 8) return;
  const int h = 1 << (cb.bits - 1);
  double w = cb.unit_bounds[h];  // the cell [0, t_1]
  for (int k = 1; k + 1 < h; ++k) w = std::min(w, cb.unit_bounds[h + k] - cb.unit_bounds[h + k - 1]);
  const double scale = 1.6 / w;
  a.bin_scale = (float)scale;
  a.n_bins = (int32_t)std::ceil(cb.unit_bounds[2 * h - 2] * scale + 0.51) + 1;
}

void fwht_inplace(double* v, int d) {
  for (int bit = 1; bit < d; bit <<= 1)
    for (int i = 0; i < d; ++i)
      if (!(i & bit)) {
        double a = v[i], b = v[i | bit];
        v[i] = a + b;
        v[i | bit] = a - b;
      }
  double s = 1.0 / std::sqrt((double)d);
  for (int i = 0; i < d; ++i) v[i] *= s;
}

}  // namespace

extern "C" {

const char* tq_status_str(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported combination";
    case TQ_ERR_WORKSPACE: return "workspace missing or too small";
    case TQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* tq_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {
void scale_codebook(tq_codebook* out) {
  const double s = 1.0 / std::sqrt((double)out->dim);
  for (int i = 0; i < (1 << out->bits); ++i) out->centroids[i] = (float)(out->unit_centroids[i] * s);
  for (int i = 0; i + 1 < (1 << out->bits); ++i) out->bounds[i] = (float)(out->unit_bounds[i] * s);
}
}  // namespace

extern "C" {

tq_status tq_codebook_init(tq_codebook* out, int bits, int dim) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_codebook_init: out is NULL");
  if (bits < 1 || bits > 8) return fail(TQ_ERR_INVALID_ARG, "tq_codebook_init: bits must be 1..8 (got %d)", bits);
  if (!is_pow2(dim) || dim < 2 || dim > 4096)
    return fail(TQ_ERR_INVALID_ARG, "tq_codebook_init: dim must be a power of two in 2..4096 (got %d)", dim);
  std::memset(out, 0, sizeof(*out));
  out->bits = bits;
  out->dim = dim;
  if (bits <= 4) {
    solve_lloyd_max(bits, GaussCell{}, 3.0, out->unit_centroids, out->unit_bounds, &out->distortion);
  } else if (!solve_lloyd_max_newton(bits, out->unit_centroids, out->unit_bounds, &out->distortion)) {
    return fail(TQ_ERR_INVALID_ARG, "tq_codebook_init: the %d-bit Lloyd-Max solve did not converge", bits);
  }
  scale_codebook(out);
  return ok();
}

tq_status tq_codebook_init_beta(tq_codebook* out, int bits, int dim) {
  if (!out) return fail(TQ_ERR_INVALID_ARG, "tq_codebook_init_beta: out is NULL");
  if (bits < 1 || bits > 4)
    return fail(TQ_ERR_INVALID_ARG, "tq_codebook_init_beta: bits must be 1..4 (got %d)", bits);
  if (!is_pow2(dim) || dim < 4 || dim > 4096)
    return fail(TQ_ERR_INVALID_ARG, "tq_codebook_init_beta: dim must be a power of two in 4..4096 (got %d)", dim);
  std::memset(out, 0, sizeof(*out));
  out->bits = bits;
  out->dim = dim;
  // start inside the support |u| < sqrt(dim)
  const double r = std::min(3.0, 0.9 * std::sqrt((double)dim));
  solve_lloyd_max(bits, SphereCell{dim}, r, out->unit_centroids, out->unit_bounds, &out->distortion);
  scale_codebook(out);
  return ok();
}

size_t tq_qjl_params_size(int m, int dt) {
  if (m <= 0 || dt <= 0) return 0;
  size_t b = (size_t)m * dt * (sizeof(double) + sizeof(float));
  return (b + 255) & ~(size_t)255;
}

tq_status tq_qjl_prepare(const tq_config* cfg, const float* S_host, void* params_dev, size_t params_bytes,
                         void* stream) {
  tq_status st = check_config(cfg, "tq_qjl_prepare");
  if (st) return st;
  if (!(cfg->flags & TQ_QJL)) return fail(TQ_ERR_INVALID_ARG, "tq_qjl_prepare: cfg has no TQ_QJL flag");
  if (!S_host || !params_dev) return fail(TQ_ERR_INVALID_ARG, "tq_qjl_prepare: NULL pointer");
  if (!aligned(params_dev, 16)) return fail(TQ_ERR_INVALID_ARG, "tq_qjl_prepare: params_dev must be 16-byte aligned");
  const int m = cfg->qjl_m, dt = cfg->dt;
  if (params_bytes < tq_qjl_params_size(m, dt))
    return fail(TQ_ERR_WORKSPACE, "tq_qjl_prepare: params buffer has %zu bytes, needs %zu", params_bytes,
                tq_qjl_params_size(m, dt));
  std::vector<double> s64((size_t)m * dt);
  std::vector<float> s32((size_t)m * dt);
  for (int p = 0; p < m; ++p) {
    double* row = &s64[(size_t)p * dt];
    for (int j = 0; j < dt; ++j) row[j] = (double)S_host[(size_t)p * dt + j] * (double)cfg->signs[j];
    fwht_inplace(row, dt);  // (S D H)[p] = H (S D)[p]^T, H symmetric
    for (int j = 0; j < dt; ++j) s32[(size_t)p * dt + j] = (float)row[j];
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(params_dev, s64.data(), s64.size() * sizeof(double), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync((char*)params_dev + s64.size() * sizeof(double), s32.data(), s32.size() * sizeof(float),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "tq_qjl_prepare");
  return ok();
}

tq_status tq_quantize(const tq_config* cfg, const void* x, int64_t n_rows, int64_t ld_x, uint8_t* codes, void* norms,
                      uint8_t* qjl_bits, void* qjl_rnorm, void* stream) {
  const char* who = "tq_quantize";
  tq_status st = check_config(cfg, who);
  if (st) return st;
  if (n_rows < 0) return fail(TQ_ERR_INVALID_ARG, "%s: n_rows < 0", who);
  if (n_rows == 0) return ok();
  if ((st = check_rows(who, "x", x, n_rows, ld_x, cfg->head_dim, esize(cfg->x_dtype)))) return st;
  if ((st = check_code_planes(cfg, who, codes, norms))) return st;
  hipStream_t s = (hipStream_t)stream;
  if (cfg->flags & TQ_QJL) {
    if ((st = check_params(cfg, who))) return st;
    if (!qjl_bits || !aligned(qjl_bits, 4) || !qjl_rnorm || !aligned(qjl_rnorm, 2))
      return fail(TQ_ERR_INVALID_ARG, "%s: QJL needs qjl_bits (4-byte aligned) and qjl_rnorm (2-byte aligned)", who);
    tq::QjlEncodeArgs a{};
    a.x = x;
    a.ld_x = ld_x;
    a.codes = codes;
    a.norms = norms;
    a.qjl_bits = qjl_bits;
    a.rnorm = (uint16_t*)qjl_rnorm;
    a.n_units = n_rows;
    a.s_rot = (const double*)cfg->qjl_params;
    a.m = cfg->qjl_m;
    fill_dbits(*cfg, a.dbits);
    fill_thr(*cfg->cb, a.thr);
    fill_levels(*cfg->cb, a.level);
    hipError_t e = tq::launch_qjl_encode(*cfg, a, s);
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
  }
  tq::EncodeArgs a{};
  a.x = x;
  a.ld_x = ld_x;
  a.codes = codes;
  a.norms = norms;
  a.groups_per_row = cfg->head_dim / 32;
  a.n_groups = n_rows * a.groups_per_row;
  a.contiguous = ld_x == cfg->head_dim;
  fill_dbits(*cfg, a.dbits);
  fill_thr(*cfg->cb, a.thr);
  fill_bins(*cfg->cb, a);
  const int max_bins = cfg->cb->bits == 4 ? tq::kLutEntries4 : tq::kMaxBins8;
  if (a.n_bins > max_bins)
    return fail(TQ_ERR_INVALID_ARG, "%s: the %d-bit codebook's narrowest cell needs %d bins (max %d)", who,
                cfg->cb->bits, a.n_bins, max_bins);
  hipError_t e = tq::launch_encode(*cfg, a, s);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

tq_status tq_dequantize(const tq_config* cfg, const uint8_t* codes, const void* norms, const uint8_t* qjl_bits,
                        const void* qjl_rnorm, int64_t n_rows, void* y, tq_dtype y_dtype, int64_t ld_y,
                        void* stream) {
  const char* who = "tq_dequantize";
  tq_status st = check_config(cfg, who);
  if (st) return st;
  if (y_dtype != TQ_F16 && y_dtype != TQ_F32) return fail(TQ_ERR_INVALID_ARG, "%s: bad y_dtype", who);
  if (n_rows < 0) return fail(TQ_ERR_INVALID_ARG, "%s: n_rows < 0", who);
  if (n_rows == 0) return ok();
  if ((st = check_rows(who, "y", y, n_rows, ld_y, cfg->head_dim, esize(y_dtype)))) return st;
  if ((st = check_code_planes(cfg, who, codes, norms))) return st;
  hipStream_t s = (hipStream_t)stream;
  const bool nc = (cfg->flags & TQ_NORM_CORRECT) != 0;
  if (cfg->flags & TQ_QJL) {
    if ((st = check_params(cfg, who))) return st;
    if (!qjl_bits || !aligned(qjl_bits, 4) || !qjl_rnorm || !aligned(qjl_rnorm, 2))
      return fail(TQ_ERR_INVALID_ARG, "%s: QJL needs qjl_bits (4-byte aligned) and qjl_rnorm (2-byte aligned)", who);
    tq::QjlDecodeArgs a{};
    a.codes = codes;
    a.norms = norms;
    a.qjl_bits = qjl_bits;
    a.rnorm = (const uint16_t*)qjl_rnorm;
    a.m = cfg->qjl_m;
    a.s_rot = (const float*)((const char*)cfg->qjl_params + (size_t)cfg->qjl_m * cfg->dt * sizeof(double));
    a.y = y;
    a.ld_y = ld_y;
    a.n_units = n_rows;
    fill_dbits(*cfg, a.dbits);
    fill_levels(*cfg->cb, a.level);
    a.qjl_scale = (float)(std::sqrt((double)cfg->dt) * std::sqrt(M_PI / 2.0) / cfg->qjl_m);
    a.inv_dt = 1.0f / cfg->dt;
    a.inv_sqrt_dt = (float)(1.0 / std::sqrt((double)cfg->dt));
    hipError_t e = tq::launch_qjl_decode(*cfg, a, nc, y_dtype, s);
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
  }
  tq::DecodeArgs a{};
  a.codes = codes;
  a.norms = norms;
  a.y = y;
  a.ld_y = ld_y;
  a.groups_per_row = cfg->head_dim / 32;
  a.n_groups = n_rows * a.groups_per_row;
  a.contiguous = ld_y == cfg->head_dim;
  fill_dbits(*cfg, a.dbits);
  fill_levels(*cfg->cb, a.level);
  a.inv_dt = 1.0f / cfg->dt;
  a.inv_sqrt_dt = (float)(1.0 / std::sqrt((double)cfg->dt));
  hipError_t e = tq::launch_decode(*cfg, a, nc, y_dtype, s);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

}  // extern "C"

namespace {

struct ScoreLayout {
  int64_t n_q_pad, n_k_pad, rq, planes;
  size_t off_qrec, off_qscale, total;
};

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

ScoreLayout score_layout(const tq_config& cfg, int64_t n_q, int64_t n_k) {
  ScoreLayout L{};
  const int64_t kd = (cfg.dt + 63) / 64 * 64, km = (cfg.qjl_m + 63) / 64 * 64;
  const int64_t tile = tq::scores_key_tile(cfg.bits);
  L.planes = (int64_t)1 << (cfg.bits - 1);
  const int64_t qb = tq::scores_query_block();
  L.n_q_pad = (n_q + qb - 1) / qb * qb;
  L.n_k_pad = (n_k + tile - 1) / tile * tile;
  L.rq = 2 * (L.planes * kd + km);
  L.off_qrec = 0;
  L.off_qscale = round256(L.off_qrec + (size_t)(L.n_q_pad * L.rq));
  L.total = round256(L.off_qscale + (size_t)L.n_q_pad * 2 * sizeof(float));
  return L;
}

tq_status check_scores_config(const tq_config* cfg, const char* who) {
  tq_status st = check_config(cfg, who);
  if (st) return st;
  if (!(cfg->flags & TQ_QJL)) return fail(TQ_ERR_INVALID_ARG, "%s: cfg has no TQ_QJL flag", who);
  if (cfg->flags & TQ_NORM_CORRECT)
    return fail(TQ_ERR_UNSUPPORTED, "%s: norm correction does not apply to inner-product scores", who);
  if (cfg->bits > 3) return fail(TQ_ERR_UNSUPPORTED, "%s: QJL scores support 1..3-bit MSE stages", who);
  if (cfg->dt > 128 || cfg->qjl_m > 128)
    return fail(TQ_ERR_UNSUPPORTED, "%s: QJL scores support head_dim <= 128 and qjl_m <= 128", who);
  return TQ_OK;
}

// Attention: block-32 K and V (fp16 norms, K at 3, 4 or 8 bits, V at 3 or 4
// bits, no QJL or norm correction), head_dim 128 or 256.
tq_status check_attn_config(const tq_config* kcfg, const tq_config* vcfg, int n_q_heads, int n_kv_heads,
                            int64_t n_tokens, const char* who) {
  tq_status st = check_config(kcfg, who);
  if (st) return st;
  if ((st = check_config(vcfg, who))) return st;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads || n_tokens < 0)
    return fail(TQ_ERR_INVALID_ARG, "%s: need n_q_heads a positive multiple of n_kv_heads and n_tokens >= 0", who);
  if (kcfg->head_dim != vcfg->head_dim) return fail(TQ_ERR_INVALID_ARG, "%s: K and V head_dim differ", who);
  if (kcfg->dt != 32 || vcfg->dt != 32 || (kcfg->head_dim != 128 && kcfg->head_dim != 256))
    return fail(TQ_ERR_UNSUPPORTED, "%s: needs the block-32 layout (dt = 32) with head_dim 128 or 256", who);
  if ((kcfg->bits != 3 && kcfg->bits != 4 && kcfg->bits != 8) || (vcfg->bits != 3 && vcfg->bits != 4))
    return fail(TQ_ERR_UNSUPPORTED, "%s: K must be 3-, 4- or 8-bit and V 3- or 4-bit", who);
  if (kcfg->flags || vcfg->flags)
    return fail(TQ_ERR_UNSUPPORTED, "%s: QJL and norm correction are not supported in attention", who);
  if (kcfg->norm_dtype != TQ_F16 || vcfg->norm_dtype != TQ_F16)
    return fail(TQ_ERR_UNSUPPORTED, "%s: K and V norms must be fp16", who);
  if (n_kv_heads > 65535 || n_tokens > ((int64_t)1 << 40))
    return fail(TQ_ERR_UNSUPPORTED, "%s: at most 65535 KV heads and 2^40 tokens", who);
  return TQ_OK;
}

// Row groups of attention: rows = n_q * group (query token, head) pairs per KV head.  Up to 16
// rows go to the decode kernel as one group; more go to the prefill kernel in groups of 128.
struct AttnShape {
  int64_t rows, n_rg, grp, per_wg, wgs;
};
AttnShape attn_shape(int n_q_heads, int n_kv_heads, int64_t n_q, int64_t n_tokens) {
  AttnShape sh{};
  sh.rows = n_q * (n_q_heads / n_kv_heads);
  const bool prefill = sh.rows > 16;
  sh.grp = prefill ? tq::attn_prefill_rows() : sh.rows;
  sh.n_rg = (sh.rows + sh.grp - 1) / sh.grp;
  sh.per_wg = tq::attn_tokens_per_wg((int64_t)n_kv_heads * sh.n_rg, n_tokens, sh.grp);
  sh.wgs = (n_tokens + sh.per_wg - 1) / sh.per_wg;
  return sh;
}

// one fp32 partial (head_dim sums, softmax reference, weight sum) per row and token range
size_t attn_workspace(const tq_config& kcfg, int n_q_heads, int n_kv_heads, int64_t n_q, int64_t n_tokens) {
  const AttnShape sh = attn_shape(n_q_heads, n_kv_heads, n_q, n_tokens);
  const int64_t parts = (int64_t)n_kv_heads * sh.n_rg * sh.wgs * sh.grp;
  return round256((size_t)parts * (size_t)(kcfg.head_dim + 2) * sizeof(float));
}

tq_status run_attn(const char* who, const tq_config* kcfg, const tq_config* vcfg, const void* q, tq_dtype q_dtype,
                   int64_t n_q, int n_q_heads, int n_kv_heads, int64_t n_tokens, const uint8_t* k_codes,
                   const void* k_norms, const uint8_t* v_codes, const void* v_norms, int causal, float scale,
                   float* out, void* ws, size_t ws_bytes, void* stream) {
  tq_status st = check_attn_config(kcfg, vcfg, n_q_heads, n_kv_heads, n_tokens, who);
  if (st) return st;
  if (q_dtype != TQ_F16 && q_dtype != TQ_F32) return fail(TQ_ERR_INVALID_ARG, "%s: bad q_dtype", who);
  if (!(scale <= 0.0f || std::isfinite(scale))) return fail(TQ_ERR_INVALID_ARG, "%s: scale is not finite", who);
  if (n_q < 0) return fail(TQ_ERR_INVALID_ARG, "%s: n_q < 0", who);
  if (causal && n_q > n_tokens)
    return fail(TQ_ERR_INVALID_ARG, "%s: a causal call needs n_q <= n_tokens (the queries are the last positions)",
                who);
  if (n_tokens == 0 || n_q == 0) return ok();
  if (n_q > ((int64_t)1 << 31) / n_q_heads) return fail(TQ_ERR_UNSUPPORTED, "%s: at most 2^31 query rows", who);
  if (!q || !aligned(q, esize(q_dtype)) || !out || !aligned(out, 4))
    return fail(TQ_ERR_INVALID_ARG, "%s: q and out must be non-NULL and element-aligned", who);
  if (!k_codes || !aligned(k_codes, 4) || !v_codes || !aligned(v_codes, 4) || !k_norms || !aligned(k_norms, 2) ||
      !v_norms || !aligned(v_norms, 2))
    return fail(TQ_ERR_INVALID_ARG, "%s: codes must be 4-byte and norms 2-byte aligned, non-NULL", who);
  const AttnShape sh = attn_shape(n_q_heads, n_kv_heads, n_q, n_tokens);
  if ((int64_t)n_kv_heads * sh.n_rg > 65535)
    return fail(TQ_ERR_UNSUPPORTED, "%s: at most 65535 (KV head, row group) columns", who);
  const size_t need = attn_workspace(*kcfg, n_q_heads, n_kv_heads, n_q, n_tokens);
  if (!ws || !aligned(ws, 256) || ws_bytes < need)
    return fail(TQ_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned with %zu bytes (got %zu)", who, need,
                ws_bytes);
  tq::AttnArgs a{};
  a.q = q;
  a.q_f32 = q_dtype == TQ_F32;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.group = n_q_heads / n_kv_heads;
  a.head_dim = kcfg->head_dim;
  a.n_tokens = n_tokens;
  a.n_q = n_q;
  a.rows = sh.rows;
  a.grp = (int32_t)sh.grp;
  a.n_rg = (int32_t)sh.n_rg;
  a.causal = causal ? 1 : 0;
  a.k_codes = k_codes;
  a.k_norms = (const uint16_t*)k_norms;
  a.v_codes = v_codes;
  a.v_norms = (const uint16_t*)v_norms;
  a.out = out;
  a.part = (float*)ws;
  a.tokens_per_wg = sh.per_wg;
  a.wg_per_head = (int32_t)sh.wgs;
  uint32_t db[8];
  fill_dbits(*kcfg, db);
  a.kdbits = db[0];
  fill_dbits(*vcfg, db);
  a.vdbits = db[0];
  fill_levels(*kcfg->cb, a.klevel);
  fill_levels(*vcfg->cb, a.vlevel);
  const double sc = scale > 0.0f ? (double)scale : 1.0 / std::sqrt((double)kcfg->head_dim);
  a.kscale = (float)(sc / std::sqrt(32.0));
  hipError_t e = tq::launch_decode_attn(kcfg->bits, vcfg->bits, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

}  // namespace

extern "C" {

tq_status tq_qjl_scores(const tq_config* cfg, const void* q, tq_dtype q_dtype, int64_t n_q, int64_t ld_q,
                        const uint8_t* codes, const void* norms, const uint8_t* qjl_bits, const void* qjl_rnorm,
                        int64_t n_k, float* scores, int64_t ld_s, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "tq_qjl_scores";
  tq_status st = check_scores_config(cfg, who);
  if (st) return st;
  if (q_dtype != TQ_F16 && q_dtype != TQ_F32) return fail(TQ_ERR_INVALID_ARG, "%s: bad q_dtype", who);
  if (n_q < 0 || n_k < 0) return fail(TQ_ERR_INVALID_ARG, "%s: negative sizes", who);
  if (n_q == 0 || n_k == 0) return ok();
  if (n_q > ((int64_t)1 << 31) || n_k > ((int64_t)1 << 31))
    return fail(TQ_ERR_UNSUPPORTED, "%s: at most 2^31 queries and keys per call", who);
  if (!q || !aligned(q, esize(q_dtype)) || ld_q < cfg->head_dim)
    return fail(TQ_ERR_INVALID_ARG, "%s: q must be non-NULL, element-aligned, ld_q >= head_dim", who);
  if (!codes || !aligned(codes, 4) || !norms || !aligned(norms, esize(cfg->norm_dtype)) || !qjl_bits ||
      !aligned(qjl_bits, 4) || !qjl_rnorm || !aligned(qjl_rnorm, 2))
    return fail(TQ_ERR_INVALID_ARG, "%s: codes, norms, qjl_bits and qjl_rnorm must be non-NULL and aligned", who);
  if (!scores || !aligned(scores, 4) || ld_s < n_k)
    return fail(TQ_ERR_INVALID_ARG, "%s: scores must be non-NULL, 4-byte aligned, ld_s >= n_k", who);
  if (n_q > INT64_MAX / 8 / ld_s) return fail(TQ_ERR_INVALID_ARG, "%s: scores size overflows", who);
  if ((st = check_params(cfg, who))) return st;
  const ScoreLayout L = score_layout(*cfg, n_q, n_k);
  if (!ws || !aligned(ws, 256) || ws_bytes < L.total)
    return fail(TQ_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned with %zu bytes (got %zu)", who, L.total,
                ws_bytes);
  tq::ScoreArgs a{};
  a.q = q;
  a.ld_q = ld_q;
  a.n_q = n_q;
  a.n_q_pad = L.n_q_pad;
  a.codes = codes;
  a.norms = norms;
  a.qjl_bits = qjl_bits;
  a.rnorm = (const uint16_t*)qjl_rnorm;
  a.n_k = n_k;
  a.n_k_pad = L.n_k_pad;
  a.scores = scores;
  a.ld_s = ld_s;
  char* w = (char*)ws;
  a.qrec = (int8_t*)(w + L.off_qrec);
  a.qscale = (float*)(w + L.off_qscale);
  a.s_rot32 = (const float*)((const char*)cfg->qjl_params + (size_t)cfg->qjl_m * cfg->dt * sizeof(double));
  fill_dbits(*cfg, a.dbits);
  // ternary plane weights: level(mag) = sum over the bit subsets t of mag of w_t (Moebius inversion)
  const int h = 1 << (cfg->bits - 1);
  for (int t = 0; t < 8; ++t) a.plane_w[t] = 0.0f;
  for (int t = 0; t < h; ++t) {
    double wt = 0.0;
    for (int s = 0; s < h; ++s)
      if ((s & t) == s)
        wt += (((__builtin_popcount(t) - __builtin_popcount(s)) & 1) ? -1.0 : 1.0) * cfg->cb->unit_centroids[h + s];
    a.plane_w[t] = (float)wt;
  }
  a.dt = cfg->dt;
  a.m = cfg->qjl_m;
  a.kd = (cfg->dt + 63) / 64 * 64;
  a.km = (cfg->qjl_m + 63) / 64 * 64;
  a.q_f32 = q_dtype == TQ_F32;
  a.inv_sqrt_dt = (float)(1.0 / std::sqrt((double)cfg->dt));
  a.qjl_const = (float)(std::sqrt(M_PI / 2.0) / cfg->qjl_m);
  hipError_t e = tq::launch_qjl_scores(*cfg, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, who);
  return ok();
}

tq_status tq_decode_attn(const tq_config* kcfg, const tq_config* vcfg, const void* q, tq_dtype q_dtype,
                         int n_q_heads, int n_kv_heads, int64_t n_tokens, const uint8_t* k_codes, const void* k_norms,
                         const uint8_t* v_codes, const void* v_norms, float scale, float* out, void* ws,
                         size_t ws_bytes, void* stream) {
  return run_attn("tq_decode_attn", kcfg, vcfg, q, q_dtype, 1, n_q_heads, n_kv_heads, n_tokens, k_codes, k_norms,
                  v_codes, v_norms, 0, scale, out, ws, ws_bytes, stream);
}

tq_status tq_decode_attn_noalloc(const tq_config* kcfg, const tq_config* vcfg, const void* q, tq_dtype q_dtype,
                                 int n_q_heads, int n_kv_heads, int64_t n_tokens, const uint8_t* k_codes,
                                 const void* k_norms, const uint8_t* v_codes, const void* v_norms, float scale,
                                 float* out, void* stream) {
  const char* who = "tq_decode_attn_noalloc";
  tq_status st = check_attn_config(kcfg, vcfg, n_q_heads, n_kv_heads, n_tokens, who);
  if (st) return st;
  if (n_tokens == 0)  // a no-op; run_attn checks the remaining arguments
    return run_attn(who, kcfg, vcfg, q, q_dtype, 1, n_q_heads, n_kv_heads, n_tokens, k_codes, k_norms, v_codes,
                    v_norms, 0, scale, out, nullptr, 0, stream);
  const size_t need = attn_workspace(*kcfg, n_q_heads, n_kv_heads, 1, n_tokens);
  if (need > tq::kAttnScratchBytes)
    return fail(TQ_ERR_UNSUPPORTED,
                "%s: this call needs %zu bytes of scratch; the library's static scratch holds %zu (use "
                "tq_decode_attn with a workspace)",
                who, need, tq::kAttnScratchBytes);
  void* ws = nullptr;
  const hipError_t e = tq::attn_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, who);
  return run_attn(who, kcfg, vcfg, q, q_dtype, 1, n_q_heads, n_kv_heads, n_tokens, k_codes, k_norms, v_codes,
                  v_norms, 0, scale, out, ws, tq::kAttnScratchBytes, stream);
}

tq_status tq_multi_attn(const tq_config* kcfg, const tq_config* vcfg, const void* q, tq_dtype q_dtype, int64_t n_q,
                        int n_q_heads, int n_kv_heads, int64_t n_tokens, const uint8_t* k_codes, const void* k_norms,
                        const uint8_t* v_codes, const void* v_norms, int causal, float scale, float* out, void* ws,
                        size_t ws_bytes, void* stream) {
  return run_attn("tq_multi_attn", kcfg, vcfg, q, q_dtype, n_q, n_q_heads, n_kv_heads, n_tokens, k_codes, k_norms,
                  v_codes, v_norms, causal, scale, out, ws, ws_bytes, stream);
}

size_t tq_workspace_size(int op, const tq_config* cfg, int64_t a, int64_t b, int64_t c) {
  (void)c;
  if (op == TQ_OP_QJL_SCORES) {
    if (check_scores_config(cfg, "tq_workspace_size") || a < 0 || b < 0) return 0;
    return score_layout(*cfg, a, b).total;
  }
  if (op == TQ_OP_DECODE_ATTN) {
    if (a <= 0 || b <= 0 || a > 65536 || a % b || c < 0 || check_config(cfg, "tq_workspace_size")) return 0;
    return attn_workspace(*cfg, (int)a, (int)b, 1, c);
  }
  if (op == TQ_OP_MULTI_ATTN) {  // a = n_q * n_q_heads query rows, b = n_kv_heads, c = n_tokens
    if (a <= 0 || b <= 0 || b > 65535 || a % b || c < 0 || check_config(cfg, "tq_workspace_size")) return 0;
    return attn_workspace(*cfg, (int)b, (int)b, a / b, c);
  }
  return 0;
}

}  // extern "C"
