// Host side of the C ABI: argument validation, the Lloyd-Max codebook builder,
// quantizer lifecycle and dispatch to the HIP kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tq_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Coordinate law of a uniform point on S^{d-1}: density proportional to
// (1-u^2)^((d-3)/2) on [-1, 1] (the Beta-shaped law of the AiBoss overview,
// section "TurboQuantの技術原理").
//
// Lloyd-Max needs, per cell [lo, hi] of the positive half-line, the cell's
// mass and first moment.  With u = sin(th) both become integrals over an
// angle:
//   mass(lo, hi)   = integral over [asin lo, asin hi] of cos(th)^(d-2) dth
//   moment(lo, hi) = ((1-lo^2)^((d-1)/2) - (1-hi^2)^((d-1)/2)) / (d-1)
// The angular integrand is analytic (no endpoint singularity for any d >= 3),
// so composite Gauss-Legendre quadrature converges geometrically.  Both
// quantities are carried relative to the density at `lo` (its maximum on the
// cell), so nothing underflows at large d; the normalising constant cancels
// in the conditional mean and is never evaluated.
// ---------------------------------------------------------------------------
constexpr int kGaussNodes = 24;

struct GaussLegendre {
  double x[kGaussNodes], w[kGaussNodes];  // nodes and weights on [-1, 1]
  GaussLegendre() {
    // Newton's method on the Legendre polynomial P_n, started from the
    // asymptotic root estimate cos(pi (i + 3/4) / (n + 1/2)); P_n and its
    // derivative come from the three-term recurrence.
    const int n = kGaussNodes;
    for (int i = 0; i < n; ++i) {
      double r = std::cos(M_PI * (i + 0.75) / (n + 0.5)), dp = 1.0;
      for (int it = 0; it < 100; ++it) {
        double p_prev = 1.0, p = r;
        for (int k = 2; k <= n; ++k) {
          const double p_next = ((2.0 * k - 1.0) * r * p - (k - 1.0) * p_prev) / k;
          p_prev = p;
          p = p_next;
        }
        dp = n * (r * p - p_prev) / (r * r - 1.0);
        const double step = p / dp;
        r -= step;
        if (std::fabs(step) < 1e-17) break;
      }
      x[i] = r;
      w[i] = 2.0 / ((1.0 - r * r) * dp * dp);
    }
  }
};

const GaussLegendre &gauss_legendre() {
  static const GaussLegendre g;
  return g;
}

// log of (1-u^2)^(1/2) = log cos(asin u), accurate for small u
double log_cos_of(double u) { return 0.5 * std::log1p(-u * u); }

// Mass of the cell [lo, hi] (0 <= lo < hi <= 1) divided by the density's
// value at lo, i.e. integral of exp((d-2) (log cos th - log cos th_lo)).
double cell_mass_rel(int d, double lo, double hi) {
  const double e = d - 2.0;
  const double th0 = std::asin(lo);
  double th1 = std::asin(hi);
  if (e > 0.0) {
    // beyond cos(th) = cos(th0) exp(-60/e) the integrand is below e^-60 of
    // its value at th0 and adds nothing at fp64 resolution
    const double c_cut = std::sqrt(1.0 - lo * lo) * std::exp(-60.0 / e);
    th1 = std::fmin(th1, std::acos(c_cut));
  }
  const double lc0 = log_cos_of(lo);
  // panels no wider than half the angular scale of the integrand
  const double scale = 1.0 / std::sqrt(e + 1.0 + e * std::tan(th0) * std::tan(th0) * e);
  const int panels = std::max(1, (int)std::ceil((th1 - th0) / (0.5 * scale)));
  const double h = (th1 - th0) / panels;
  const GaussLegendre &g = gauss_legendre();
  double total = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double mid = th0 + (p + 0.5) * h;
    double part = 0.0;
    for (int i = 0; i < kGaussNodes; ++i) {
      const double th = mid + 0.5 * h * g.x[i];
      part += g.w[i] * std::exp(e * (log_cos_of(std::sin(th)) - lc0));
    }
    total += 0.5 * h * part;
  }
  return total;
}

// First moment of the cell divided by the density's value at lo (closed form).
double cell_moment_rel(int d, double lo, double hi) {
  const double lc0 = log_cos_of(lo);
  const double top = std::exp(lc0);  // (1-lo^2)^((d-1)/2) / (1-lo^2)^((d-2)/2)
  const double bot = hi >= 1.0 ? 0.0 : std::exp((d - 1.0) * log_cos_of(hi) - (d - 2.0) * lc0);
  return (top - bot) / (d - 1.0);
}

double cell_mean(int d, double lo, double hi) { return cell_moment_rel(d, lo, hi) / cell_mass_rel(d, lo, hi); }

int lloyd_max(int d, int bits, double *c, double *t) {
  if (bits == 0) {  // one cell: its centroid is the mean of the symmetric law
    c[0] = 0.0;
    return TQ_OK;
  }
  const int L = 1 << bits, H = L / 2;
  std::vector<double> pos(H), nxt(H);
  // start from the Gaussian-limit quantiles of the positive half
  auto norm_ppf = [](double p) {
    double lo = -40.0, hi = 40.0;
    for (int i = 0; i < 200; ++i) {
      double mid = 0.5 * (lo + hi);
      double cdf = 0.5 * std::erfc(-mid / std::sqrt(2.0));
      if (cdf < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
  };
  for (int k = 0; k < H; ++k) pos[k] = norm_ppf((H + k + 0.5) / L) / std::sqrt((double)d);
  for (int it = 0; it < 20000; ++it) {
    double step = 0.0, cmax = 0.0;
    for (int k = 0; k < H; ++k) {
      double lo = k == 0 ? 0.0 : 0.5 * (pos[k - 1] + pos[k]);
      double hi = k == H - 1 ? 1.0 : 0.5 * (pos[k] + pos[k + 1]);
      nxt[k] = cell_mean(d, lo, hi);
    }
    for (int k = 0; k < H; ++k) {
      step = std::fmax(step, std::fabs(nxt[k] - pos[k]));
      cmax = std::fmax(cmax, std::fabs(nxt[k]));
      pos[k] = nxt[k];
    }
    if (step <= 1e-16 * cmax) break;
  }
  for (int k = 0; k < H; ++k) {
    c[H + k] = pos[k];
    c[H - 1 - k] = -pos[k];
  }
  if (t) for (int k = 1; k < L; ++k) t[k - 1] = k == H ? 0.0 : 0.5 * (c[k - 1] + c[k]);
  return TQ_OK;
}

template <class T>
int dev_upload(T **dst, const T *src, size_t count) {
  hipError_t e = hipMalloc((void **)dst, count * sizeof(T));
  if (e != hipSuccess) { *dst = nullptr; g_last_hip_error = e; return TQ_ERR_NOMEM; }
  if (src) {
    e = hipMemcpy(*dst, src, count * sizeof(T), hipMemcpyHostToDevice);
    if (e != hipSuccess) return tq::hip_fail(e);
  }
  return TQ_OK;
}

void free_q(tq_quantizer *q) {
  if (!q) return;
  int prev = -1;
  hipGetDevice(&prev);
  hipSetDevice(q->device);
  hipFree(q->pi);
  hipFree(q->piT);
  hipFree(q->s);
  hipFree(q->sT);
  hipFree(q->m);
  hipFree(q->pi3);
  hipFree(q->m3);
  hipFree(q->pih);
  hipFree(q->mh);
  hipFree(q->pit3);
  hipFree(q->st3);
  if (prev >= 0) hipSetDevice(prev);
  delete q;
}

bool valid_dtype(int t) { return t == TQ_F32 || t == TQ_BF16 || t == TQ_F16; }
size_t dtype_size(int t) { return t == TQ_F32 ? 4 : 2; }

}  // namespace

namespace tq {

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return TQ_ERR_HIP;
}

int launch_check() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  return TQ_OK;
}

}  // namespace tq

static int attn_decode_impl(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq,
                            int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                            const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                            int64_t Tstride, const int32_t *seq_len, float scale, float *out, void *ws,
                            size_t ws_bytes, const tq::AppendArgs *app, void *stream) {
  if (!kq || !vq || vq->mode != TQ_PROD || kq->d != vq->d) return TQ_ERR_INVALID;
  const bool kprod = kq->mode == TQ_PROD;
  if (kq->device != vq->device) return TQ_ERR_INVALID;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Tstride < 0 || !valid_dtype(qt)) return TQ_ERR_INVALID;
  if (vlayout != TQ_LAYOUT_ROWS && vlayout != TQ_LAYOUT_TILE32) return TQ_ERR_INVALID;
  if ((int64_t)B * Hq > 2147483647 / 2 || (int64_t)B * Hkv * ((Hq / Hkv + 3) / 4) > 2147483647) return TQ_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return TQ_ERR_INVALID;
  if (B == 0) return TQ_OK;
  if (!q || !out || !seq_len) return TQ_ERR_INVALID;
  if (Tstride > 0 && (!kcodes || !knorms || !vcodes || !vnorms || !vgammas || (kprod && !kgammas)))
    return TQ_ERR_INVALID;
  if ((Tstride > 0 && (!aligned16(kcodes) || !aligned16(vcodes))) || !aligned16(out) || !aligned16(q))
    return TQ_ERR_INVALID;
  size_t need = tq::attn_ws_bytes(kq, B, Hq, Hkv, Tstride, vlayout);
  if (need > 0 && (!ws || ws_bytes < need)) return TQ_ERR_WORKSPACE;
  return tq::run_attn_decode(kq, vq, q, qt, B, Hq, Hkv, kcodes, knorms, kprod ? kgammas : nullptr, vcodes, vnorms,
                             vgammas, vlayout, Tstride, seq_len, scale, out, ws, ws_bytes, app, (hipStream_t)stream);
}

extern "C" {

const char *tq_version(void) { return "0.1.0"; }

const char *tq_status_str(int s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_INVALID: return "TQ_ERR_INVALID";
    case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
    case TQ_ERR_HIP: return "TQ_ERR_HIP";
    case TQ_ERR_NOMEM: return "TQ_ERR_NOMEM";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
    default: return "TQ_ERR_UNKNOWN";
  }
}

int tq_last_hip_error(void) { return g_last_hip_error; }

int tq_codebook_build(int d, int bits, double *centroids, double *bounds) {
  if (d < 3 || d > 65536 || bits < 1 || bits > 8 || !centroids) return TQ_ERR_INVALID;
  return lloyd_max(d, bits, centroids, bounds);
}

int tq_quantizer_create(tq_quantizer **out, int d, int bits, int mode, const float *pi, const float *s) {
  if (!out) return TQ_ERR_INVALID;
  *out = nullptr;
  if (d < 64 || d > 2048 || d % 64 != 0 || !pi) return TQ_ERR_INVALID;
  if (mode == TQ_MSE) {
    if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
  } else if (mode == TQ_PROD) {
    if (bits < 1 || bits > 4) return TQ_ERR_UNSUPPORTED;
    if (!s) return TQ_ERR_INVALID;
  } else {
    return TQ_ERR_INVALID;
  }
  tq_quantizer *q = new (std::nothrow) tq_quantizer();
  if (!q) return TQ_ERR_NOMEM;
  q->d = d;
  q->bits = bits;
  q->mode = mode;
  q->bmse = mode == TQ_MSE ? bits : bits - 1;
  q->planes = bits;
  q->code_bytes = (size_t)bits * d / 8;
  q->qjl_scale = (float)(std::sqrt(M_PI / 2.0) / d);
  hipError_t e = hipGetDevice(&q->device);
  if (e != hipSuccess) { delete q; return tq::hip_fail(e); }
  lloyd_max(d, q->bmse, q->c64, q->t64);
  q->cb.L = 1 << q->bmse;
  for (int k = 0; k < q->cb.L; ++k) q->cb.c[k] = (float)q->c64[k];
  for (int k = 0; k + 1 < q->cb.L; ++k) q->cb.t[k] = (float)q->t64[k];

  const size_t dd = (size_t)d * d;
  std::vector<float> tr(dd);
  int rc = dev_upload(&q->pi, pi, dd);
  if (rc == TQ_OK) {
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) tr[(size_t)j * d + i] = pi[(size_t)i * d + j];
    rc = dev_upload(&q->piT, tr.data(), dd);
  }
  if (rc == TQ_OK && mode == TQ_PROD) {
    rc = dev_upload(&q->s, s, dd);
    if (rc == TQ_OK) {
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) tr[(size_t)j * d + i] = s[(size_t)i * d + j];
      rc = dev_upload(&q->sT, tr.data(), dd);
    }
    if (rc == TQ_OK) rc = dev_upload<float>(&q->m, nullptr, dd);
    if (rc == TQ_OK) rc = tq::compute_sPiT(d, q->s, q->pi, q->m, nullptr);
    if (rc == TQ_OK) rc = dev_upload<uint16_t>(&q->m3, nullptr, 3 * dd);
    if (rc == TQ_OK) rc = tq::make_pieces(q->m, (int64_t)dd, q->m3, nullptr);
  }
  if (rc == TQ_OK) rc = dev_upload<uint16_t>(&q->pi3, nullptr, 3 * dd);
  if (rc == TQ_OK) rc = tq::make_pieces(q->pi, (int64_t)dd, q->pi3, nullptr);
  if (rc == TQ_OK && d <= 512) {  // fp16 pieces: the fused encode (d <= 128) and the bf16 / fp16 row rotation
    // exponent e of v = m 2^e, m in [0.5, 1): v 2^(14 - e) < 2^14
    auto scale_exp = [](double v) {
      int e = 0;
      std::frexp(v, &e);
      return v > 0.0 ? 14 - e : 0;
    };
    double pmax = 0.0, prow = 0.0, srow = 0.0;
    for (int i = 0; i < d; ++i) {
      double r2 = 0.0, s2 = 0.0;
      for (int j = 0; j < d; ++j) {
        const double v = pi[(size_t)i * d + j];
        pmax = std::max(pmax, std::fabs(v));
        r2 += v * v;
        if (mode == TQ_PROD) s2 += (double)s[(size_t)i * d + j] * s[(size_t)i * d + j];
      }
      prow = std::max(prow, std::sqrt(r2));
      srow = std::max(srow, std::sqrt(s2));
    }
    q->kp = scale_exp(pmax);
    // |(S Pi^T)_ij| = |S_i . Pi_j| <= ||S_i|| ||Pi_j|| (with room for the fp32 rounding of the product)
    q->km = scale_exp(srow * prow * (1.0 + 1e-4));
    rc = dev_upload<uint16_t>(&q->pih, nullptr, 2 * dd);
    if (rc == TQ_OK) rc = tq::make_pieces_f16(q->pi, (int64_t)dd, q->kp, q->pih, nullptr);
    if (rc == TQ_OK && mode == TQ_PROD && d <= 128) rc = dev_upload<uint16_t>(&q->mh, nullptr, 2 * dd);
    if (rc == TQ_OK && mode == TQ_PROD && d <= 128) rc = tq::make_pieces_f16(q->m, (int64_t)dd, q->km, q->mh, nullptr);
  }
  if (rc == TQ_OK && d <= 128) {  // the fused decode's register-resident matrices
    rc = dev_upload<uint16_t>(&q->pit3, nullptr, 3 * dd);
    if (rc == TQ_OK) rc = tq::make_pieces(q->piT, (int64_t)dd, q->pit3, nullptr);
    if (rc == TQ_OK && mode == TQ_PROD) rc = dev_upload<uint16_t>(&q->st3, nullptr, 3 * dd);
    if (rc == TQ_OK && mode == TQ_PROD) rc = tq::make_pieces(q->sT, (int64_t)dd, q->st3, nullptr);
  }
  if (rc == TQ_OK) {
    e = hipDeviceSynchronize();
    if (e != hipSuccess) rc = tq::hip_fail(e);
  }
  if (rc != TQ_OK) { free_q(q); return rc; }
  *out = q;
  return TQ_OK;
}

void tq_quantizer_destroy(tq_quantizer *q) { free_q(q); }

int tq_quantizer_info(const tq_quantizer *q, int *d, int *bits, int *mode, int *planes, size_t *code_bytes) {
  if (!q) return TQ_ERR_INVALID;
  if (d) *d = q->d;
  if (bits) *bits = q->bits;
  if (mode) *mode = q->mode;
  if (planes) *planes = q->planes;
  if (code_bytes) *code_bytes = q->code_bytes;
  return TQ_OK;
}

static int check_encode(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx, const uint8_t *codes,
                        const uint16_t *norms) {
  if (!q || n < 0 || !valid_dtype(xt) || ldx < q->d) return TQ_ERR_INVALID;
  if (n == 0) return TQ_OK;
  if (!x || !codes || !norms) return TQ_ERR_INVALID;
  if (!aligned16(x) || !aligned16(codes) || (ldx * (int64_t)dtype_size(xt)) % 16 != 0) return TQ_ERR_INVALID;
  return TQ_OK;
}

int tq_encode_mse(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx, uint8_t *codes,
                  uint16_t *norms, void *stream) {
  int rc = check_encode(q, x, xt, n, ldx, codes, norms);
  if (rc != TQ_OK) return rc;
  if (q->mode != TQ_MSE) return TQ_ERR_INVALID;
  if (n == 0) return TQ_OK;
  return tq::run_encode(q, x, xt, n, ldx, codes, norms, nullptr, (hipStream_t)stream);
}

int tq_encode_prod(const tq_quantizer *q, const void *x, int xt, int64_t n, int64_t ldx, uint8_t *codes,
                   uint16_t *norms, uint16_t *gammas, void *stream) {
  int rc = check_encode(q, x, xt, n, ldx, codes, norms);
  if (rc != TQ_OK) return rc;
  if (q->mode != TQ_PROD) return TQ_ERR_INVALID;
  if (n == 0) return TQ_OK;
  if (!gammas) return TQ_ERR_INVALID;
  return tq::run_encode(q, x, xt, n, ldx, codes, norms, gammas, (hipStream_t)stream);
}

int tq_encode_cache(const tq_quantizer *q, const void *x, int xt, int64_t nseq, int64_t T, int64_t ldx, int64_t t0,
                    int64_t Tstride, int layout, void *codes, uint16_t *norms, uint16_t *gammas, void *stream) {
  if (!q || nseq < 0 || T < 0 || t0 < 0 || Tstride < 0 || !valid_dtype(xt) || ldx < q->d) return TQ_ERR_INVALID;
  if (layout != TQ_LAYOUT_ROWS && layout != TQ_LAYOUT_TILE32) return TQ_ERR_INVALID;
  if (t0 + T > Tstride || (layout == TQ_LAYOUT_TILE32 && t0 % 32 != 0)) return TQ_ERR_INVALID;
  if (nseq == 0 || T == 0) return TQ_OK;
  if (!x || !codes || !norms || (q->mode == TQ_PROD && !gammas)) return TQ_ERR_INVALID;
  if (!aligned16(x) || !aligned16(codes) || (ldx * (int64_t)dtype_size(xt)) % 16 != 0) return TQ_ERR_INVALID;
  if (layout == TQ_LAYOUT_TILE32 && nseq > 65535) return TQ_ERR_UNSUPPORTED;
  return tq::run_encode_cache(q, x, xt, nseq, T, ldx, t0, Tstride, layout, codes, norms,
                              q->mode == TQ_PROD ? gammas : nullptr, (hipStream_t)stream);
}

int tq_decode(const tq_quantizer *q, const uint8_t *codes, const uint16_t *norms, const uint16_t *gammas, int64_t n,
              float *out, int64_t ldo, void *stream) {
  if (!q || n < 0 || ldo < (q ? q->d : 0)) return TQ_ERR_INVALID;
  if (n == 0) return TQ_OK;
  if (!codes || !norms || !out || (q->mode == TQ_PROD && !gammas)) return TQ_ERR_INVALID;
  if (!aligned16(codes) || !aligned16(out) || ldo % 4 != 0) return TQ_ERR_INVALID;
  return tq::run_decode(q, codes, norms, gammas, n, out, ldo, (hipStream_t)stream);
}

size_t tq_score_ws_bytes(const tq_quantizer *q, int64_t m, int64_t n, int k) {
  if (!q || m < 0 || n < 0 || k < 0) return 0;
  return tq::score_ws_bytes(q, m, n, k);
}

int tq_score(const tq_quantizer *q, const float *queries, int64_t m, int64_t ldq, const uint8_t *codes,
             const uint16_t *norms, const uint16_t *gammas, int64_t n, int k, float *scores, int64_t *idx, void *ws,
             size_t ws_bytes, void *stream) {
  if (!q || m < 0 || n < 0 || k < 0 || k > 64 || ldq < q->d) return TQ_ERR_INVALID;
  if (k > 0 && k > n) return TQ_ERR_INVALID;
  if (m == 0 || (n == 0 && k == 0)) return TQ_OK;
  if (!queries || !codes || !norms || !scores || (k > 0 && !idx) || (q->mode == TQ_PROD && !gammas))
    return TQ_ERR_INVALID;
  if (!aligned16(queries) || !aligned16(codes) || ldq % 4 != 0) return TQ_ERR_INVALID;
  size_t need = tq::score_ws_bytes(q, m, n, k);
  if (need > 0 && (!ws || ws_bytes < need)) return TQ_ERR_WORKSPACE;
  return tq::run_score(q, queries, m, ldq, codes, norms, gammas, n, k, scores, idx, ws, ws_bytes,
                       (hipStream_t)stream);
}

size_t tq_attn_decode_ws_bytes(const tq_quantizer *kq, int B, int Hq, int Hkv, int64_t Tstride, int vlayout) {
  if (!kq || B < 0 || Hq <= 0 || Hkv <= 0 || Tstride < 0) return 0;
  if (vlayout != TQ_LAYOUT_ROWS && vlayout != TQ_LAYOUT_TILE32) return 0;
  return tq::attn_ws_bytes(kq, B, Hq, Hkv, Tstride, vlayout);
}

int tq_tile_records(const tq_quantizer *q, const uint8_t *codes, int64_t nseq, int64_t T, uint32_t *tiles,
                    void *stream) {
  if (!q || nseq < 0 || T < 0) return TQ_ERR_INVALID;
  if (nseq == 0 || T == 0) return TQ_OK;
  if (!codes || !tiles || !aligned16(codes) || !aligned16(tiles)) return TQ_ERR_INVALID;
  if (nseq > 65535) return TQ_ERR_UNSUPPORTED;
  return tq::run_tile_records(q, codes, nseq, T, tiles, (hipStream_t)stream);
}

int tq_attn_decode(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq, int Hkv,
                   const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas, const uint8_t *vcodes,
                   const uint16_t *vnorms, const uint16_t *vgammas, int vlayout, int64_t Tstride,
                   const int32_t *seq_len, float scale, float *out, void *ws, size_t ws_bytes, void *stream) {
  return attn_decode_impl(kq, vq, q, qt, B, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, vgammas, vlayout,
                          Tstride, seq_len, scale, out, ws, ws_bytes, nullptr, stream);
}

size_t tq_attn_prefill_ws_bytes(const tq_quantizer *kq, int B, int M, int Hq, int Hkv, int64_t Tstride, int vlayout) {
  if (!kq || B < 0 || M <= 0 || Hq <= 0 || Hkv <= 0 || Tstride < 0) return 0;
  if (vlayout != TQ_LAYOUT_ROWS && vlayout != TQ_LAYOUT_TILE32) return 0;
  if ((int64_t)B * M * Hq > 2147483647 / 2) return 0;
  return tq::attn_prefill_ws_bytes(kq, B, M, Hq, Hkv, Tstride, vlayout);
}

int tq_attn_prefill(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int M, int Hq,
                    int Hkv, const uint8_t *kcodes, const uint16_t *knorms, const uint16_t *kgammas,
                    const uint8_t *vcodes, const uint16_t *vnorms, const uint16_t *vgammas, int vlayout,
                    int64_t Tstride, const int32_t *q_pos, float scale, float *out, void *ws, size_t ws_bytes,
                    void *stream) {
  if (!kq || !vq || vq->mode != TQ_PROD || kq->d != vq->d || kq->device != vq->device) return TQ_ERR_INVALID;
  const bool kprod = kq->mode == TQ_PROD;
  if (B < 0 || M <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Tstride < 0 || !valid_dtype(qt)) return TQ_ERR_INVALID;
  if (vlayout != TQ_LAYOUT_ROWS && vlayout != TQ_LAYOUT_TILE32) return TQ_ERR_INVALID;
  if ((int64_t)B * M * Hq > 2147483647 / 2 || (int64_t)B * M * Hkv * ((Hq / Hkv + 3) / 4) > 2147483647)
    return TQ_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return TQ_ERR_INVALID;
  if (B == 0) return TQ_OK;
  if (!q || !out || !q_pos) return TQ_ERR_INVALID;
  if (Tstride > 0 && (!kcodes || !knorms || !vcodes || !vnorms || !vgammas || (kprod && !kgammas)))
    return TQ_ERR_INVALID;
  if ((Tstride > 0 && (!aligned16(kcodes) || !aligned16(vcodes))) || !aligned16(out) || !aligned16(q))
    return TQ_ERR_INVALID;
  const size_t need = tq::attn_prefill_ws_bytes(kq, B, M, Hq, Hkv, Tstride, vlayout);
  if (need > 0 && (!ws || ws_bytes < need)) return TQ_ERR_WORKSPACE;
  return tq::run_attn_prefill(kq, vq, q, qt, B, M, Hq, Hkv, kcodes, knorms, kprod ? kgammas : nullptr, vcodes, vnorms,
                              vgammas, vlayout, Tstride, q_pos, scale, out, ws, (hipStream_t)stream);
}

int tq_attn_decode_append(const tq_quantizer *kq, const tq_quantizer *vq, const void *q, int qt, int B, int Hq,
                          int Hkv, const void *k_new, const void *v_new, int xt, uint8_t *kcodes, uint16_t *knorms,
                          uint16_t *kgammas, uint8_t *vcodes, uint16_t *vnorms, uint16_t *vgammas, int vlayout,
                          int64_t Tstride, const int32_t *seq_len, float scale, float *out, void *ws,
                          size_t ws_bytes, void *stream) {
  if (!kq || !vq || !valid_dtype(xt)) return TQ_ERR_INVALID;
  if (kq->d > tq::APPEND_DMAX_HOST) return TQ_ERR_UNSUPPORTED;
  if (B > 0 && (Tstride <= 0 || !k_new || !v_new)) return TQ_ERR_INVALID;
  tq::AppendArgs app{};
  app.on = 1;
  app.k_new = k_new;
  app.v_new = v_new;
  app.xt = xt;
  app.d = kq->d;
  app.Hkv = Hkv;
  app.vlayout = vlayout;
  app.Tstride = Tstride;
  app.seq_len = seq_len;
  app.kcodes = kcodes;
  app.knorms = knorms;
  app.kgammas = kgammas;
  app.vcodes = vcodes;
  app.vnorms = vnorms;
  app.vgammas = vgammas;
  auto side = [](const tq_quantizer *z, tq::AppendSide &sd) {
    sd.bm = z->bmse;
    sd.prod = z->mode == TQ_PROD ? 1 : 0;
    sd.piT = z->piT;
    sd.pi = z->pi;
    sd.sT = z->sT;
    for (int k = 0; k < (1 << z->bmse); ++k) sd.c[k] = z->c64[k];
    for (int k = 0; k + 1 < (1 << z->bmse); ++k) sd.t[k] = z->t64[k];
  };
  side(kq, app.k);
  side(vq, app.v);
  return attn_decode_impl(kq, vq, q, qt, B, Hq, Hkv, kcodes, knorms, kgammas, vcodes, vnorms, vgammas, vlayout,
                          Tstride, seq_len, scale, out, ws, ws_bytes, &app, stream);
}

}  // extern "C"
