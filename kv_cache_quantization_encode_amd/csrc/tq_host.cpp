// Host side of libtq: argument validation helpers and the seed-derived tables
// (Lloyd-Max codebook, random signs, QJL matrix, bucketize hint grid).
//
// Codebook: the "tqlite" README (三种量化模式: rotation + Lloyd-Max codebook)
// and the validation script's get_codebook(d, bits)["mse_total"]
// (test_mse_codebook_table1).  The quantiser is the MSE-optimal one for
// N(0,1): boundaries at midpoints of neighbouring centroids, each centroid the
// conditional mean of its cell.  It is solved here in double precision by a
// short run of Lloyd steps followed by Newton's method on c = lloyd(c) with
// the tridiagonal Jacobian of the Lloyd map, keeping c antisymmetric.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "tq.h"
#include "tq_internal.h"
#include "tq_tables.h"

extern "C" const char* tq_status_string(int32_t s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_WORKSPACE: return "workspace missing or too small";
    case TQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

namespace tq {

int index_width(int bits) {
  if (bits == 1) return 1;
  if (bits == 2) return 2;
  if (bits == 3 || bits == 4) return 4;
  if (bits >= 5 && bits <= 8) return 8;
  return 0;
}

tq_status describe(const tq_key_config* cfg, Parts* p) {
  if (!cfg || !p) return TQ_ERR_ARG;
  const int d = cfg->d;
  if (d < 16 || d > 256 || (d & (d - 1))) return TQ_ERR_ARG;
  const bool grouped = cfg->mode == TQ_MODE_GROUPED || cfg->mode == TQ_MODE_GROUPED_PROD;
  if (!grouped && cfg->d_outlier != 0) return TQ_ERR_ARG;
  if (grouped && cfg->d_outlier != 0 && cfg->d_outlier != d / 2) {
    // only the even split gives two power-of-two halves
    return cfg->d_outlier > 0 && cfg->d_outlier < d ? TQ_ERR_UNSUPPORTED : TQ_ERR_ARG;
  }
  memset(p, 0, sizeof(*p));
  p->d = d;
  p->mode = cfg->mode;
  switch (cfg->mode) {
    case TQ_MODE_MSE:
      if (cfg->bits < 1 || cfg->bits > 8) return TQ_ERR_ARG;
      p->n_parts = 1;
      p->part_d[0] = d;
      p->part_bits[0] = cfg->bits;
      break;
    case TQ_MODE_PROD:
      if (cfg->bits < 2 || cfg->bits > 9) return TQ_ERR_ARG;
      p->n_parts = 1;
      p->part_d[0] = d;
      p->part_bits[0] = cfg->bits - 1;
      p->m = d;
      break;
    case TQ_MODE_GROUPED:
    case TQ_MODE_GROUPED_PROD:
      if (cfg->bits_outlier < 1 || cfg->bits_outlier > 8) return TQ_ERR_ARG;
      if (cfg->bits_normal < 1 || cfg->bits_normal > 8) return TQ_ERR_ARG;
      p->n_parts = 2;
      p->part_d[0] = p->part_d[1] = d / 2;
      p->part_bits[0] = cfg->bits_outlier;
      p->part_bits[1] = cfg->bits_normal;
      if (cfg->mode == TQ_MODE_GROUPED_PROD) p->m = d;
      break;
    default:
      return TQ_ERR_ARG;
  }
  size_t row = 0;
  for (int i = 0; i < p->n_parts; ++i) {
    p->part_width[i] = index_width(p->part_bits[i]);
    p->part_row_off[i] = (int)row;
    row += (size_t)p->part_d[i] * p->part_width[i] / 8;
  }
  p->idx_row_bytes = (int)row;
  return TQ_OK;
}

int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < 64) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace tq

extern "C" size_t tq_idx_row_bytes(const tq_key_config* cfg) {
  tq::Parts p;
  if (tq::describe(cfg, &p) != TQ_OK) return 0;
  return (size_t)p.idx_row_bytes;
}

namespace {

// ---- SplitMix64 (Steele, Lea & Flood 2014): output i of the stream started at
// state s0 is mix(s0 + (i+1) * gamma).
const uint64_t kGamma = 0x9E3779B97F4A7C15ull;

uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct Stream {
  uint64_t s;
  Stream(uint64_t seed, uint64_t tag) : s(seed ^ (tag * kGamma)) {}
  uint64_t next() {
    s += kGamma;
    return mix64(s);
  }
};

// ---- fp16 rounding from double, round to nearest even, written out on the
// bit level so that it does not depend on the compiler's conversion.
uint16_t f64_to_f16_bits(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return 0x7E00u;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (a >= 65520.0) return sign | 0x7C00u;  // at or past the midpoint to 2^16
  int e2;
  frexp(a, &e2);
  int E = e2 - 1;                            // a in [2^E, 2^(E+1))
  int qexp = (E < -14) ? -24 : E - 10;       // spacing of fp16 values near a
  double r = nearbyint(ldexp(a, -qexp));     // exact scaling, then RNE
  uint32_t rr = (uint32_t)r;
  if (E < -14) return sign | (uint16_t)rr;   // subnormal (1024 carries to the min normal)
  if (rr == 2048u) {
    rr = 1024u;
    ++E;
  }
  if (E + 15 >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)(((uint32_t)(E + 15) << 10) | (rr - 1024u));
}

// ---- standard normal helpers
const double kInvSqrt2Pi = 0.39894228040143267794;
const double kSqrtHalf = 0.70710678118654752440;

double pdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) * kInvSqrt2Pi; }

// P(a <= X < b), taken on the side of zero that avoids cancellation.
double cell_prob(double a, double b) {
  if (a >= 0) return 0.5 * (erfc(a * kSqrtHalf) - erfc(b * kSqrtHalf));
  return 0.5 * (erfc(-b * kSqrtHalf) - erfc(-a * kSqrtHalf));
}

double inv_cdf(double p) {  // bisection, only used for the starting point
  double lo = -40, hi = 40;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (0.5 * erfc(-mid * kSqrtHalf) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

struct Cells {
  std::vector<double> lo, hi, p, g;
};

void lloyd_eval(const std::vector<double>& c, Cells* s) {
  const int L = (int)c.size();
  s->lo.resize(L); s->hi.resize(L); s->p.resize(L); s->g.resize(L);
  for (int k = 0; k < L; ++k) {
    s->lo[k] = k == 0 ? -INFINITY : 0.5 * (c[k - 1] + c[k]);
    s->hi[k] = k == L - 1 ? INFINITY : 0.5 * (c[k] + c[k + 1]);
    s->p[k] = cell_prob(s->lo[k], s->hi[k]);
    s->g[k] = (pdf(s->lo[k]) - pdf(s->hi[k])) / s->p[k];
  }
}

void antisymmetrize(std::vector<double>* c) {
  const int L = (int)c->size();
  for (int k = 0; k < L / 2; ++k) {
    double v = 0.5 * ((*c)[L - 1 - k] - (*c)[k]);
    (*c)[k] = -v;
    (*c)[L - 1 - k] = v;
  }
}

// Lloyd-Max quantiser of N(0,1) with L levels; returns distortion D.
double lloyd_max(int L, std::vector<double>* c_out, std::vector<double>* t_out) {
  std::vector<double> c(L);
  for (int k = 0; k < L; ++k) c[k] = sqrt(3.0) * inv_cdf((k + 0.5) / L);
  antisymmetrize(&c);
  Cells s;
  for (int it = 0; it < 200; ++it) {
    lloyd_eval(c, &s);
    c = s.g;
    antisymmetrize(&c);
  }
  std::vector<double> sub(L), dia(L), sup(L), rhs(L);
  for (int it = 0; it < 60; ++it) {
    lloyd_eval(c, &s);
    for (int k = 0; k < L; ++k) {
      double dlo = isinf(s.lo[k]) ? 0.0 : pdf(s.lo[k]) * (s.g[k] - s.lo[k]) / s.p[k];
      double dhi = isinf(s.hi[k]) ? 0.0 : pdf(s.hi[k]) * (s.hi[k] - s.g[k]) / s.p[k];
      // (I - J) step = c - g, J the Jacobian of the Lloyd map (tridiagonal)
      sub[k] = -0.5 * dlo;
      sup[k] = -0.5 * dhi;
      dia[k] = 1.0 - 0.5 * (dlo + dhi);
      rhs[k] = c[k] - s.g[k];
    }
    // Thomas algorithm
    for (int k = 1; k < L; ++k) {
      double w = sub[k] / dia[k - 1];
      dia[k] -= w * sup[k - 1];
      rhs[k] -= w * rhs[k - 1];
    }
    std::vector<double> step(L);
    step[L - 1] = rhs[L - 1] / dia[L - 1];
    for (int k = L - 2; k >= 0; --k) step[k] = (rhs[k] - sup[k] * step[k + 1]) / dia[k];
    double mx = 0;
    for (int k = 0; k < L; ++k) {
      c[k] -= step[k];
      mx = fmax(mx, fabs(step[k]));
    }
    antisymmetrize(&c);
    if (mx <= 1e-15) break;
  }
  std::vector<double> t(L - 1);
  for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
  t[L / 2 - 1] = 0.0;
  // distortion: sum over cells of int (x - c)^2 phi, with
  // int x^2 phi = P - [x phi]_a^b and int x phi = phi(a) - phi(b)
  double D = 0;
  for (int k = 0; k < L; ++k) {
    double a = k == 0 ? -INFINITY : t[k - 1];
    double b = k == L - 1 ? INFINITY : t[k];
    double P = cell_prob(a, b);
    double xa = isinf(a) ? 0.0 : a * pdf(a);
    double xb = isinf(b) ? 0.0 : b * pdf(b);
    double m2 = P - (xb - xa);
    double m1 = pdf(a) - pdf(b);
    D += m2 - 2 * c[k] * m1 + c[k] * c[k] * P;
  }
  *c_out = c;
  *t_out = t;
  return D;
}

// Bucketize hint grid over [t_0 - 1, t_last + 1].
bool build_hint(const std::vector<float>& t, std::vector<tq_hint>* out, float* lo_out,
                float* scale_out) {
  const int nb = (int)t.size();  // boundaries
  const double lo = (double)t[0] - 1.0, hi = (double)t[nb - 1] + 1.0;
  auto bound = [&](int k) -> float { return k < nb ? t[k] : INFINITY; };
  for (int G = 16; G <= TQ_MAX_HINT; G *= 2) {
    const double scale = (double)(float)(G / (hi - lo));
    const double w = 1.0 / scale, margin = 0.01 * w;
    std::vector<tq_hint> h(G);
    bool ok = true;
    for (int g = 0; g < G && ok; ++g) {
      double b0 = (double)(float)lo + g * w, b1 = b0 + w;
      int below = 0;
      while (below < nb && (double)t[below] < b0 - margin) ++below;
      int upto = 0;
      while (upto < nb && (double)t[upto] <= b1 + margin) ++upto;
      if (g == G - 1) upto = nb;  // the last bin also takes every y beyond it
      if (g == 0) below = 0;      // the first bin also takes every y below it
      if (upto - below > 2) ok = false;
      h[g].h = below;
      h[g].t_h = bound(below);
      h[g].t_h1 = bound(below + 1);
      h[g].pad = 0;
    }
    if (ok) {
      *out = h;
      *lo_out = (float)lo;
      *scale_out = (float)scale;
      return true;
    }
  }
  return false;
}

size_t align_up(size_t x) { return (x + TQ_BLOB_ALIGN - 1) / TQ_BLOB_ALIGN * TQ_BLOB_ALIGN; }

}  // namespace

extern "C" tq_status tq_build_codebook(const tq_key_config* cfg, void* blob_host, size_t* bytes,
                                       double* mse_total_host) {
  tq::Parts P;
  tq_status st = tq::describe(cfg, &P);
  if (st != TQ_OK) return st;
  if (!bytes) return TQ_ERR_ARG;

  std::vector<double> cd[TQ_MAX_PARTS], td[TQ_MAX_PARTS];
  std::vector<float> cf[TQ_MAX_PARTS], tf[TQ_MAX_PARTS];
  std::vector<tq_hint> hint[TQ_MAX_PARTS];
  float hlo[TQ_MAX_PARTS] = {0, 0}, hsc[TQ_MAX_PARTS] = {0, 0};
  double D[TQ_MAX_PARTS] = {0, 0};
  for (int i = 0; i < P.n_parts; ++i) {
    const int L = 1 << P.part_bits[i];
    D[i] = lloyd_max(L, &cd[i], &td[i]);
    cf[i].resize(L);
    tf[i].resize(L - 1);
    for (int k = 0; k < L; ++k) cf[i][k] = (float)cd[i][k];
    for (int k = 0; k + 1 < L; ++k) tf[i][k] = (float)td[i][k];
    if (!build_hint(tf[i], &hint[i], &hlo[i], &hsc[i])) return TQ_ERR_UNSUPPORTED;
  }

  tq_blob_header H;
  memset(&H, 0, sizeof(H));
  size_t off = align_up(sizeof(tq_blob_header));
  H.header_bytes = (uint32_t)off;
  for (int i = 0; i < P.n_parts; ++i) {
    const int L = 1 << P.part_bits[i];
    H.part_d[i] = P.part_d[i];
    H.part_bits[i] = P.part_bits[i];
    H.part_levels[i] = L;
    H.off_centroids[i] = (uint32_t)off; off = align_up(off + sizeof(float) * L);
    H.off_bounds[i] = (uint32_t)off;    off = align_up(off + sizeof(float) * (L + 1));
    H.off_sigma[i] = (uint32_t)off;     off = align_up(off + sizeof(float) * P.part_d[i]);
    H.off_hint[i] = (uint32_t)off;      off = align_up(off + sizeof(tq_hint) * hint[i].size());
    H.hint_n[i] = (int32_t)hint[i].size();
    H.hint_lo[i] = hlo[i];
    H.hint_scale[i] = hsc[i];
    H.mse[i] = D[i];
  }
  if (P.m > 0) {
    H.off_S = (uint32_t)off;
    off = align_up(off + sizeof(uint16_t) * (size_t)P.m * P.d);
  }
  H.magic = TQ_BLOB_MAGIC;
  H.version = TQ_BLOB_VERSION;
  H.total_bytes = (uint32_t)off;
  H.d = P.d;
  H.mode = P.mode;
  H.m = P.m;
  H.n_parts = P.n_parts;

  if (mse_total_host)
    for (int i = 0; i < P.n_parts; ++i) mse_total_host[i] = D[i];
  if (!blob_host) {
    *bytes = off;
    return TQ_OK;
  }
  if (*bytes < off) {
    *bytes = off;
    return TQ_ERR_ARG;
  }
  *bytes = off;
  unsigned char* b = (unsigned char*)blob_host;
  memset(b, 0, off);
  memcpy(b, &H, sizeof(H));
  for (int i = 0; i < P.n_parts; ++i) {
    const int L = 1 << P.part_bits[i];
    memcpy(b + H.off_centroids[i], cf[i].data(), sizeof(float) * L);
    float* bd = (float*)(b + H.off_bounds[i]);
    for (int k = 0; k + 1 < L; ++k) bd[k] = tf[i][k];
    bd[L - 1] = INFINITY;
    bd[L] = INFINITY;
    // sigma_j = +1 if the top bit of output j is 0, else -1
    const uint64_t tag = P.n_parts == 2 ? (i == 0 ? 3 : 4) : 1;
    Stream sg(cfg->seed, tag);
    float* sig = (float*)(b + H.off_sigma[i]);
    for (int j = 0; j < P.part_d[i]; ++j) sig[j] = (sg.next() >> 63) ? -1.0f : 1.0f;
    memcpy(b + H.off_hint[i], hint[i].data(), sizeof(tq_hint) * hint[i].size());
  }
  if (P.m > 0) {
    // S: m x d i.i.d. N(0,1) by Box-Muller on consecutive outputs, each value
    // rounded to fp16.  u1 in (0,1], u2 in [0,1) from the top 53 bits.
    Stream ss(cfg->seed, 2);
    uint16_t* S = (uint16_t*)(b + H.off_S);
    const size_t n = (size_t)P.m * P.d;
    const double two_pi = 6.283185307179586;
    for (size_t k = 0; k < n; k += 2) {
      double u1 = (double)((ss.next() >> 11) + 1) * 0x1.0p-53;
      double u2 = (double)(ss.next() >> 11) * 0x1.0p-53;
      double r = sqrt(-2.0 * log(u1));
      S[k] = f64_to_f16_bits(r * cos(two_pi * u2));
      if (k + 1 < n) S[k + 1] = f64_to_f16_bits(r * sin(two_pi * u2));
    }
  }
  return TQ_OK;
}
