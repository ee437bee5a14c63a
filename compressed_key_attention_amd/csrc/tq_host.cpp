// Host runtime of libtq: the C ABI, argument validation, the handle's constants
// (seeded Gaussians, Householder QR, Lloyd-Max codebooks) and the device upload.
// Compiled with -ffp-contract=off so that its float64 arithmetic is plain IEEE.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local tq::ProfileEvents g_events;

// The events armed by tq_set_profile_events, handed to one call and then cleared.
tq::ProfileEvents take_events() {
  tq::ProfileEvents e = g_events;
  g_events = tq::ProfileEvents();
  return e;
}

tq_status fail(tq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tq_status ok() {
  g_last_error.clear();
  return TQ_OK;
}

tq_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(TQ_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------------------
// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): word i of stream `seed` is
// mix(seed + (i + 1) * 0x9E3779B97F4A7C15), a counter-based generator.
// ---------------------------------------------------------------------------------------
uint64_t splitmix_word(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// n standard normals: Box-Muller (Box & Muller 1958) on word pairs (2k, 2k+1).
std::vector<double> normals(uint64_t seed, size_t n) {
  std::vector<double> out(n);
  const double two_pi = 6.283185307179586;
  const double inv53 = 1.0 / 9007199254740992.0;  // 2^-53
  for (size_t k = 0; 2 * k < n; ++k) {
    const double u1 = (double)((splitmix_word(seed, 2 * k) >> 11) + 1) * inv53;
    const double u2 = (double)(splitmix_word(seed, 2 * k + 1) >> 11) * inv53;
    const double rad = std::sqrt(-2.0 * std::log(u1));
    const double ang = two_pi * u2;
    out[2 * k] = rad * std::cos(ang);
    if (2 * k + 1 < n) out[2 * k + 1] = rad * std::sin(ang);
  }
  return out;
}

// Random rotation: Q of the Householder QR of the row-major d x d Gaussian G, with
// column j of Q negated when R_jj < 0 (so R = Q^T G has a positive diagonal).
std::vector<float> make_rotation(uint64_t seed, int d) {
  std::vector<double> A = normals(seed, (size_t)d * d);  // overwritten by R
  std::vector<double> V((size_t)d * d, 0.0);              // Householder vectors, column k
  std::vector<double> rdiag(d, 0.0);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += A[(size_t)i * d + k] * A[(size_t)i * d + k];
    const double norm = std::sqrt(norm2);
    if (norm == 0.0) { rdiag[k] = 0.0; continue; }
    const double x0 = A[(size_t)k * d + k];
    const double alpha = x0 >= 0.0 ? -norm : norm;       // avoids cancellation in v0
    double vn2 = 0.0;
    for (int i = k; i < d; ++i) {
      const double vi = A[(size_t)i * d + k] - (i == k ? alpha : 0.0);
      V[(size_t)i * d + k] = vi;
      vn2 += vi * vi;
    }
    const double vn = std::sqrt(vn2);
    for (int i = k; i < d; ++i) V[(size_t)i * d + k] /= vn;
    for (int j = k; j < d; ++j) {          // A[k:, j] -= 2 v (v . A[k:, j])
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += V[(size_t)i * d + k] * A[(size_t)i * d + j];
      for (int i = k; i < d; ++i) A[(size_t)i * d + j] -= 2.0 * dot * V[(size_t)i * d + k];
    }
    rdiag[k] = alpha;
  }
  // Q = H_0 H_1 ... H_{d-1} I, applied from the right-most reflection outwards.
  std::vector<double> Q((size_t)d * d, 0.0);
  for (int i = 0; i < d; ++i) Q[(size_t)i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    if (rdiag[k] == 0.0 && k < d) {
      bool zero = true;
      for (int i = k; i < d; ++i) zero &= V[(size_t)i * d + k] == 0.0;
      if (zero) continue;
    }
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += V[(size_t)i * d + k] * Q[(size_t)i * d + j];
      for (int i = k; i < d; ++i) Q[(size_t)i * d + j] -= 2.0 * dot * V[(size_t)i * d + k];
    }
  }
  std::vector<float> pi((size_t)d * d);
  for (int j = 0; j < d; ++j) {
    const double sgn = rdiag[j] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < d; ++i) pi[(size_t)i * d + j] = (float)(sgn * Q[(size_t)i * d + j]);
  }
  return pi;
}

std::vector<float> make_qjl(uint64_t seed, int m, int d) {
  std::vector<double> g = normals(seed, (size_t)m * d);
  std::vector<float> s(g.size());
  for (size_t i = 0; i < g.size(); ++i) s[i] = (float)g[i];
  return s;
}

// Standard normal: mass and first moment of the cell (lo, hi).  The upper tail uses erfc
// directly so that small tail masses keep their relative accuracy.
void cell(double lo, double hi, double* mass, double* moment) {
  const double r2 = 0.7071067811865476;  // 1/sqrt(2)
  auto upper = [&](double t) {           // P(X > t)
    if (std::isinf(t)) return t > 0 ? 0.0 : 1.0;
    return 0.5 * std::erfc(t * r2);
  };
  auto dens = [](double t) {
    if (std::isinf(t)) return 0.0;
    return std::exp(-0.5 * t * t) * 0.3989422804014327;  // 1/sqrt(2 pi)
  };
  *mass = upper(lo) - upper(hi);
  *moment = dens(lo) - dens(hi);
}

// Lloyd-Max quantizer for N(0,1): alternate midpoint boundaries and conditional-mean
// levels in float64 until the levels move less than 1e-14, keeping the levels exactly
// antisymmetric (the density is symmetric).  Start: levels evenly spaced on [-2, 2].
void lloyd_max(int bits, std::vector<double>* levels, std::vector<double>* bounds) {
  const int L = 1 << bits;
  std::vector<double> lev(L), nxt(L);
  for (int i = 0; i < L; ++i) lev[i] = -2.0 + 4.0 * (i + 0.5) / L;
  for (int i = 0; i < L / 2; ++i) { lev[L - 1 - i] = 0.5 * (lev[L - 1 - i] - lev[i]); lev[i] = -lev[L - 1 - i]; }
  for (int it = 0; it < 20000; ++it) {
    for (int i = 0; i < L; ++i) {
      const double lo = i == 0 ? -INFINITY : 0.5 * (lev[i - 1] + lev[i]);
      const double hi = i == L - 1 ? INFINITY : 0.5 * (lev[i] + lev[i + 1]);
      double mass, mom;
      cell(lo, hi, &mass, &mom);
      nxt[i] = mom / mass;
    }
    double delta = 0.0;
    for (int i = 0; i < L / 2; ++i) {
      const double a = 0.5 * (nxt[L - 1 - i] - nxt[i]);
      delta = std::fmax(delta, std::fabs(a - lev[L - 1 - i]));
      lev[L - 1 - i] = a;
      lev[i] = -a;
    }
    if (delta < 1e-14) break;
  }
  levels->assign(lev.begin(), lev.end());
  bounds->resize(L - 1);
  for (int i = 0; i + 1 < L; ++i) (*bounds)[i] = 0.5 * (lev[i] + lev[i + 1]);
}

// ---------------------------------------------------------------------------------------
// Polar angle grids.  Level 1: uniform on the circle, 2^b cells of width 2 pi / 2^b from -pi,
// reconstruction at the centres.  Level l >= 2: the angle of two child radii over
// n = 2^(l-1) coordinates each has density proportional to sin(2 psi)^(n-1) on [0, pi/2]
// (sin^2 psi ~ Beta(n/2, n/2) for a random direction); its Lloyd-Max grid is iterated in
// float64 with cell masses and first moments from composite 16-point Gauss-Legendre
// quadrature (32 panels per cell), levels kept mirror-symmetric about pi/4.
// ---------------------------------------------------------------------------------------
constexpr double kPi = 3.141592653589793;

struct GaussLegendre16 {
  double x[16], w[16];
  GaussLegendre16() {
    // roots of P_16 by Newton's method from the Chebyshev-like guesses cos(pi (i + 3/4) / (n + 1/2))
    const int n = 16;
    for (int i = 0; i < n; ++i) {
      double z = std::cos(kPi * (i + 0.75) / (n + 0.5)), dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = 0.0;
        for (int j = 1; j <= n; ++j) {   // Bonnet's recurrence
          const double p2 = p1;
          p1 = p0;
          p0 = ((2.0 * j - 1.0) * z * p1 - (j - 1.0) * p2) / j;
        }
        dp = n * (z * p0 - p1) / (z * z - 1.0);
        const double dz = p0 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

void angle_cell(int n, double lo, double hi, double* mass, double* moment) {
  static const GaussLegendre16 gl;
  const int panels = 32;
  const double h = (hi - lo) / panels;
  double m0 = 0.0, m1 = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double a = lo + p * h, half = 0.5 * h, mid = a + half;
    for (int i = 0; i < 16; ++i) {
      const double t = mid + half * gl.x[i];
      const double f = std::pow(std::sin(2.0 * t), n - 1) * gl.w[i] * half;
      m0 += f;
      m1 += t * f;
    }
  }
  *mass = m0;
  *moment = m1;
}

void angle_lloyd_max(int level, int bits, std::vector<double>* levels, std::vector<double>* bounds) {
  const int n = 1 << (level - 1), L = 1 << bits;
  const double half_pi = 0.5 * kPi, quarter = 0.25 * kPi;
  // start: evenly spread over about two standard deviations of the law, sd ~ 1 / (2 sqrt(n - 1))
  const double spread = std::min(0.9 * quarter, 1.0 / std::sqrt((double)(n - 1)));
  std::vector<double> lev(L), nxt(L);
  for (int i = 0; i < L; ++i) lev[i] = quarter + spread * (-1.0 + 2.0 * (i + 0.5) / L);
  for (int it = 0; it < 200000; ++it) {
    for (int i = 0; i < L; ++i) {
      const double lo = i == 0 ? 0.0 : 0.5 * (lev[i - 1] + lev[i]);
      const double hi = i == L - 1 ? half_pi : 0.5 * (lev[i] + lev[i + 1]);
      double mass, mom;
      angle_cell(n, lo, hi, &mass, &mom);
      nxt[i] = mom / mass;
    }
    double delta = 0.0;
    for (int i = 0; i < L; ++i) {
      const double a = 0.5 * (nxt[i] + (half_pi - nxt[L - 1 - i]));
      delta = std::fmax(delta, std::fabs(a - lev[i]));
      lev[i] = a;
    }
    if (delta < 1e-13) break;
  }
  levels->assign(lev.begin(), lev.end());
  bounds->resize(L - 1);
  for (int i = 0; i + 1 < L; ++i) (*bounds)[i] = 0.5 * (lev[i] + lev[i + 1]);
}

// float32 grids of every level: levels[l][16], bounds[l][16] (+inf past the used entries).
// Computed once per (head_dim, b1, bh) and kept for the process.
void polar_grids(int d, int b1, int bh, float (*levels)[16], float (*bounds)[16]) {
  struct Entry { int d, b1, bh; float lv[tq::kMaxPolarLevels][16], bd[tq::kMaxPolarLevels][16]; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  std::lock_guard<std::mutex> lock(mu);
  const Entry* hit = nullptr;
  for (const Entry& e : cache)
    if (e.d == d && e.b1 == b1 && e.bh == bh) hit = &e;
  if (!hit) {
    Entry e;
    e.d = d;
    e.b1 = b1;
    e.bh = bh;
    for (int l = 0; l < tq::kMaxPolarLevels; ++l)
      for (int i = 0; i < 16; ++i) {
        e.lv[l][i] = 0.0f;
        e.bd[l][i] = INFINITY;
      }
    const int L = (int)std::lround(std::log2((double)d));
    const double w = 2.0 * kPi / (1 << b1);
    for (int i = 0; i < (1 << b1); ++i) e.lv[0][i] = (float)(-kPi + (i + 0.5) * w);
    for (int j = 1; j < (1 << b1); ++j) e.bd[0][j - 1] = (float)(-kPi + j * w);
    for (int l = 2; l <= L; ++l) {
      std::vector<double> lv, bd;
      angle_lloyd_max(l, bh, &lv, &bd);
      for (size_t i = 0; i < lv.size(); ++i) e.lv[l - 1][i] = (float)lv[i];
      for (size_t i = 0; i < bd.size(); ++i) e.bd[l - 1][i] = (float)bd[i];
    }
    cache.push_back(e);
    hit = &cache.back();
  }
  std::memcpy(levels, hit->lv, sizeof hit->lv);
  std::memcpy(bounds, hit->bd, sizeof hit->bd);
}

// Scale F for two-limb fixed-point key levels (level ~= round(level * F) / F, |round| <= 32512):
// among F in [F_max / 2, F_max] the one whose products with the float32 levels lie closest
// to integers (worst case over the levels), so integer score products lose the least.
float key_fixed_point_scale(const float* levels, int n) {
  double gmax = 0.0;
  for (int i = 0; i < n; ++i) gmax = std::max(gmax, std::fabs((double)levels[i]));
  if (gmax == 0.0) return 1.0f;
  const double f_max = 32512.0 / gmax;
  const int steps = 1 << 18;
  double best_f = f_max, best_err = INFINITY;
  for (int s = 0; s <= steps; ++s) {
    const double f = (float)(f_max * (0.5 + 0.5 * s / steps));   // candidates exact in float32
    double err = 0.0;
    for (int i = 0; i < n; ++i) {
      const double v = (double)levels[i] * f;
      err = std::max(err, std::fabs(v - std::nearbyint(v)) / f);
    }
    if (err < best_err) {
      best_err = err;
      best_f = f;
    }
  }
  return (float)best_f;
}

tq_status check_config(const tq_config* cfg) {
  if (!cfg) return fail(TQ_ERR_INVALID_ARGUMENT, "config is NULL");
  if (cfg->head_dim <= 0 || cfg->key_bits <= 0 || cfg->value_bits <= 0 || cfg->qjl_dim < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "head_dim, key_bits, value_bits must be > 0, qjl_dim >= 0");
  if (cfg->key_bits > 4 || cfg->value_bits > 4)
    return fail(TQ_ERR_INVALID_ARGUMENT, "key_bits and value_bits must be in 1..4");
  if (cfg->qjl_dim % 32 != 0 || cfg->qjl_dim > 256)
    return fail(TQ_ERR_INVALID_ARGUMENT, "qjl_dim must be 0 or a multiple of 32 up to 256");
  if (cfg->head_dim % 8 != 0 || cfg->head_dim > 256)
    return fail(TQ_ERR_UNSUPPORTED, "head_dim %d not built (a multiple of 8 up to 256)", cfg->head_dim);
  if (cfg->key_codec == TQ_KEY_POLAR && cfg->head_dim != 64 && cfg->head_dim != 128)
    return fail(TQ_ERR_UNSUPPORTED, "polar keys need head_dim 64 or 128");
  if (cfg->key_codec == TQ_KEY_SCALAR) {
    if (cfg->polar_upper_bits != 0)
      return fail(TQ_ERR_INVALID_ARGUMENT, "polar_upper_bits must be 0 for the scalar key codec");
  } else if (cfg->key_codec == TQ_KEY_POLAR) {
    if (cfg->key_bits != 2 && cfg->key_bits != 4)
      return fail(TQ_ERR_UNSUPPORTED, "polar keys: key_bits (level-1 angle bits) must be 2 or 4");
    if (cfg->polar_upper_bits != 1 && cfg->polar_upper_bits != 2 && cfg->polar_upper_bits != 4)
      return fail(TQ_ERR_UNSUPPORTED, "polar keys: polar_upper_bits must be 1, 2 or 4");
  } else {
    return fail(TQ_ERR_INVALID_ARGUMENT, "unknown key_codec %d", cfg->key_codec);
  }
  return TQ_OK;
}

void fill_consts(const tq_config* cfg, tq::Consts* c) {
  std::memset(c, 0, sizeof *c);
  c->d = cfg->head_dim;
  c->kb = cfg->key_bits;
  c->m = cfg->qjl_dim;
  c->vb = cfg->value_bits;
  c->kbytes = (c->d * c->kb / 8 + 3) / 4 * 4;   // fields start on 32-bit words
  if (cfg->key_codec == TQ_KEY_POLAR) {
    c->polar = 1;
    c->pb1 = cfg->key_bits;
    c->pbh = cfg->polar_upper_bits;
    c->plevels = (int)std::lround(std::log2((double)c->d));
    c->l1_bytes = c->d / 2 * c->pb1 / 8;
    c->kbytes = c->l1_bytes + 4 * (((c->d / 2 - 1) * c->pbh + 31) / 32);
  }
  c->sbytes = c->m / 8;
  c->vbytes = (c->d * c->vb / 8 + 3) / 4 * 4;
  c->norm_off = c->kbytes + c->sbytes + c->vbytes;
  c->rec_bytes = (c->norm_off + 12 + 15) / 16 * 16;
  c->sqrt_d = std::sqrt((double)c->d);
  c->inv_sqrt_d = (float)(1.0 / c->sqrt_d);
  c->qjl_coef = c->m ? (float)(std::sqrt(3.141592653589793 / 2.0) / c->m) : 0.0f;
  for (int i = 0; i < tq::kMaxLevels; ++i) c->key_bounds[i] = c->val_bounds[i] = INFINITY;
  std::vector<double> lv, bd;
  lloyd_max(c->kb, &lv, &bd);
  for (size_t i = 0; i < lv.size(); ++i) c->key_levels[i] = (float)lv[i];
  for (size_t i = 0; i < bd.size(); ++i) c->key_bounds[i] = (float)bd[i];
  c->key_fix = key_fixed_point_scale(c->key_levels, 1 << c->kb);
  {
    double gmax = 0.0;
    for (int i = 0; i < (1 << c->kb); ++i) gmax = std::max(gmax, std::fabs((double)c->key_levels[i]));
    c->key_fix3 = gmax > 0.0 ? (float)(8323072.0 / gmax) : 1.0f;
  }
  lloyd_max(c->vb, &lv, &bd);
  for (size_t i = 0; i < lv.size(); ++i) c->val_levels[i] = (float)lv[i];
  for (size_t i = 0; i < bd.size(); ++i) c->val_bounds[i] = (float)bd[i];
}

// MFMA A-operand order used by the compress kernel: entry ((ct * (d/4) + s) * 64 + l)
// holds M[row(ct, l % 16)][(d/4) * (l / 16) + s] with row(ct, i) = (rows/4)(i % 4) + 4 ct + i/4.
std::vector<float> mfma_order(const std::vector<float>& M, int rows, int d) {
  std::vector<float> out((size_t)rows * d);
  const int q = d / 4, rq = rows / 4;
  for (int ct = 0; ct < rows / 16; ++ct)
    for (int s = 0; s < q; ++s)
      for (int l = 0; l < 64; ++l) {
        const int i = l % 16;
        const int row = rq * (i % 4) + 4 * ct + i / 4;
        const int col = q * (l / 16) + s;
        out[((size_t)ct * q + s) * 64 + l] = M[(size_t)row * d + col];
      }
  return out;
}

bool elem_size(tq_dtype dt, size_t* sz) {
  switch (dt) {
    case TQ_F32: *sz = 4; return true;
    case TQ_F16: case TQ_BF16: *sz = 2; return true;
  }
  return false;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

struct tq_handle {
  tq_config cfg;
  tq::Consts c;
  tq::DevConsts dc;
  void* dev_block;
  int device;
};

namespace {

// Calls built for head_dim 64 and 128 only (every other supported head_dim has every call but
// the hot/cold step).
bool dim_unsupported(const tq_handle* h, const char* what, tq_status* st) {
  if (h && h->c.d != 64 && h->c.d != 128) {
    *st = fail(TQ_ERR_UNSUPPORTED, "%s is built for head_dim 64 and 128 only (handle has %d)", what, h->c.d);
    return true;
  }
  return false;
}

// Calls built for the scalar key codec only.
bool polar_unsupported(const tq_handle* h, const char* what, tq_status* st) {
  if (h && h->c.polar) {
    *st = fail(TQ_ERR_UNSUPPORTED, "%s is not built for polar key codes", what);
    return true;
  }
  return false;
}

}  // namespace

extern "C" {

const char* tq_last_error(void) { return g_last_error.c_str(); }

tq_status tq_set_profile_events(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr))
    return fail(TQ_ERR_INVALID_ARGUMENT, "start and stop must both be set or both be NULL");
  g_events.start = start;
  g_events.stop = stop;
  return ok();
}

tq_status tq_monarch_workspace_size(const tq_handle* h, int32_t batch, int32_t q_heads, int32_t kv_heads,
                                    int64_t hot_capacity, int64_t cold_capacity, size_t* bytes) {
  {
    tq_status dst;
    if (dim_unsupported(h, "the hot/cold step", &dst)) return dst;
  }
  if (!h || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL handle or output");
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads || hot_capacity <= 0 || cold_capacity < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "bad hot/cold shape");
  bool okp = false;
  tq::MonarchPlan plan = tq::plan_monarch(h->c, batch, q_heads, kv_heads, hot_capacity, cold_capacity, &okp);
  if (!okp) return fail(TQ_ERR_UNSUPPORTED, "group size %d not supported", q_heads / kv_heads);
  *bytes = plan.ws_total;
  return ok();
}

tq_status tq_monarch_step(const tq_handle* h, const tq_monarch_config* cfg, const tq_monarch_state* st,
                          const void* q, tq_dtype q_dt, int32_t batch, int32_t q_heads, int32_t kv_heads,
                          const void* k_new, const void* v_new, float scale, float* out, float* lse,
                          int32_t* gate_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  {
    tq_status dst;
    if (dim_unsupported(h, "the hot/cold step", &dst)) return dst;
  }
  if (!h || !cfg || !st) return fail(TQ_ERR_INVALID_ARGUMENT, "handle, config or state is NULL");
  size_t es, hs;
  if (!elem_size(q_dt, &es)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown query dtype");
  if (!elem_size(st->hot_dt, &hs)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown hot dtype");
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads)
    return fail(TQ_ERR_INVALID_ARGUMENT, "q_heads must be a positive multiple of kv_heads");
  if (q_heads / kv_heads > 16 || q_heads > 64 || kv_heads > 16)
    return fail(TQ_ERR_UNSUPPORTED,
                "hot/cold step supports up to 16 query heads per KV head, 64 query and 16 KV heads per sequence");
  if (!(scale >= 0.0f) || std::isinf(scale)) return fail(TQ_ERR_INVALID_ARGUMENT, "scale must be finite and >= 0");
  if (cfg->window < 0 || cfg->promote_steps < 0 || std::isnan(cfg->cold_gate))
    return fail(TQ_ERR_INVALID_ARGUMENT, "window and promote_steps must be >= 0, cold_gate not NaN");
  int64_t promote_max = 0;
  if (cfg->promote_steps > 0) {
    if (!(cfg->promote_weight > 0.0f) || std::isinf(cfg->promote_weight))
      return fail(TQ_ERR_INVALID_ARGUMENT, "promote_weight must be > 0 and finite when promotion is on");
    // a head's weights sum to 1, so at most floor(1 / w) of its tokens reach w
    promote_max = (int64_t)std::floor(1.0 / (double)cfg->promote_weight) * q_heads;
    if (promote_max > 1024) return fail(TQ_ERR_UNSUPPORTED, "more than 1024 possible promotions per step");
    promote_max = std::min<int64_t>(promote_max, st->cold_capacity);
  }
  if (st->hot_capacity < (int64_t)cfg->window + 1 + promote_max)
    return fail(TQ_ERR_INVALID_ARGUMENT, "hot_capacity must be >= window + 1 + %lld possible promotions",
                (long long)promote_max);
  if (st->cold_capacity < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "negative cold_capacity");
  if (batch == 0) return ok();
  if (!q || !out || !k_new || !v_new || !st->hot_k || !st->hot_v || !st->hot_start || !st->hot_len ||
      !st->cold_len || !st->hits || !st->overflow || (st->cold_capacity > 0 && !st->records))
    return fail(TQ_ERR_INVALID_ARGUMENT, "NULL input, output or state buffer");
  if (!aligned(st->hot_k, hs * 8) || !aligned(st->hot_v, hs * 8) || !aligned(k_new, hs * 8) ||
      !aligned(v_new, hs * 8))
    return fail(TQ_ERR_INVALID_ARGUMENT, "hot buffers and k_new / v_new must be aligned to 8 elements");
  if (st->records && !aligned(st->records, 16)) return fail(TQ_ERR_INVALID_ARGUMENT, "records not 16-byte aligned");
  bool okp = false;
  tq::MonarchPlan plan = tq::plan_monarch(h->c, batch, q_heads, kv_heads, st->hot_capacity, st->cold_capacity, &okp);
  if (!okp) return fail(TQ_ERR_UNSUPPORTED, "group size %d not supported", q_heads / kv_heads);
  if (!workspace || ws_bytes < plan.ws_total || !aligned(workspace, 256))
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "hot/cold step needs %zu bytes of 256-byte aligned workspace",
                plan.ws_total);
  tq::MonarchStep s;
  s.q = q;
  s.q_dt = q_dt;
  s.k_new = k_new;
  s.v_new = v_new;
  s.hot_k = st->hot_k;
  s.hot_v = st->hot_v;
  s.hot_dt = st->hot_dt;
  s.hot_cap = st->hot_capacity;
  s.cold_cap = st->cold_capacity;
  s.hot_start = st->hot_start;
  s.hot_len = st->hot_len;
  s.records = st->records;
  s.cold_len = st->cold_len;
  s.hits = st->hits;
  s.overflow = st->overflow;
  s.out = out;
  s.lse = lse;
  s.gate_out = gate_out;
  s.batch = batch;
  s.q_heads = q_heads;
  s.kv_heads = kv_heads;
  s.window = cfg->window;
  s.promote_steps = cfg->promote_steps;
  s.cold_gate = cfg->cold_gate;
  s.promote_weight = cfg->promote_weight;
  s.scale = scale;
  return device_status(tq::launch_monarch_step(h->c, h->dc, plan, s, workspace, stream, take_events()),
                       "hot/cold step launch");
}

tq_status tq_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t stream) {
  if (!buf || !sink) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL buffer or sink");
  if (!aligned(buf, 16) || bytes % 16) return fail(TQ_ERR_INVALID_ARGUMENT, "buffer must be 16-byte aligned and sized");
  const int blocks = tq::stream_read_blocks();
  if (sink_words < tq::stream_read_sink_words())
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "sink needs %zu words", tq::stream_read_sink_words());
  return device_status(tq::launch_stream_read(buf, bytes, sink, blocks, stream, take_events()), "stream read launch");
}

tq_status tq_host_constants(const tq_config* cfg, float* pi, float* s, float* key_levels,
                            float* key_bounds, float* value_levels, float* value_bounds) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  tq::Consts c;
  fill_consts(cfg, &c);
  if (pi) {
    std::vector<float> p = make_rotation(cfg->rotation_seed, c.d);
    std::memcpy(pi, p.data(), p.size() * sizeof(float));
  }
  if (s && c.m) {
    std::vector<float> q = make_qjl(cfg->qjl_seed, c.m, c.d);
    std::memcpy(s, q.data(), q.size() * sizeof(float));
  }
  if (key_levels) std::memcpy(key_levels, c.key_levels, sizeof(float) << c.kb);
  if (key_bounds) std::memcpy(key_bounds, c.key_bounds, sizeof(float) * ((1 << c.kb) - 1));
  if (value_levels) std::memcpy(value_levels, c.val_levels, sizeof(float) << c.vb);
  if (value_bounds) std::memcpy(value_bounds, c.val_bounds, sizeof(float) * ((1 << c.vb) - 1));
  return ok();
}

tq_status tq_polar_host_constants(const tq_config* cfg, float* levels, float* bounds) {
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  if (cfg->key_codec != TQ_KEY_POLAR) return fail(TQ_ERR_INVALID_ARGUMENT, "config is not a polar key codec");
  float lv[tq::kMaxPolarLevels][16], bd[tq::kMaxPolarLevels][16];
  polar_grids(cfg->head_dim, cfg->key_bits, cfg->polar_upper_bits, lv, bd);
  const int L = (int)std::lround(std::log2((double)cfg->head_dim));
  for (int l = 0; l < L; ++l) {
    const int bits = l == 0 ? cfg->key_bits : cfg->polar_upper_bits;
    for (int i = 0; i < (1 << bits); ++i)
      if (levels) levels[l * 16 + i] = lv[l][i];
    for (int i = 0; i + 1 < (1 << bits); ++i)
      if (bounds) bounds[l * 16 + i] = bd[l][i];
  }
  return ok();
}

tq_status tq_create(const tq_config* cfg, tq_handle** out) {
  if (!out) return fail(TQ_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  tq_status st = check_config(cfg);
  if (st != TQ_OK) return st;
  tq_handle* h = new (std::nothrow) tq_handle();
  if (!h) return fail(TQ_ERR_OUT_OF_MEMORY, "host allocation failed");
  h->cfg = *cfg;
  fill_consts(cfg, &h->c);
  const int d = h->c.d, m = h->c.m;
  std::vector<float> pi = make_rotation(cfg->rotation_seed, d);
  std::vector<float> s = m ? make_qjl(cfg->qjl_seed, m, d) : std::vector<float>();
  std::vector<float> pi_m = mfma_order(pi, d, d);
  std::vector<float> s_m = m ? mfma_order(s, m, d) : std::vector<float>();
  std::vector<float> pi_t((size_t)d * d);
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) pi_t[(size_t)j * d + i] = pi[(size_t)i * d + j];
  std::vector<float> s_pi((size_t)m * d);
  for (int k = 0; k < m; ++k)
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += (double)s[(size_t)k * d + i] * (double)pi[(size_t)i * d + j];
      s_pi[(size_t)k * d + j] = (float)acc;
    }
  const size_t n_pi = (size_t)d * d, n_s = (size_t)m * d;
  // polar tables: bounds f32 [8][16], cos/sin f64 [8][16][2], cos/sin f32 [8][16][2]
  constexpr size_t kPT = (size_t)tq::kMaxPolarLevels * 16;
  const size_t polar_bytes = h->c.polar ? kPT * 4 + kPT * 16 + kPT * 8 : 0;
  std::vector<float> s_t(n_s);
  for (int k = 0; k < m; ++k)
    for (int i = 0; i < d; ++i) s_t[(size_t)i * m + k] = s[(size_t)k * d + i];
  const size_t main_bytes = (3 * n_pi + 4 * n_s) * sizeof(float);
  const size_t total = main_bytes + polar_bytes;
  if (hipGetDevice(&h->device) != hipSuccess) { delete h; return fail(TQ_ERR_DEVICE, "no HIP device"); }
  {
    // once per device: the address of the allocation-free decode's fixed scratch
    const hipError_t se = tq::scratch_setup();
    if (se != hipSuccess) {
      delete h;
      return device_status(se, "lookup of the fixed device scratch");
    }
  }
  if (hipMalloc(&h->dev_block, total) != hipSuccess) {
    delete h;
    return fail(TQ_ERR_OUT_OF_MEMORY, "hipMalloc of %zu bytes failed", total);
  }
  float* base = (float*)h->dev_block;
  std::vector<float> host;
  host.reserve(total / sizeof(float));
  host.insert(host.end(), pi.begin(), pi.end());
  host.insert(host.end(), pi_m.begin(), pi_m.end());
  host.insert(host.end(), s.begin(), s.end());
  host.insert(host.end(), s_m.begin(), s_m.end());
  host.insert(host.end(), pi_t.begin(), pi_t.end());
  host.insert(host.end(), s_pi.begin(), s_pi.end());
  host.insert(host.end(), s_t.begin(), s_t.end());
  std::vector<uint8_t> ptab(polar_bytes);
  if (h->c.polar) {
    float lv[tq::kMaxPolarLevels][16], bd[tq::kMaxPolarLevels][16];
    polar_grids(d, h->c.pb1, h->c.pbh, lv, bd);
    float* pb = reinterpret_cast<float*>(ptab.data());
    double* c64 = reinterpret_cast<double*>(ptab.data() + kPT * 4);
    float* c32 = reinterpret_cast<float*>(ptab.data() + kPT * 4 + kPT * 16);
    for (size_t i = 0; i < kPT; ++i) {
      pb[i] = bd[i / 16][i % 16];
      const double a = (double)lv[i / 16][i % 16];
      c64[2 * i] = std::cos(a);
      c64[2 * i + 1] = std::sin(a);
      c32[2 * i] = (float)c64[2 * i];
      c32[2 * i + 1] = (float)c64[2 * i + 1];
    }
  }
  hipError_t e = hipMemcpy(base, host.data(), main_bytes, hipMemcpyHostToDevice);
  if (e == hipSuccess && polar_bytes)
    e = hipMemcpy(reinterpret_cast<uint8_t*>(h->dev_block) + main_bytes, ptab.data(), polar_bytes,
                  hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(h->dev_block);
    delete h;
    return device_status(e, "upload of handle constants");
  }
  h->dc.pi = base;
  h->dc.pi_mfma = base + n_pi;
  h->dc.s = m ? base + 2 * n_pi : nullptr;
  h->dc.s_mfma = m ? base + 2 * n_pi + n_s : nullptr;
  h->dc.pi_t = base + 2 * n_pi + 2 * n_s;
  h->dc.s_pi = m ? base + 3 * n_pi + 2 * n_s : nullptr;
  h->dc.s_t = m ? base + 3 * n_pi + 3 * n_s : nullptr;
  h->dc.polar = tq::PolarTables{nullptr, nullptr, nullptr};
  if (h->c.polar) {
    uint8_t* pt = reinterpret_cast<uint8_t*>(h->dev_block) + main_bytes;
    h->dc.polar.bounds = reinterpret_cast<const float*>(pt);
    h->dc.polar.cs64 = reinterpret_cast<const double*>(pt + kPT * 4);
    h->dc.polar.cs32 = reinterpret_cast<const float*>(pt + kPT * 4 + kPT * 16);
  }
  *out = h;
  return ok();
}

tq_status tq_destroy(tq_handle* h) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  hipError_t e = hipFree(h->dev_block);
  delete h;
  return device_status(e, "hipFree");
}

tq_status tq_record_bytes(const tq_handle* h, size_t* record_bytes, size_t* index_record_bytes) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (record_bytes) *record_bytes = (size_t)h->c.rec_bytes;
  if (index_record_bytes) *index_record_bytes = (size_t)h->c.d / 8;
  return ok();
}

static tq_status check_kv_addressing(const tq_handle* h, const void* k, tq_dtype dt, int32_t batch,
                                     int64_t n_tokens, int32_t heads, int64_t seq_stride,
                                     int64_t tok_stride, int64_t head_stride, int64_t capacity,
                                     int64_t first_slot) {
  size_t es;
  if (!elem_size(dt, &es)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
  if (batch < 0 || n_tokens < 0 || heads <= 0) return fail(TQ_ERR_INVALID_ARGUMENT, "bad batch/tokens/heads");
  if (capacity < 0 || first_slot < 0 || first_slot + n_tokens > capacity)
    return fail(TQ_ERR_INVALID_ARGUMENT, "first_slot + n_tokens (%lld) exceeds capacity (%lld)",
                (long long)(first_slot + n_tokens), (long long)capacity);
  if (seq_stride < 0 || tok_stride < 0 || head_stride < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "negative stride");
  if (batch * n_tokens == 0) return TQ_OK;
  if (!k) return fail(TQ_ERR_INVALID_ARGUMENT, "key/value pointer is NULL");
  const size_t a = 16;
  if (!aligned(k, a) || (seq_stride * es) % a || (tok_stride * es) % a || (head_stride * es) % a)
    return fail(TQ_ERR_INVALID_ARGUMENT, "key/value base and strides must be 16-byte aligned");
  (void)h;
  return TQ_OK;
}

tq_status tq_compress_kv(const tq_handle* h, const void* k, const void* v, tq_dtype dt,
                         int32_t batch, int64_t n_tokens, int32_t kv_heads, int64_t seq_stride,
                         int64_t tok_stride, int64_t head_stride, void* records,
                         int64_t capacity, int64_t first_slot, hipStream_t stream) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  tq_status st = check_kv_addressing(h, k, dt, batch, n_tokens, kv_heads, seq_stride, tok_stride,
                                     head_stride, capacity, first_slot);
  if (st != TQ_OK) return st;
  if ((int64_t)batch * n_tokens == 0) return ok();
  st = check_kv_addressing(h, v, dt, batch, n_tokens, kv_heads, seq_stride, tok_stride,
                           head_stride, capacity, first_slot);
  if (st != TQ_OK) return st;
  if (!records || !aligned(records, 16)) return fail(TQ_ERR_INVALID_ARGUMENT, "records NULL or not 16-byte aligned");
  return device_status(tq::launch_compress(h->c, h->dc, k, v, dt, batch, n_tokens, kv_heads,
                                           seq_stride, tok_stride, head_stride, records,
                                           capacity, first_slot, stream, take_events()),
                       "compress launch");
}

tq_status tq_debug_quantize(const tq_handle* h, const float* z_k, const float* p,
                            const float* r_k, const float* rho, const float* z_v,
                            const float* r_v, int64_t n, void* records, hipStream_t stream) {
  {
    tq_status pst;
    if (polar_unsupported(h, "the debug quantize entry", &pst)) return pst;
  }
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (n < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "n < 0");
  if (n == 0) return ok();
  if (!z_k || !r_k || !rho || !z_v || !r_v || !records || (h->c.m && !p))
    return fail(TQ_ERR_INVALID_ARGUMENT, "NULL input");
  if (!aligned(records, 16)) return fail(TQ_ERR_INVALID_ARGUMENT, "records not 16-byte aligned");
  return device_status(tq::launch_debug_quantize(h->c, z_k, p, r_k, rho, z_v, r_v, n, records, stream),
                       "debug quantize launch");
}

tq_status tq_decode_workspace_size(const tq_handle* h, int32_t batch, int32_t q_heads,
                                   int32_t kv_heads, int64_t capacity, int32_t k_sel,
                                   size_t* bytes) {
  if (!h || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL handle or output");
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads || capacity < 0 || k_sel < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "bad decode shape");
  tq::DecodePlan plan;
  if (!tq::plan_decode(h->c, batch, q_heads, kv_heads, k_sel > 0 ? k_sel : capacity, &plan))
    return fail(TQ_ERR_UNSUPPORTED, "group size %d not supported", q_heads / kv_heads);
  *bytes = plan.ws_total;
  return ok();
}

// Checks shared by the two decode entry points; fills the plan.
static tq_status check_decode(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                              int32_t q_heads, int32_t kv_heads, const void* records,
                              int64_t capacity, const int32_t* seq_lens, const void* hot_k,
                              const void* hot_v, tq_dtype hot_dt, const int32_t* hot_lens,
                              int64_t hot_capacity, const int32_t* sel_idx, int32_t k_sel,
                              float scale, float* out, tq::DecodePlan* plan) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  size_t es;
  if (!elem_size(q_dt, &es)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown query dtype");
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads)
    return fail(TQ_ERR_INVALID_ARGUMENT, "q_heads must be a positive multiple of kv_heads");
  if (capacity < 0 || k_sel < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "negative capacity or k_sel");
  if (!(scale >= 0.0f) || std::isinf(scale)) return fail(TQ_ERR_INVALID_ARGUMENT, "scale must be finite and >= 0");
  if (batch == 0) return ok();
  if (!q || !out || !seq_lens) return fail(TQ_ERR_INVALID_ARGUMENT, "q, out and seq_lens are required");
  if (capacity > 0 && !records) return fail(TQ_ERR_INVALID_ARGUMENT, "records is NULL");
  if (records && !aligned(records, 16)) return fail(TQ_ERR_INVALID_ARGUMENT, "records not 16-byte aligned");
  if (sel_idx && k_sel == 0) return fail(TQ_ERR_INVALID_ARGUMENT, "gather mode needs k_sel > 0");
  if (hot_lens) {
    size_t hs;
    if (!elem_size(hot_dt, &hs)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown hot dtype");
    if (hot_capacity <= 0 || !hot_k || !hot_v)
      return fail(TQ_ERR_INVALID_ARGUMENT, "exact segment needs hot_k, hot_v and hot_capacity > 0");
    if (!aligned(hot_k, hs * 8) || !aligned(hot_v, hs * 8))
      return fail(TQ_ERR_INVALID_ARGUMENT, "hot_k and hot_v must be aligned to 8 elements");
  }
  if (!tq::plan_decode(h->c, batch, q_heads, kv_heads, sel_idx ? k_sel : capacity, plan))
    return fail(TQ_ERR_UNSUPPORTED, "group size %d not supported", q_heads / kv_heads);
  return ok();
}

tq_status tq_decode_attention(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                              int32_t q_heads, int32_t kv_heads, const void* records,
                              int64_t capacity, const int32_t* seq_lens, const void* hot_k,
                              const void* hot_v, tq_dtype hot_dt, const int32_t* hot_lens,
                              int64_t hot_capacity, const int32_t* sel_idx, int32_t k_sel,
                              float scale, float* out, float* lse, float* logits,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  tq::DecodePlan plan;
  const tq_status st = check_decode(h, q, q_dt, batch, q_heads, kv_heads, records, capacity, seq_lens, hot_k,
                                    hot_v, hot_dt, hot_lens, hot_capacity, sel_idx, k_sel, scale, out, &plan);
  if (st != TQ_OK || batch == 0) return st;
  if (!workspace || ws_bytes < plan.ws_total || !aligned(workspace, 256))
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu bytes of 256-byte aligned workspace",
                plan.ws_total);
  return device_status(tq::launch_decode(h->c, h->dc, plan, q, q_dt, batch, q_heads, kv_heads,
                                         records, capacity, seq_lens, hot_k, hot_v, hot_dt,
                                         hot_lens, hot_capacity, sel_idx, k_sel, scale, out, lse,
                                         logits, workspace, stream, take_events()),
                       "decode launch");
}

tq_status tq_decode_attention_noalloc(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                                      int32_t q_heads, int32_t kv_heads, const void* records,
                                      int64_t capacity, const int32_t* seq_lens, const void* hot_k,
                                      const void* hot_v, tq_dtype hot_dt, const int32_t* hot_lens,
                                      int64_t hot_capacity, const int32_t* sel_idx, int32_t k_sel,
                                      float scale, float* out, float* lse, float* logits,
                                      hipStream_t stream) {
  tq::DecodePlan plan;
  const tq_status st = check_decode(h, q, q_dt, batch, q_heads, kv_heads, records, capacity, seq_lens, hot_k,
                                    hot_v, hot_dt, hot_lens, hot_capacity, sel_idx, k_sel, scale, out, &plan);
  if (st != TQ_OK || batch == 0) return st;
  if (plan.ws_total > tq::kScratchBytes)
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL,
                "this decode needs %zu bytes of scratch; the fixed device scratch holds %zu "
                "(use tq_decode_attention with a workspace)", plan.ws_total, tq::kScratchBytes);
  void* ws = tq::scratch_address(h->device);
  if (!ws) return fail(TQ_ERR_DEVICE, "the fixed device scratch is not set up on device %d", h->device);
  return device_status(tq::launch_decode(h->c, h->dc, plan, q, q_dt, batch, q_heads, kv_heads,
                                         records, capacity, seq_lens, hot_k, hot_v, hot_dt,
                                         hot_lens, hot_capacity, sel_idx, k_sel, scale, out, lse,
                                         logits, ws, stream, take_events()),
                       "decode launch");
}

tq_status tq_index_workspace_size(const tq_handle* h, int32_t batch, int32_t kv_heads,
                                  size_t* bytes) {
  if (!h || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL handle or output");
  if (batch < 0 || kv_heads <= 0) return fail(TQ_ERR_INVALID_ARGUMENT, "bad shape");
  // worst case over n_tokens: the plan caps the number of chunks
  *bytes = tq::plan_index(h->c, batch, kv_heads, (int64_t)1 << 40).ws_total;
  return ok();
}

tq_status tq_build_sign_index(const tq_handle* h, const void* k, tq_dtype dt, int32_t batch,
                              int64_t n_tokens, int32_t kv_heads, int64_t seq_stride,
                              int64_t tok_stride, int64_t head_stride, void* index,
                              float* codebook, float* mean, int64_t capacity,
                              int64_t first_slot, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  tq_status st = check_kv_addressing(h, k, dt, batch, n_tokens, kv_heads, seq_stride, tok_stride,
                                     head_stride, capacity, first_slot);
  if (st != TQ_OK) return st;
  if (batch == 0) return ok();
  if (!index || !codebook) return fail(TQ_ERR_INVALID_ARGUMENT, "index and codebook are required");
  tq::IndexPlan plan = tq::plan_index(h->c, batch, kv_heads, n_tokens);
  if (!workspace || ws_bytes < plan.ws_total || !aligned(workspace, 256))
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "sign index needs %zu bytes of workspace", plan.ws_total);
  return device_status(tq::launch_sign_index(h->c, plan, k, dt, batch, n_tokens, kv_heads,
                                             seq_stride, tok_stride, head_stride, index, codebook,
                                             mean, capacity, first_slot, workspace, stream),
                       "sign index launch");
}

tq_status tq_select_workspace_size(const tq_handle* h, int32_t batch, int32_t kv_heads,
                                   int64_t capacity, size_t* bytes) {
  if (!h || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL handle or output");
  if (batch < 0 || kv_heads <= 0 || capacity < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "bad shape");
  *bytes = tq::plan_select(h->c, batch, kv_heads, capacity).ws_total;
  return ok();
}

tq_status tq_select_topk(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                         int32_t q_heads, int32_t kv_heads, const void* index,
                         const float* codebook, int64_t capacity, const int32_t* seq_lens,
                         int32_t k, int32_t* out_idx, int32_t* out_count, int32_t* out_scores,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  size_t es;
  if (!elem_size(q_dt, &es)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown query dtype");
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads || capacity < 0 || k < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "bad select shape");
  if (q_heads / kv_heads > 16) return fail(TQ_ERR_UNSUPPORTED, "group size above 16");
  if (capacity > (int64_t(1) << 26)) return fail(TQ_ERR_UNSUPPORTED, "select capacity above 2^26 tokens");
  if (batch == 0) return ok();
  if (!q || !seq_lens || !out_count || (k > 0 && !out_idx) || (capacity > 0 && (!index || !codebook)))
    return fail(TQ_ERR_INVALID_ARGUMENT, "NULL input or output");
  tq::SelectPlan plan = tq::plan_select(h->c, batch, kv_heads, capacity);
  if (!workspace || ws_bytes < plan.ws_total || !aligned(workspace, 256))
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "select needs %zu bytes of workspace", plan.ws_total);
  return device_status(tq::launch_select(h->c, plan, q, q_dt, batch, q_heads, kv_heads, index,
                                         codebook, capacity, seq_lens, k, out_idx, out_count,
                                         out_scores, workspace, stream, take_events()),
                       "select launch");
}

tq_status tq_sparse_workspace_size(const tq_handle* h, int32_t batch, int32_t q_heads,
                                   int32_t kv_heads, int64_t capacity, size_t* bytes) {
  if (!h || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL handle or output");
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads || capacity < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "bad shape");
  *bytes = tq::plan_sparse(h->c, batch, q_heads, kv_heads, capacity).ws_total;
  return ok();
}

tq_status tq_sparse_attention(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                              int32_t q_heads, int32_t kv_heads, const void* index,
                              const float* codebook, const void* records, int64_t capacity,
                              const int32_t* seq_lens, int32_t k, const void* hot_k,
                              const void* hot_v, tq_dtype hot_dt, const int32_t* hot_lens,
                              int64_t hot_capacity, float scale, float* out, float* lse,
                              void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  size_t es;
  if (!elem_size(q_dt, &es)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown query dtype");
  if (batch < 0 || q_heads <= 0 || kv_heads <= 0 || q_heads % kv_heads || capacity < 0 || k < 0)
    return fail(TQ_ERR_INVALID_ARGUMENT, "bad sparse attention shape");
  if (q_heads / kv_heads > 16) return fail(TQ_ERR_UNSUPPORTED, "group size above 16");
  const int max_m = (h->c.d == 64 || h->c.d == 128) ? 128 : 256;
  if (h->c.m > max_m || h->c.m % 32)
    return fail(TQ_ERR_UNSUPPORTED, "qjl_dim must be a multiple of 32 up to %d at head_dim %d", max_m, h->c.d);
  if (capacity > (int64_t(1) << 26)) return fail(TQ_ERR_UNSUPPORTED, "capacity above 2^26 tokens");
  if (!(scale >= 0.0f) || std::isinf(scale)) return fail(TQ_ERR_INVALID_ARGUMENT, "scale must be finite and >= 0");
  if (batch == 0) return ok();
  if (!q || !out || !seq_lens) return fail(TQ_ERR_INVALID_ARGUMENT, "q, out and seq_lens are required");
  if (capacity > 0 && (!index || !codebook || !records))
    return fail(TQ_ERR_INVALID_ARGUMENT, "index, codebook and records are required");
  if (records && !aligned(records, 16)) return fail(TQ_ERR_INVALID_ARGUMENT, "records not 16-byte aligned");
  if (hot_lens) {
    size_t hs;
    if (!elem_size(hot_dt, &hs)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown hot dtype");
    if (hot_capacity <= 0 || !hot_k || !hot_v)
      return fail(TQ_ERR_INVALID_ARGUMENT, "exact segment needs hot_k, hot_v and hot_capacity > 0");
    if (!aligned(hot_k, hs * 8) || !aligned(hot_v, hs * 8))
      return fail(TQ_ERR_INVALID_ARGUMENT, "hot_k and hot_v must be aligned to 8 elements");
  }
  tq::SparsePlan plan = tq::plan_sparse(h->c, batch, q_heads, kv_heads, capacity);
  if (!workspace || ws_bytes < plan.ws_total || !aligned(workspace, 256))
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "sparse attention needs %zu bytes of 256-byte aligned workspace",
                plan.ws_total);
  return device_status(tq::launch_sparse(h->c, h->dc, plan, q, q_dt, batch, q_heads, kv_heads, index,
                                         codebook, records, capacity, seq_lens, k, hot_k, hot_v, hot_dt,
                                         hot_lens, hot_capacity, scale, out, lse, workspace, stream,
                                         take_events()),
                       "sparse attention launch");
}

tq_status tq_scan_workspace_size(const tq_handle* h, int32_t batch, int32_t kv_heads,
                                 int32_t n_queries, size_t* bytes) {
  if (!h || !bytes) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL handle or output");
  if (batch < 0 || kv_heads <= 0 || n_queries < 0) return fail(TQ_ERR_INVALID_ARGUMENT, "bad shape");
  *bytes = tq::plan_scan(h->c, batch, kv_heads, n_queries).ws_total;
  return ok();
}

tq_status tq_score_scan(const tq_handle* h, const void* q, tq_dtype q_dt, int32_t batch,
                        int32_t kv_heads, int32_t n_queries, const void* records,
                        int64_t capacity, int64_t n_tokens, float* scores, void* workspace,
                        size_t ws_bytes, hipStream_t stream) {
  if (!h) return fail(TQ_ERR_INVALID_ARGUMENT, "handle is NULL");
  size_t es;
  if (!elem_size(q_dt, &es)) return fail(TQ_ERR_INVALID_ARGUMENT, "unknown query dtype");
  if (batch < 0 || kv_heads <= 0 || n_queries < 0 || n_tokens < 0 || n_tokens > capacity)
    return fail(TQ_ERR_INVALID_ARGUMENT, "bad scan shape (n_tokens must be <= capacity)");
  if ((int64_t)batch * n_queries * n_tokens == 0) return ok();
  if (!q || !records || !scores) return fail(TQ_ERR_INVALID_ARGUMENT, "NULL input or output");
  if (!aligned(records, 16)) return fail(TQ_ERR_INVALID_ARGUMENT, "records not 16-byte aligned");
  tq::ScanPlan plan = tq::plan_scan(h->c, batch, kv_heads, n_queries);
  if (!workspace || ws_bytes < plan.ws_total || !aligned(workspace, 256))
    return fail(TQ_ERR_WORKSPACE_TOO_SMALL, "scan needs %zu bytes of workspace", plan.ws_total);
  return device_status(tq::launch_scan(h->c, h->dc, plan, q, q_dt, batch, kv_heads, n_queries,
                                       records, capacity, n_tokens, scores, workspace, stream,
                                       take_events()),
                       "scan launch");
}

}  // extern "C"
