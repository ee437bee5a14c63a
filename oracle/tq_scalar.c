/* Scalar C oracle of the compressed-key attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py load this library (through oracle/scalar.py).  The product
 * path never links, loads or calls it, and it shares no source, table or constant generator
 * with the HIP library.  It is a second, independent statement of the same definition as
 * oracle/tq_oracle.py, written as plain loops in C99 (no SIMD intrinsics, no BLAS), built
 * with -O2 -ffp-contract=off -fno-fast-math, accumulating in double.
 *
 * What it follows (page title, section):
 *  - TurboQuant page (de.news.hada.io topic 27867), "Funktionsweise von TurboQuant":
 *    step 1 rotates each vector at random and codes every coordinate on its own with one
 *    fixed quantizer; step 2 spends one more bit per sketch coordinate on the residual with
 *    QJL.  "QJL: Eine 1-Bit-Methode ohne Overhead": a Gaussian projection whose outputs keep
 *    only their sign, read back by an estimator that pairs the full-precision query with
 *    the sign bits.  The comments under the same page: Lloyd-Max boundaries and levels.
 *  - TurboQuant explainer (chatgpz.de), "Stufe 1" and "Stufe 2": random preconditioning,
 *    then a 1-bit unbiased residual estimator.
 *  - Self-Indexing KVCache page (gist.science 2603.14224), "Methodologie" 1-4: channel
 *    mean subtracted before taking signs, 4-channel sign patterns 0..15 with 16 centroids per
 *    group, LUT-GEMV scoring in the compressed domain, top-k of the scores.
 *  - Monarch v3 page, "Wie es funktioniert": exact recent tokens and compressed older
 *    tokens share one softmax.
 *
 * Readings where the pages leave a step open (the same readings as the numpy oracle):
 *  - generator: SplitMix64 (Steele, Lea, Flood, OOPSLA 2014), output i of stream s is
 *    mix(s + (i+1) * 0x9E3779B97F4A7C15); normals by Box-Muller (1958) of word pairs,
 *    u1 = ((w0 >> 11) + 1) 2^-53, u2 = (w1 >> 11) 2^-53, sqrt(-2 ln u1) (cos, sin)(2 pi u2);
 *  - rotation Pi: Q of the Householder QR of a seeded row-major d x d Gaussian, columns
 *    signed so that R has a positive diagonal, rounded to float; x = Pi k;
 *  - QJL matrix S: m x d row-major normals of its own stream, rounded to float; the
 *    residual is sketched in the rotated basis;
 *  - code c = number of float boundaries tau_j with z >= tau_j, z = float(x sqrt(d) / r),
 *    r = |k| in double; r = 0 gives z = 0;
 *  - sign bit = [float(S e) >= 0]; estimator constant sqrt(pi/2) / m;
 *  - record: [key codes | sign bits | value codes | r_k | rho | r_v | zero pad to 16 B],
 *    code fields padded to 4 B; 1/2/4-bit fields a little-endian bitstream, 3-bit fields in
 *    groups of 32 codes per 12 bytes (bit positions below), a trailing partial 3-bit group
 *    a plain bitstream;
 *  - logit scale 1/sqrt(d) unless given; values carry no residual;
 *  - sign index: bit = [k >= mu] in float, mu the float-rounded channel mean; centroids the
 *    float-rounded mean of the members' (k - mu), 0 for an empty pattern; the LUT entry
 *    ((q0 c0 + q1 c1) + q2 c2) + q3 c3 in double, summed over the group's query heads
 *    after scaling by 2^s and rounding half to even, s the largest integer with
 *    n_terms * max|entry| * 2^s <= 2^30; ties in the top-k go to the lower index.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SC_PI 3.14159265358979323846

/* ---------------------------------------------------------------------------------------
 * Generator
 * ------------------------------------------------------------------------------------- */
static uint64_t sm64_word(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

void sc_splitmix64(uint64_t seed, int64_t n, uint64_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = sm64_word(seed, (uint64_t)i);
}

void sc_gaussians(uint64_t seed, int64_t n, double* out) {
    for (int64_t k = 0; 2 * k < n; ++k) {
        uint64_t w0 = sm64_word(seed, (uint64_t)(2 * k));
        uint64_t w1 = sm64_word(seed, (uint64_t)(2 * k + 1));
        double u1 = (double)((w0 >> 11) + 1u) * 0x1p-53;
        double u2 = (double)(w1 >> 11) * 0x1p-53;
        double rad = sqrt(-2.0 * log(u1));
        double ang = 6.283185307179586 * u2;
        out[2 * k] = rad * cos(ang);
        if (2 * k + 1 < n) out[2 * k + 1] = rad * sin(ang);
    }
}

/* ---------------------------------------------------------------------------------------
 * Rotation: Householder QR, Q with sign(R_jj) folded into column j
 * ------------------------------------------------------------------------------------- */
int sc_rotation(uint64_t seed, int d, float* pi_out) {
    double* A = (double*)malloc(sizeof(double) * (size_t)d * d);
    double* Q = (double*)malloc(sizeof(double) * (size_t)d * d);
    double* v = (double*)malloc(sizeof(double) * (size_t)d);
    double* rdiag = (double*)malloc(sizeof(double) * (size_t)d);
    if (!A || !Q || !v || !rdiag) { free(A); free(Q); free(v); free(rdiag); return -1; }
    sc_gaussians(seed, (int64_t)d * d, A);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) Q[i * d + j] = (i == j) ? 1.0 : 0.0;
    for (int j = 0; j < d; ++j) {
        double nrm2 = 0.0;
        for (int i = j; i < d; ++i) nrm2 += A[i * d + j] * A[i * d + j];
        double nrm = sqrt(nrm2);
        double alpha = A[j * d + j] >= 0.0 ? -nrm : nrm;     /* R_jj after the reflection */
        for (int i = 0; i < d; ++i) v[i] = 0.0;
        for (int i = j; i < d; ++i) v[i] = A[i * d + j];
        v[j] -= alpha;
        double vv = 0.0;
        for (int i = j; i < d; ++i) vv += v[i] * v[i];
        if (vv > 0.0) {
            /* A <- (I - 2 v v^T / v^T v) A on rows j.., columns j.. */
            for (int c = j; c < d; ++c) {
                double s = 0.0;
                for (int i = j; i < d; ++i) s += v[i] * A[i * d + c];
                s = 2.0 * s / vv;
                for (int i = j; i < d; ++i) A[i * d + c] -= s * v[i];
            }
            /* Q <- Q (I - 2 v v^T / v^T v) on columns j.. */
            for (int r = 0; r < d; ++r) {
                double s = 0.0;
                for (int i = j; i < d; ++i) s += Q[r * d + i] * v[i];
                s = 2.0 * s / vv;
                for (int i = j; i < d; ++i) Q[r * d + i] -= s * v[i];
            }
            rdiag[j] = alpha;
        } else {
            rdiag[j] = A[j * d + j];
        }
    }
    for (int r = 0; r < d; ++r)
        for (int c = 0; c < d; ++c) {
            double sg = rdiag[c] < 0.0 ? -1.0 : 1.0;
            pi_out[r * d + c] = (float)(Q[r * d + c] * sg);
        }
    free(A); free(Q); free(v); free(rdiag);
    return 0;
}

void sc_qjl_matrix(uint64_t seed, int m, int d, float* out) {
    if (m <= 0) return;
    double* g = (double*)malloc(sizeof(double) * (size_t)m * d);
    if (!g) return;
    sc_gaussians(seed, (int64_t)m * d, g);
    for (int64_t i = 0; i < (int64_t)m * d; ++i) out[i] = (float)g[i];
    free(g);
}

/* ---------------------------------------------------------------------------------------
 * Lloyd-Max quantizer for N(0, 1): boundaries at midpoints, levels at cell means
 * ------------------------------------------------------------------------------------- */
static double sc_pdf(double t) { return isinf(t) ? 0.0 : exp(-0.5 * t * t) / sqrt(2.0 * SC_PI); }
static double sc_cdf(double t) { return 0.5 * erfc(-t / sqrt(2.0)); }

int sc_lloyd_max(int bits, double* levels, double* bounds) {
    int L = 1 << bits;
    double lev[16], nw[16], edge[17];
    /* start: levels evenly spaced over [-2, 2]; the iteration has one fixed point for the
       Gaussian (log-concave) density, so the start only sets the number of iterations */
    for (int i = 0; i < L; ++i) lev[i] = -2.0 + 4.0 * i / (L - 1);
    for (int it = 0; it < 200000; ++it) {
        edge[0] = -INFINITY;
        edge[L] = INFINITY;
        for (int i = 1; i < L; ++i) edge[i] = 0.5 * (lev[i - 1] + lev[i]);
        for (int i = 0; i < L; ++i) {
            double mass = sc_cdf(edge[i + 1]) - sc_cdf(edge[i]);
            double mom = sc_pdf(edge[i]) - sc_pdf(edge[i + 1]);
            nw[i] = mom / mass;
        }
        double delta = 0.0;
        for (int i = 0; i < L; ++i) {
            double s = 0.5 * (nw[i] - nw[L - 1 - i]);      /* exact antisymmetry */
            double dd = fabs(s - lev[i]);
            if (dd > delta) delta = dd;
            lev[i] = s;
        }
        if (delta < 1e-15) break;
    }
    for (int i = 0; i < L; ++i) levels[i] = lev[i];
    for (int i = 0; i + 1 < L; ++i) bounds[i] = 0.5 * (lev[i] + lev[i + 1]);
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Codec: the constants of one configuration
 * ------------------------------------------------------------------------------------- */
typedef struct {
    int d, kb, m, vb;
    int kbytes, sbytes, vbytes, rbytes;
    float* Pi;        /* d x d */
    float* S;         /* m x d */
    float kl[16], kt[16], vl[16], vt[16];
} sc_codec;

static int ceil_to(int x, int a) { return (x + a - 1) / a * a; }

sc_codec* sc_codec_new(int d, int kb, int m, int vb, uint64_t rseed, uint64_t qseed) {
    if (d < 1 || kb < 1 || kb > 4 || vb < 1 || vb > 4 || m < 0 || m % 8) return NULL;
    sc_codec* c = (sc_codec*)calloc(1, sizeof(sc_codec));
    if (!c) return NULL;
    c->d = d; c->kb = kb; c->m = m; c->vb = vb;
    c->kbytes = ceil_to(d * kb / 8, 4);
    c->sbytes = m / 8;
    c->vbytes = ceil_to(d * vb / 8, 4);
    c->rbytes = ceil_to(c->kbytes + c->sbytes + c->vbytes + 12, 16);
    c->Pi = (float*)malloc(sizeof(float) * (size_t)d * d);
    c->S = (float*)malloc(sizeof(float) * (size_t)(m ? m : 1) * d);
    if (!c->Pi || !c->S || sc_rotation(rseed, d, c->Pi)) {
        free(c->Pi); free(c->S); free(c); return NULL;
    }
    sc_qjl_matrix(qseed, m, d, c->S);
    double l[16], t[16];
    sc_lloyd_max(kb, l, t);
    for (int i = 0; i < (1 << kb); ++i) c->kl[i] = (float)l[i];
    for (int i = 0; i + 1 < (1 << kb); ++i) c->kt[i] = (float)t[i];
    sc_lloyd_max(vb, l, t);
    for (int i = 0; i < (1 << vb); ++i) c->vl[i] = (float)l[i];
    for (int i = 0; i + 1 < (1 << vb); ++i) c->vt[i] = (float)t[i];
    return c;
}

void sc_codec_free(sc_codec* c) {
    if (!c) return;
    free(c->Pi); free(c->S); free(c);
}

int sc_record_bytes(const sc_codec* c) { return c->rbytes; }

/* Pi [d*d], S [m*d], key levels / bounds, value levels / bounds */
void sc_codec_tables(const sc_codec* c, float* pi, float* s, float* kl, float* kt, float* vl, float* vt) {
    memcpy(pi, c->Pi, sizeof(float) * (size_t)c->d * c->d);
    if (c->m) memcpy(s, c->S, sizeof(float) * (size_t)c->m * c->d);
    memcpy(kl, c->kl, sizeof(float) * (1u << c->kb));
    memcpy(kt, c->kt, sizeof(float) * ((1u << c->kb) - 1));
    memcpy(vl, c->vl, sizeof(float) * (1u << c->vb));
    memcpy(vt, c->vt, sizeof(float) * ((1u << c->vb) - 1));
}

/* ---------------------------------------------------------------------------------------
 * Bit fields
 * ------------------------------------------------------------------------------------- */
static void put_bit(uint8_t* buf, int pos, int bit) {
    if (bit) buf[pos >> 3] |= (uint8_t)(1u << (pos & 7));
}
static int get_bit(const uint8_t* buf, int pos) { return (buf[pos >> 3] >> (pos & 7)) & 1; }

/* bit position (within a 96-bit group of three little-endian 32-bit words) of bit t of
   code j of a 3-bit group */
static int group3_pos(int j, int t) {
    int word, bit;
    if (j < 24) {
        word = j / 8;
        bit = 8 * (j % 4) + 3 * ((j % 8) / 4) + t;
    } else {
        int r = j - 24, lane = r % 4, tt = 3 * (r / 4) + t;
        word = tt / 2;
        bit = 8 * lane + 6 + tt % 2;
    }
    return 32 * word + bit;
}

static void pack_codes(const int* codes, int n, int b, uint8_t* out) {
    if (b == 3) {
        int ng = n / 32;
        for (int g = 0; g < ng; ++g)
            for (int j = 0; j < 32; ++j)
                for (int t = 0; t < 3; ++t) put_bit(out + 12 * g, group3_pos(j, t), (codes[32 * g + j] >> t) & 1);
        for (int i = 32 * ng; i < n; ++i)
            for (int t = 0; t < 3; ++t) put_bit(out + 12 * ng, 3 * (i - 32 * ng) + t, (codes[i] >> t) & 1);
        return;
    }
    for (int i = 0; i < n; ++i)
        for (int t = 0; t < b; ++t) put_bit(out, b * i + t, (codes[i] >> t) & 1);
}

static void unpack_codes(const uint8_t* in, int n, int b, int* codes) {
    if (b == 3) {
        int ng = n / 32;
        for (int g = 0; g < ng; ++g)
            for (int j = 0; j < 32; ++j) {
                int c = 0;
                for (int t = 0; t < 3; ++t) c |= get_bit(in + 12 * g, group3_pos(j, t)) << t;
                codes[32 * g + j] = c;
            }
        for (int i = 32 * ng; i < n; ++i) {
            int c = 0;
            for (int t = 0; t < 3; ++t) c |= get_bit(in + 12 * ng, 3 * (i - 32 * ng) + t) << t;
            codes[i] = c;
        }
        return;
    }
    for (int i = 0; i < n; ++i) {
        int c = 0;
        for (int t = 0; t < b; ++t) c |= get_bit(in, b * i + t) << t;
        codes[i] = c;
    }
}

static void put_f32(uint8_t* p, float x) { memcpy(p, &x, 4); }   /* little-endian host */
static float get_f32(const uint8_t* p) { float x; memcpy(&x, p, 4); return x; }

/* One record from its fields: key codes [d], sign bits [m], value codes [d], three norms. */
static void pack_record(const sc_codec* c, const int* kc, const int* bits, const int* vc,
                        float r_k, float rho, float r_v, uint8_t* rec) {
    memset(rec, 0, (size_t)c->rbytes);
    pack_codes(kc, c->d, c->kb, rec);
    for (int j = 0; j < c->m; ++j) put_bit(rec + c->kbytes, j, bits[j]);
    pack_codes(vc, c->d, c->vb, rec + c->kbytes + c->sbytes);
    uint8_t* nb = rec + c->kbytes + c->sbytes + c->vbytes;
    put_f32(nb, r_k);
    put_f32(nb + 4, rho);
    put_f32(nb + 8, r_v);
}

/* kc [d], bits [m], vc [d], norms [3] */
void sc_unpack_record(const sc_codec* c, const uint8_t* rec, int* kc, int* bits, int* vc, float* norms) {
    unpack_codes(rec, c->d, c->kb, kc);
    for (int j = 0; j < c->m; ++j) bits[j] = get_bit(rec + c->kbytes, j);
    unpack_codes(rec + c->kbytes + c->sbytes, c->d, c->vb, vc);
    const uint8_t* nb = rec + c->kbytes + c->sbytes + c->vbytes;
    norms[0] = get_f32(nb);
    norms[1] = get_f32(nb + 4);
    norms[2] = get_f32(nb + 8);
}

/* ---------------------------------------------------------------------------------------
 * Compression (TurboQuant page, "Funktionsweise" steps 1 and 2)
 * ------------------------------------------------------------------------------------- */
static int code_of(float z, const float* bounds, int b) {
    int c = 0;
    for (int j = 0; j + 1 < (1 << b); ++j) c += z >= bounds[j];
    return c;
}

/* Step 1 on one vector: r = |k| (double), x = Pi k (double over float Pi), z = float(x sqrt(d)/r),
   codes.  Returns r. */
static double rotate_and_code(const sc_codec* c, const float* k, const float* bounds, int b, double* x, int* codes) {
    int d = c->d;
    double r2 = 0.0;
    for (int i = 0; i < d; ++i) r2 += (double)k[i] * (double)k[i];
    double r = sqrt(r2);
    for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int j = 0; j < d; ++j) s += (double)c->Pi[i * d + j] * (double)k[j];
        x[i] = s;
    }
    double scale = r > 0.0 ? sqrt((double)d) / r : 0.0;
    for (int i = 0; i < d; ++i) codes[i] = code_of((float)(x[i] * scale), bounds, b);
    return r;
}

/* k, v [n, d] float -> n records (rbytes each, zero padded). */
int sc_compress(const sc_codec* c, const float* k, const float* v, int64_t n, uint8_t* records) {
    int d = c->d, m = c->m;
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
    double* e = (double*)malloc(sizeof(double) * (size_t)d);
    int* kc = (int*)malloc(sizeof(int) * (size_t)d);
    int* vc = (int*)malloc(sizeof(int) * (size_t)d);
    int* bits = (int*)malloc(sizeof(int) * (size_t)(m ? m : 1));
    if (!x || !e || !kc || !vc || !bits) { free(x); free(e); free(kc); free(vc); free(bits); return -1; }
    double sd = sqrt((double)d);
    for (int64_t t = 0; t < n; ++t) {
        const float* kt = k + t * d;
        const float* vt = v + t * d;
        float r_k = (float)rotate_and_code(c, kt, c->kt, c->kb, x, kc);
        double rho2 = 0.0;
        for (int i = 0; i < d; ++i) {
            e[i] = x[i] - ((double)r_k / sd) * (double)c->kl[kc[i]];
            rho2 += e[i] * e[i];
        }
        for (int j = 0; j < m; ++j) {
            double p = 0.0;
            for (int i = 0; i < d; ++i) p += (double)c->S[j * d + i] * e[i];
            bits[j] = (float)p >= 0.0f;
        }
        float r_v = (float)rotate_and_code(c, vt, c->vt, c->vb, x, vc);
        pack_record(c, kc, bits, vc, r_k, (float)sqrt(rho2), r_v, records + t * c->rbytes);
    }
    free(x); free(e); free(kc); free(vc); free(bits);
    return 0;
}

/* The intermediate values of step 1 for n vectors x_in [n, d] (keys when is_value = 0, else
   values): z [n, d] the float coordinates that are coded, r [n] the norms in double. */
int sc_rotated(const sc_codec* c, const float* x_in, int is_value, int64_t n, float* z, double* r) {
    int d = c->d;
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
    int* codes = (int*)malloc(sizeof(int) * (size_t)d);
    if (!x || !codes) { free(x); free(codes); return -1; }
    for (int64_t t = 0; t < n; ++t) {
        double rr = rotate_and_code(c, x_in + t * d, is_value ? c->vt : c->kt, is_value ? c->vb : c->kb, x, codes);
        double scale = rr > 0.0 ? sqrt((double)d) / rr : 0.0;
        for (int i = 0; i < d; ++i) z[t * d + i] = (float)(x[i] * scale);
        r[t] = rr;
    }
    free(x); free(codes);
    return 0;
}

/* Step 2 from given key codes: k [n, d], kc [n, d], stored norms r_k [n] -> rho [n] (double)
   and the sketch p [n, m] = S e (double), e = Pi k - (r_k / sqrt d) gamma[kc]. */
int sc_residual(const sc_codec* c, const float* k, const int32_t* kc, const float* r_k, int64_t n,
                double* rho, double* p) {
    int d = c->d, m = c->m;
    double* x = (double*)malloc(sizeof(double) * (size_t)d);
    double* e = (double*)malloc(sizeof(double) * (size_t)d);
    if (!x || !e) { free(x); free(e); return -1; }
    double sd = sqrt((double)d);
    for (int64_t t = 0; t < n; ++t) {
        const float* kt = k + t * d;
        double r2 = 0.0;
        for (int i = 0; i < d; ++i) {
            double s = 0.0;
            for (int j = 0; j < d; ++j) s += (double)c->Pi[i * d + j] * (double)kt[j];
            e[i] = s - ((double)r_k[t] / sd) * (double)c->kl[kc[t * d + i]];
            r2 += e[i] * e[i];
        }
        rho[t] = sqrt(r2);
        for (int j = 0; j < m; ++j) {
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += (double)c->S[j * d + i] * e[i];
            p[t * m + j] = s;
        }
    }
    free(x); free(e);
    return 0;
}

/* Records from given float rotated coordinates (z already scaled by sqrt(d)/r):
   z_k, z_v [n, d], p [n, m], norms [n] each. */
int sc_quantize_from_rotated(const sc_codec* c, const float* z_k, const float* p, const float* r_k,
                             const float* rho, const float* z_v, const float* r_v, int64_t n, uint8_t* records) {
    int d = c->d, m = c->m;
    int* kc = (int*)malloc(sizeof(int) * (size_t)d);
    int* vc = (int*)malloc(sizeof(int) * (size_t)d);
    int* bits = (int*)malloc(sizeof(int) * (size_t)(m ? m : 1));
    if (!kc || !vc || !bits) { free(kc); free(vc); free(bits); return -1; }
    for (int64_t t = 0; t < n; ++t) {
        for (int i = 0; i < d; ++i) {
            kc[i] = code_of(z_k[t * d + i], c->kt, c->kb);
            vc[i] = code_of(z_v[t * d + i], c->vt, c->vb);
        }
        for (int j = 0; j < m; ++j) bits[j] = p[t * m + j] >= 0.0f;
        pack_record(c, kc, bits, vc, r_k[t], rho[t], r_v[t], records + t * c->rbytes);
    }
    free(kc); free(vc); free(bits);
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Scores from the packed records (TurboQuant page, "QJL", the asymmetric estimator)
 * ------------------------------------------------------------------------------------- */
/* q_x = Pi q, q_s = S q_x */
static void prepare_query(const sc_codec* c, const float* q, double* qx, double* qs) {
    int d = c->d;
    for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int j = 0; j < d; ++j) s += (double)c->Pi[i * d + j] * (double)q[j];
        qx[i] = s;
    }
    for (int j = 0; j < c->m; ++j) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += (double)c->S[j * d + i] * qx[i];
        qs[j] = s;
    }
}

/* s = (r_k / sqrt d) <q_x, gamma[c]> + sqrt(pi/2) / m * rho <q_s, 2 bit - 1> */
static double estimate(const sc_codec* c, const double* qx, const double* qs, const int* kc, const int* bits,
                       const float* norms) {
    double a = 0.0;
    for (int i = 0; i < c->d; ++i) a += qx[i] * (double)c->kl[kc[i]];
    double s = (double)norms[0] / sqrt((double)c->d) * a;
    if (c->m) {
        double b = 0.0;
        for (int j = 0; j < c->m; ++j) b += bits[j] ? qs[j] : -qs[j];
        s += sqrt(SC_PI / 2.0) / c->m * (double)norms[1] * b;
    }
    return s;
}

typedef struct {
    double *qx, *qs, *vsum;
    int *kc, *bits, *vc;
} sc_scratch;

static int scratch_new(const sc_codec* c, sc_scratch* w) {
    int d = c->d, m = c->m ? c->m : 1;
    w->qx = (double*)malloc(sizeof(double) * (size_t)d);
    w->qs = (double*)malloc(sizeof(double) * (size_t)m);
    w->vsum = (double*)malloc(sizeof(double) * (size_t)d);
    w->kc = (int*)malloc(sizeof(int) * (size_t)d);
    w->bits = (int*)malloc(sizeof(int) * (size_t)m);
    w->vc = (int*)malloc(sizeof(int) * (size_t)d);
    return (w->qx && w->qs && w->vsum && w->kc && w->bits && w->vc) ? 0 : -1;
}

static void scratch_free(sc_scratch* w) {
    free(w->qx); free(w->qs); free(w->vsum); free(w->kc); free(w->bits); free(w->vc);
}

/* Decode attention of one query head over one KV head.
 *   q [d] float; records [cap, rbytes]; the cold tokens are idx[0..n) when idx is given,
 *   else 0..n-1; hot_k, hot_v [nh, d] float (exact tokens, same softmax);
 *   scale 0 -> 1/sqrt(d).
 * Output out [d] (o = Pi^T sum_cold p vhat + sum_hot p v, over sum p), *lse, and when
 * logits is given the n cold logits then the nh hot logits.  With no token at all,
 * out = 0 and lse = -inf. */
int sc_decode_head(const sc_codec* c, const float* q, const uint8_t* records, const int32_t* idx, int64_t n,
                   const float* hot_k, const float* hot_v, int64_t nh, double scale, double* out, double* lse,
                   double* logits) {
    int d = c->d;
    double sc = scale != 0.0 ? scale : 1.0 / sqrt((double)d);
    sc_scratch w;
    double* lg = (double*)malloc(sizeof(double) * (size_t)(n + nh + 1));
    if (scratch_new(c, &w) || !lg) { scratch_free(&w); free(lg); return -1; }
    prepare_query(c, q, w.qx, w.qs);
    float norms[3];
    double mx = -INFINITY;
    for (int64_t t = 0; t < n; ++t) {
        const uint8_t* rec = records + (int64_t)(idx ? idx[t] : t) * c->rbytes;
        sc_unpack_record(c, rec, w.kc, w.bits, w.vc, norms);
        lg[t] = sc * estimate(c, w.qx, w.qs, w.kc, w.bits, norms);
        if (lg[t] > mx) mx = lg[t];
    }
    for (int64_t t = 0; t < nh; ++t) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += (double)hot_k[t * d + i] * (double)q[i];
        lg[n + t] = sc * s;
        if (lg[n + t] > mx) mx = lg[n + t];
    }
    if (logits)
        for (int64_t t = 0; t < n + nh; ++t) logits[t] = lg[t];
    for (int i = 0; i < d; ++i) { w.vsum[i] = 0.0; out[i] = 0.0; }
    if (n + nh == 0) {
        *lse = -INFINITY;
        scratch_free(&w); free(lg);
        return 0;
    }
    double l = 0.0, sd = sqrt((double)d);
    for (int64_t t = 0; t < n; ++t) {
        double p = exp(lg[t] - mx);
        l += p;
        const uint8_t* rec = records + (int64_t)(idx ? idx[t] : t) * c->rbytes;
        sc_unpack_record(c, rec, w.kc, w.bits, w.vc, norms);
        double a = p * ((double)norms[2] / sd);
        for (int i = 0; i < d; ++i) w.vsum[i] += a * (double)c->vl[w.vc[i]];
    }
    for (int j = 0; j < d; ++j) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += (double)c->Pi[i * d + j] * w.vsum[i];
        out[j] = s;
    }
    for (int64_t t = 0; t < nh; ++t) {
        double p = exp(lg[n + t] - mx);
        l += p;
        for (int i = 0; i < d; ++i) out[i] += p * (double)hot_v[t * d + i];
    }
    for (int i = 0; i < d; ++i) out[i] /= l;
    *lse = mx + log(l);
    scratch_free(&w); free(lg);
    return 0;
}

/* Bulk scan (TurboQuant page, "Leistung bei der Vektorsuche"): estimates of nq queries
   q [nq, d] against records [0, n) -> out [nq, n]. */
int sc_score_scan(const sc_codec* c, const float* q, int64_t nq, const uint8_t* records, int64_t n, double* out) {
    sc_scratch w;
    int d = c->d, m = c->m;
    double* qx = (double*)malloc(sizeof(double) * (size_t)(nq * d));
    double* qs = (double*)malloc(sizeof(double) * (size_t)(nq * (m ? m : 1)));
    if (scratch_new(c, &w) || !qx || !qs) { scratch_free(&w); free(qx); free(qs); return -1; }
    for (int64_t i = 0; i < nq; ++i) prepare_query(c, q + i * d, qx + i * d, qs + i * m);
    float norms[3];
    for (int64_t t = 0; t < n; ++t) {
        sc_unpack_record(c, records + t * c->rbytes, w.kc, w.bits, w.vc, norms);
        for (int64_t i = 0; i < nq; ++i) out[i * n + t] = estimate(c, qx + i * d, qs + i * m, w.kc, w.bits, norms);
    }
    scratch_free(&w); free(qx); free(qs);
    return 0;
}

/* ---------------------------------------------------------------------------------------
 * Self-Indexing sign index and LUT top-k ("Methodologie" 1-4)
 * ------------------------------------------------------------------------------------- */
/* mu [d] = float(mean over n tokens of k [n, d]) */
void sc_channel_mean(int d, const float* k, int64_t n, float* mu) {
    for (int i = 0; i < d; ++i) {
        double s = 0.0;
        for (int64_t t = 0; t < n; ++t) s += (double)k[t * d + i];
        mu[i] = n ? (float)(s / (double)n) : 0.0f;
    }
}

/* index [n, d/8]: pattern of group g (bit j = [k_(4g+j) >= mu_(4g+j)]) in bits [4g, 4g+4)
   of the token's little-endian bitstream; book [d/4, 16, 4]: centroids. */
void sc_sign_index(int d, const float* k, int64_t n, const float* mu, uint8_t* index, float* book) {
    int ng = d / 4;
    double* sum = (double*)calloc((size_t)ng * 16 * 4, sizeof(double));
    int64_t* cnt = (int64_t*)calloc((size_t)ng * 16, sizeof(int64_t));
    if (!sum || !cnt) { free(sum); free(cnt); return; }
    memset(index, 0, (size_t)n * (d / 8));
    for (int64_t t = 0; t < n; ++t) {
        const float* kt = k + t * d;
        for (int g = 0; g < ng; ++g) {
            int p = 0;
            for (int j = 0; j < 4; ++j) p |= (kt[4 * g + j] >= mu[4 * g + j]) << j;
            for (int j = 0; j < 4; ++j) put_bit(index + t * (d / 8), 4 * g + j, (p >> j) & 1);
            cnt[g * 16 + p] += 1;
            for (int j = 0; j < 4; ++j) sum[(g * 16 + p) * 4 + j] += (double)kt[4 * g + j] - (double)mu[4 * g + j];
        }
    }
    for (int g = 0; g < ng; ++g)
        for (int p = 0; p < 16; ++p)
            for (int j = 0; j < 4; ++j) {
                int64_t c = cnt[g * 16 + p];
                book[(g * 16 + p) * 4 + j] = c ? (float)(sum[(g * 16 + p) * 4 + j] / (double)c) : 0.0f;
            }
    free(sum); free(cnt);
}

typedef struct { int64_t score; int32_t idx; } sc_cand;

static int cand_order(const void* a, const void* b) {
    const sc_cand* x = (const sc_cand*)a;
    const sc_cand* y = (const sc_cand*)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

static int cmp_i32(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return x < y ? -1 : (x > y);
}

/* Largest integer s with n_terms * maxabs * 2^s <= 2^30 (0 when maxabs = 0). */
int sc_lut_scale_exponent(double maxabs, int n_terms) {
    double a = (double)n_terms * maxabs;
    if (a == 0.0) return 0;
    int e;
    double f = frexp(a, &e);
    return 30 - e + (f == 0.5 ? 1 : 0);
}

/* Top-k of one (sequence, KV head): G query heads q [G, d], index [n, d/8], book [d/4,16,4].
 * idx_out [k]: the chosen token indices ascending, -1 padded; scores_out [k] (or NULL): their
 * scores.  Returns the count min(k, n), or -1 when a score leaves int32. */
int sc_select_topk(int d, int G, const float* q, const uint8_t* index, const float* book, int64_t n, int k,
                   int32_t* idx_out, int32_t* scores_out) {
    int ng = d / 4;
    double* t = (double*)malloc(sizeof(double) * (size_t)G * ng * 16);
    int64_t* lut = (int64_t*)calloc((size_t)ng * 16, sizeof(int64_t));
    sc_cand* cand = (sc_cand*)malloc(sizeof(sc_cand) * (size_t)(n ? n : 1));
    if (!t || !lut || !cand) { free(t); free(lut); free(cand); return -1; }
    double maxabs = 0.0;
    for (int h = 0; h < G; ++h)
        for (int g = 0; g < ng; ++g)
            for (int p = 0; p < 16; ++p) {
                const float* cg = book + (g * 16 + p) * 4;
                const float* qg = q + h * d + 4 * g;
                double v = (double)qg[0] * (double)cg[0];
                v = v + (double)qg[1] * (double)cg[1];
                v = v + (double)qg[2] * (double)cg[2];
                v = v + (double)qg[3] * (double)cg[3];
                t[(h * ng + g) * 16 + p] = v;
                if (fabs(v) > maxabs) maxabs = fabs(v);
            }
    int s = sc_lut_scale_exponent(maxabs, G * ng);
    for (int h = 0; h < G; ++h)
        for (int i = 0; i < ng * 16; ++i) lut[i] += (int64_t)nearbyint(ldexp(t[h * ng * 16 + i], s));
    int bad = 0;
    for (int64_t tok = 0; tok < n; ++tok) {
        int64_t sc = 0;
        for (int g = 0; g < ng; ++g) {
            int p = 0;
            for (int j = 0; j < 4; ++j) p |= get_bit(index + tok * (d / 8), 4 * g + j) << j;
            sc += lut[g * 16 + p];
        }
        if (sc >= 2147483648ll || sc <= -2147483648ll) bad = 1;
        cand[tok].score = sc;
        cand[tok].idx = (int32_t)tok;
    }
    if (bad) { free(t); free(lut); free(cand); return -1; }
    int64_t cnt = n < k ? n : k;
    qsort(cand, (size_t)n, sizeof(sc_cand), cand_order);
    for (int64_t i = 0; i < cnt; ++i) idx_out[i] = cand[i].idx;
    qsort(idx_out, (size_t)cnt, sizeof(int32_t), cmp_i32);
    for (int64_t i = cnt; i < k; ++i) idx_out[i] = -1;
    if (scores_out) {
        /* scores of the chosen tokens, in the order of idx_out */
        for (int64_t i = 0; i < k; ++i) scores_out[i] = 0;
        for (int64_t i = 0; i < cnt; ++i) {
            int64_t tok = idx_out[i], sc = 0;
            for (int g = 0; g < ng; ++g) {
                int p = 0;
                for (int j = 0; j < 4; ++j) p |= get_bit(index + tok * (d / 8), 4 * g + j) << j;
                sc += lut[g * 16 + p];
            }
            scores_out[i] = (int32_t)sc;
        }
    }
    free(t); free(lut); free(cand);
    return (int)cnt;
}
