/*
 * tqref.c -- the oracle: a plain, slow, double-precision CPU implementation of
 * TurboQuant KV-cache compression (quantize, score, dequantize, decode
 * attention) as the benchmark pages describe it.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code, header, table or constant generator
 * with the GPU path.
 *
 * Sources (page titles as given on the pages):
 *  [P2] "[Benchmark] TurboQuant 實測：KV Cache 3-bit 壓縮，真的零損失？",
 *       section "TurboQuant 是什麼：30 秒懶人包" (random rotation, per-coordinate
 *       Lloyd-Max, QJL 1-bit residual sign, unbiased scores), section
 *       "Lloyd-Max Codebook" (distortion per coordinate), "GB10 速度"
 *       (packed size).
 *  [P4] "TurboQuant 是什麼" section of the vLLM benchmark summary: random
 *       rotation concentrates coordinates, each coordinate gets an optimal
 *       scalar quantizer, a 1-bit QJL residual corrects inner-product bias.
 *  [P1] WHT rotation to "Gaussianize", then scalar quantization.
 *
 * Readings where the pages are silent:
 *  - codebook law N(0, 1/d); centroids stored rounded to fp16-representable
 *    values, boundaries = fp32 midpoints of the stored centroids;
 *  - rotation y = H (D .* x) / (sqrt(d) * ||x||), H the natural-order
 *    Sylvester Hadamard matrix, D a seeded +-1 diagonal;
 *  - code index = number of boundaries strictly below y (ties go low);
 *  - QJL: r = y - c[idx], gamma = ||r||, u = S r with S the stored fp16-valued
 *    m x d Gaussian matrix, sign bit = [u >= 0], correction scale
 *    gamma * sqrt(pi/2) / m;
 *  - norm and gamma stored as fp16 (RNE); later steps use the stored values;
 *  - zero vector: y := 0.
 *
 * Packed layout (group-major): the d coordinates form d/8 groups; group c
 * holds coordinates c + (d/8) t for t = 0..7. A vector's codes are a bit
 * stream of b*d bits (little-endian: stream bit k is bit k%32 of uint32 word
 * k/32): group c occupies bits [8 b c, 8 b c + 8 b), and inside it code t
 * occupies bits [b t, b t + b) with code bit p at b t + p. Signs use the same
 * grouping of the m projection rows with one bit per code: bit t of byte j0
 * is the sign bit of row j0 + (m/8) t.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define TQREF_MAXL 256

/* ------------------------------------------------------------ fp16 by hand */

double tqref_half_to_double(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f + 1024), e - 25);
    return s ? -v : v;
}

/* round-to-nearest-even conversion of a double to IEEE binary16 */
uint16_t tqref_double_to_half(double x)
{
    uint16_t sign = 0;
    if (x != x) return 0x7E00;
    if (signbit(x)) { sign = 0x8000; x = -x; }
    if (x == 0.0) return sign;
    if (x >= 65520.0) return sign | 0x7C00;         /* rounds to inf */
    int e;
    frexp(x, &e);                                    /* x = f 2^e, f in [0.5,1) */
    int ulp_exp = (e - 1) - 10;                      /* spacing exponent */
    if (ulp_exp < -24) ulp_exp = -24;                /* subnormal spacing */
    double q = ldexp(x, -ulp_exp);                   /* exact */
    double fl = floor(q), rem = q - fl;
    uint32_t n = (uint32_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (n & 1))) n++;
    /* n * 2^ulp_exp; encode */
    if (ulp_exp == -24) {
        if (n >= 1024) return sign | (uint16_t)(1 << 10 | (n - 1024)); /* became normal */
        return sign | (uint16_t)n;
    }
    if (n >= 2048) { n >>= 1; ulp_exp++; }
    int be = ulp_exp + 25;                            /* biased exponent */
    if (be >= 31) return sign | 0x7C00;
    return sign | (uint16_t)(be << 10) | (uint16_t)(n - 1024);
}

/* ------------------------------------------------------------ Hadamard */

static int had(int i, int j) { return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1; }

/* ------------------------------------------------------------ laws */

typedef struct {
    int kind;              /* 0 = N(0, sigma^2); 1 = exact coordinate law in dimension dim */
    double sigma;          /* 1 / sqrt(d): the scale of both laws */
    int dim;               /* kind 1 */
} law_t;

/*
 * The exact law of one coordinate of a uniformly random unit vector in R^d
 * ([vLLM] "TurboQuant 是什麼：30 秒懶人包": after the random rotation the
 * coordinates follow a Beta law): density proportional to (1 - t^2)^((d-3)/2)
 * on [-1, 1], i.e. Y^2 ~ Beta(1/2, (d-1)/2). Its upper tail is
 *   P(Y > t) = 1/2 I_{1 - t^2}((d-1)/2, 1/2)  for t >= 0,
 * with I the regularized incomplete beta function, evaluated here from its
 * continued fraction (modified Lentz) on the side where it converges.
 */
static double ibeta_fraction(double a, double b, double x)
{
    /* h = 1 + d1 / (1 + d2 / (1 + ...)) with
     *   d_{2m+1} = -(a + m)(a + b + m) x / ((a + 2m)(a + 2m + 1)),
     *   d_{2m}   = m (b - m) x / ((a + 2m - 1)(a + 2m)),
     * evaluated by the modified Lentz method; I_x(a, b) = front / (a h) */
    const double tiny = 1e-300;
    double h = 1.0, C = 1.0, Dd = 0.0;
    for (int i = 1; i <= 40000; ++i) {
        double num;
        if (i % 2 == 0) {
            int m = i / 2;
            num = m * (b - m) * x / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
        } else {
            int m = (i - 1) / 2;
            num = -(a + m) * (a + b + m) * x / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
        }
        Dd = 1.0 + num * Dd;
        if (fabs(Dd) < tiny) Dd = tiny;
        Dd = 1.0 / Dd;
        C = 1.0 + num / C;
        if (fabs(C) < tiny) C = tiny;
        double step = C * Dd;
        h *= step;
        if (fabs(step - 1.0) < 1e-16) break;
    }
    return 1.0 / h;
}

static double ibeta(double a, double b, double x)
{
    if (x <= 0.0) return 0.0;
    if (x >= 1.0) return 1.0;
    double lfront = a * log(x) + b * log1p(-x) - (lgamma(a) + lgamma(b) - lgamma(a + b));
    if (x < (a + 1.0) / (a + b + 2.0)) return exp(lfront) / a * ibeta_fraction(a, b, x);
    return 1.0 - exp(lfront) / b * ibeta_fraction(b, a, 1.0 - x);
}

/* P(Y > t) under the coordinate law in dimension d (d >= 2) */
static double sphere_upper(int d, double t)
{
    if (t >= 1.0) return 0.0;
    if (t <= -1.0) return 1.0;
    if (t >= 0.0) return 0.5 * ibeta(0.5 * (d - 1), 0.5, 1.0 - t * t);
    return 1.0 - 0.5 * ibeta(0.5 * (d - 1), 0.5, 1.0 - t * t);
}

/* P(a < Y <= b), from the nearer tail */
static double sphere_mass(int d, double a, double b)
{
    if (a >= 0) return sphere_upper(d, a) - sphere_upper(d, b);
    if (b <= 0) return sphere_upper(d, -b) - sphere_upper(d, -a);
    return 1.0 - sphere_upper(d, -a) - sphere_upper(d, b);
}

static double phi(double t) { return isinf(t) ? 0.0 : exp(-0.5 * t * t) / sqrt(2.0 * M_PI); }

/* P(a < Y <= b) for the standard normal, accurate in both tails */
static double norm_mass(double a, double b)
{
    if (a >= 0) return 0.5 * (erfc(a / M_SQRT2) - erfc(b / M_SQRT2));
    if (b <= 0) return 0.5 * (erfc(-b / M_SQRT2) - erfc(-a / M_SQRT2));
    return 1.0 - 0.5 * erfc(-a / M_SQRT2) - 0.5 * erfc(b / M_SQRT2);
}

static double tphi(double t) { return isinf(t) ? 0.0 : t * phi(t); }

/* zeroth, first and second moments of the law over (a, b] */
static void law_moments(const law_t* L, double a, double b, double* m0, double* m1, double* m2)
{
    if (L->kind == 0) {
        double s = L->sigma, al = a / s, be = b / s;
        *m0 = norm_mass(al, be);
        *m1 = s * (phi(al) - phi(be));
        *m2 = s * s * (*m0 + tphi(al) - tphi(be));
    } else if (L->kind == 1) {
        /* first moment in closed form: the density times t integrates to
         * -K (1 - t^2)^((d-1)/2) / (d - 1), K the density's normalizer
         * 1 / B(1/2, (d-1)/2); the second from t^2 (1-t^2)^k = (1-t^2)^k -
         * (1-t^2)^(k+1): the law in dimension d minus (d-1)/d times the law in
         * dimension d + 2 */
        int d = L->dim;
        double lo = a < -1.0 ? -1.0 : a, hi = b > 1.0 ? 1.0 : b;
        if (hi <= lo) { *m0 = *m1 = *m2 = 0.0; return; }
        double K = exp(lgamma(0.5 * d) - lgamma(0.5 * (d - 1)) - 0.5 * log(M_PI));
        double e = 0.5 * (d - 1);
        *m0 = sphere_mass(d, lo, hi);
        *m1 = K / (d - 1) * (pow(1.0 - lo * lo, e) - pow(1.0 - hi * hi, e));
        *m2 = *m0 - (double)(d - 1) / d * sphere_mass(d + 2, lo, hi);
    }
}

/* Lloyd-Max fixed point: boundaries are midpoints of neighbouring centroids,
 * each centroid is the conditional mean of its cell. Returns iterations used,
 * or -1 without convergence. */
static int lloyd(const law_t* L, int nl, double* c, double tol, int maxit, int symmetric)
{
    double sg = L->sigma;
    /* start spread over +-2.5 sigma (inside the support for the bounded law) */
    double r = 2.5 * sg;
    if (L->kind == 1 && r > 1.0 - 1.0 / nl) r = 1.0 - 1.0 / nl;
    for (int l = 0; l < nl; ++l)
        c[l] = (nl == 1) ? 0.0 : r * (-1.0 + 2.0 * l / (nl - 1));
    double t[TQREF_MAXL + 1], cn[TQREF_MAXL];
    for (int it = 1; it <= maxit; ++it) {
        t[0] = -INFINITY; t[nl] = INFINITY;
        for (int l = 1; l < nl; ++l) t[l] = 0.5 * (c[l - 1] + c[l]);
        for (int l = 0; l < nl; ++l) {
            double m0, m1, m2;
            law_moments(L, t[l], t[l + 1], &m0, &m1, &m2);
            cn[l] = (m0 > 0) ? m1 / m0 : c[l];
        }
        if (symmetric)
            for (int l = 0; l < nl / 2; ++l) {
                double v = 0.5 * (cn[nl - 1 - l] - cn[l]);
                cn[l] = -v; cn[nl - 1 - l] = v;
            }
        double dmax = 0;
        for (int l = 0; l < nl; ++l) { double dd = fabs(cn[l] - c[l]); if (dd > dmax) dmax = dd; c[l] = cn[l]; }
        if (dmax < tol * sg) return it;
    }
    return -1;
}

/* E[(Y - q(Y))^2] for centroids c and boundaries t (t[0..nl-2]) under the law */
static double law_distortion(const law_t* L, int nl, const double* c, const double* t)
{
    double D = 0;
    for (int l = 0; l < nl; ++l) {
        double a = (l == 0) ? -INFINITY : t[l - 1];
        double b = (l == nl - 1) ? INFINITY : t[l];
        double m0, m1, m2;
        law_moments(L, a, b, &m0, &m1, &m2);
        D += m2 - 2.0 * c[l] * m1 + c[l] * c[l] * m0;
    }
    return D;
}

/*
 * Lloyd-Max codebook for N(0, 1/d) with 2^bits levels ([P2] "Lloyd-Max
 * Codebook"; law: reading of [P1] "Gaussianize" confirmed by the printed
 * distortions). Outputs the exact solution (c_exact), the stored centroids
 * (fp16-representable, as fp32), the stored boundaries (fp32 midpoints of the
 * stored centroids) and the analytic distortion per coordinate of the exact
 * and of the stored codebook. Returns iterations, or -1 if not converged,
 * -2 for bad arguments.
 */
int tqref_codebook_law(int d, int bits, int law, double* c_exact, float* c_stored, float* t_stored,
                       double* dist_exact, double* dist_stored)
{
    if (d < 1 || bits < 1 || bits > 8 || law < 0 || law > 1) return -2;
    if (law == 1 && d < 2) return -2;
    int nl = 1 << bits;
    law_t L = {law, 1.0 / sqrt((double)d), d};
    double c[TQREF_MAXL];
    /* 1e-15 sigma for the widths the cache uses (<= 4 bits); wider codebooks
     * have cells of tiny mass whose conditional means carry more rounding
     * noise, so they stop at 1e-12 sigma. The exact law's masses come from a
     * continued fraction accurate to a few 1e-15, so it stops at 1e-13 sigma. */
    double tol = bits <= 4 ? 1e-15 : 1e-12;
    if (law == 1 && tol < 1e-13) tol = 1e-13;
    int it = lloyd(&L, nl, c, tol, 2000000, 1);
    if (it < 0) return -1;
    double t[TQREF_MAXL], cs[TQREF_MAXL], ts[TQREF_MAXL];
    for (int l = 0; l < nl; ++l) {
        c_exact[l] = c[l];
        cs[l] = tqref_half_to_double(tqref_double_to_half(c[l]));
        c_stored[l] = (float)cs[l];
    }
    for (int l = 0; l + 1 < nl; ++l) {
        t[l] = 0.5 * (c[l] + c[l + 1]);
        t_stored[l] = (float)(0.5 * (cs[l] + cs[l + 1]));
        ts[l] = (double)t_stored[l];
    }
    if (dist_exact) *dist_exact = law_distortion(&L, nl, c, t);
    if (dist_stored) *dist_stored = law_distortion(&L, nl, cs, ts);
    return it;
}

/* moments (m0, m1, m2) of the coordinate law in dimension d over (a, b] */
void tqref_sphere_moments(int d, double a, double b, double* m)
{
    law_t L = {1, 1.0 / sqrt((double)d), d};
    law_moments(&L, a, b, &m[0], &m[1], &m[2]);
}

/* ------------------------------------------------------------ quantizer */

typedef struct {
    int d, bits, m;            /* m = 0: MSE only; m = d: with QJL */
    const float* cent;         /* [2^bits] stored centroids */
    const float* bnd;          /* [2^bits - 1] stored boundaries */
    const uint32_t* diag;      /* [ceil(d/32)] bit set -> -1 */
    const uint16_t* S;         /* [m][d] fp16 bits */
} tqref_quantizer;

/* S widened to double once per call (same values, fewer conversions) */
static double* widen_S(const tqref_quantizer* Q)
{
    int64_t n = (int64_t)Q->m * Q->d;
    double* s = malloc(sizeof(double) * (n + 1));
    for (int64_t i = 0; i < n; ++i) s[i] = tqref_half_to_double(Q->S[i]);
    return s;
}

static int diag_sign(const uint32_t* D, int j) { return ((D[j >> 5] >> (j & 31)) & 1) ? -1 : 1; }

static int words_of(int d) { return (d + 31) / 32; }

/* stream bit of code bit p of coordinate i (group-major layout) */
static int64_t code_bit(int d, int bits, int i, int p)
{
    int G = d >= 8 ? d / 8 : 1, c = i % G, t = i / G;
    return (int64_t)8 * bits * c + (int64_t)bits * t + p;
}

/* stream bit of the sign of projection row j */
static int64_t sign_bit(int m, int j)
{
    int G = m >= 8 ? m / 8 : 1;
    return (int64_t)8 * (j % G) + j / G;
}

/* the d x d matrix H D (entries +-1), built once per call */
static double* build_HD(const tqref_quantizer* Q)
{
    int d = Q->d;
    double* h = malloc(sizeof(double) * d * d);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) h[i * d + j] = had(i, j) * diag_sign(Q->diag, j);
    return h;
}

/* rotation: out_i = sum_j H_ij D_j x_j / sqrt(d) */
static void rotate(const tqref_quantizer* Q, const double* HD, const double* x, double* out)
{
    int d = Q->d;
    for (int i = 0; i < d; ++i) {
        double s = 0;
        for (int j = 0; j < d; ++j) s += HD[i * d + j] * x[j];
        out[i] = s / sqrt((double)d);
    }
}

/*
 * The QJL stage of one vector ([P2] "TurboQuant 是什麼：30 秒懶人包", step two):
 * residual r = y - c[idx] of the rotated unit vector y against its chosen
 * centroids, gamma = ||r||, u = S r, sign bit j = [u_j >= 0]. Writes the sign
 * words sv (m bits, grouped as the codes), returns gamma; u_out (nullable)
 * receives u.
 */
static double qjl_stage(const tqref_quantizer* Q, const double* Sd, const double* y, const int* idx,
                        double* r, uint32_t* sv, double* u_out)
{
    int d = Q->d, m = Q->m;
    double g2 = 0;
    for (int i = 0; i < d; ++i) {
        r[i] = y[i] - (double)Q->cent[idx[i]];
        g2 += r[i] * r[i];
    }
    memset(sv, 0, sizeof(uint32_t) * words_of(m));
    for (int j = 0; j < m; ++j) {
        double u = 0;
        for (int i = 0; i < d; ++i) u += Sd[(int64_t)j * d + i] * r[i];
        if (u_out) u_out[j] = u;
        if (u >= 0) {
            int64_t b = sign_bit(m, j);
            sv[b >> 5] |= 1u << (b & 31);
        }
    }
    return sqrt(g2);
}

/*
 * Quantize n vectors x[n][d] (values given exactly as doubles).
 * Writes packed codes, signs (if m > 0), fp16 norms and fp16 residual norms.
 * Optional y_out[n][d] receives the rotated unit vector, u_out[n][m] the
 * projection S r, both in double, for boundary-window analysis in tests.
 */
void tqref_quantize(const tqref_quantizer* Q, const double* x, int64_t n,
                    uint32_t* codes, uint32_t* signs, uint16_t* norm16, uint16_t* rnorm16,
                    double* y_out, double* u_out)
{
    int d = Q->d, m = Q->m, nl = 1 << Q->bits, W = words_of(d), WS = words_of(m);
    double* Sd = widen_S(Q);
    double* HD = build_HD(Q);
#pragma omp parallel
    {
        double* y = malloc(sizeof(double) * d);
        double* r = malloc(sizeof(double) * d);
        double* z = malloc(sizeof(double) * d);
        int* idx = malloc(sizeof(int) * d);
#pragma omp for schedule(static)
        for (int64_t v = 0; v < n; ++v) {
            const double* xv = x + v * d;
            double ss = 0;
            for (int j = 0; j < d; ++j) ss += xv[j] * xv[j];
            double nrm = sqrt(ss);
            if (nrm > 0) {
                for (int j = 0; j < d; ++j) z[j] = xv[j] / nrm;
                rotate(Q, HD, z, y);
            } else {
                for (int j = 0; j < d; ++j) y[j] = 0.0;
            }
            uint32_t* cv = codes + v * (int64_t)Q->bits * W;
            memset(cv, 0, sizeof(uint32_t) * Q->bits * W);
            for (int i = 0; i < d; ++i) {
                int k = 0;
                for (int l = 0; l + 1 < nl; ++l) if ((double)Q->bnd[l] < y[i]) k++;
                idx[i] = k;
                for (int p = 0; p < Q->bits; ++p)
                    if ((k >> p) & 1) {
                        int64_t b = code_bit(d, Q->bits, i, p);
                        cv[b >> 5] |= 1u << (b & 31);
                    }
            }
            if (y_out) memcpy(y_out + v * d, y, sizeof(double) * d);
            norm16[v] = tqref_double_to_half(nrm);
            if (m > 0)
                rnorm16[v] = tqref_double_to_half(qjl_stage(Q, Sd, y, idx, r, signs + v * WS,
                                                            u_out ? u_out + v * m : NULL));
        }
        free(y); free(r); free(z); free(idx);
    }
    free(Sd); free(HD);
}

static int code_at(const uint32_t* cv, int d, int bits, int i);

/*
 * The QJL stage alone, for n rotated unit vectors y[n][d] whose codes are
 * given (packed codes[n][bits*d/32]) rather than chosen here: signs, fp16
 * gamma and (nullable) u[n][m] exactly as tqref_quantize computes them from
 * its own codes. Tests use it to check a sketch built on codes that differ
 * from the oracle's by one level inside the boundary window. m must be > 0.
 */
void tqref_sketch(const tqref_quantizer* Q, const double* y, const uint32_t* codes, int64_t n,
                  uint32_t* signs, uint16_t* rnorm16, double* u_out)
{
    int d = Q->d, m = Q->m, W = words_of(d), WS = words_of(m);
    if (m <= 0) return;
    double* Sd = widen_S(Q);
#pragma omp parallel
    {
        double* r = malloc(sizeof(double) * d);
        int* idx = malloc(sizeof(int) * d);
#pragma omp for schedule(static)
        for (int64_t v = 0; v < n; ++v) {
            const uint32_t* cv = codes + v * (int64_t)Q->bits * W;
            for (int i = 0; i < d; ++i) idx[i] = code_at(cv, d, Q->bits, i);
            rnorm16[v] = tqref_double_to_half(qjl_stage(Q, Sd, y + v * d, idx, r, signs + v * WS,
                                                        u_out ? u_out + v * m : NULL));
        }
        free(r); free(idx);
    }
    free(Sd);
}

/* code index of coordinate i of packed vector cv */
static int code_at(const uint32_t* cv, int d, int bits, int i)
{
    int k = 0;
    for (int p = 0; p < bits; ++p) {
        int64_t b = code_bit(d, bits, i, p);
        k |= (int)((cv[b >> 5] >> (b & 31)) & 1) << p;
    }
    return k;
}

/* +1 / -1 from the stored sign of projection row j (m rows) */
static int sign_at(const uint32_t* sv, int m, int j)
{
    int64_t b = sign_bit(m, j);
    return ((sv[b >> 5] >> (b & 31)) & 1) ? 1 : -1;
}

/* query prep: qr = H D q / sqrt(d); p = S qr (p only when m > 0) */
static void prep_query(const tqref_quantizer* Q, const double* Sd, const double* HD,
                       const double* q, double* qr, double* p)
{
    rotate(Q, HD, q, qr);
    for (int j = 0; j < Q->m; ++j) {
        double s = 0;
        for (int i = 0; i < Q->d; ++i) s += Sd[(int64_t)j * Q->d + i] * qr[i];
        p[j] = s;
    }
}

/* estimated <q, k> for one packed key given the prepared query */
static double score_one(const tqref_quantizer* Q, const double* qr, const double* p,
                        const uint32_t* cv, const uint32_t* sv, uint16_t n16, uint16_t g16)
{
    int d = Q->d;
    double mse = 0;
    for (int i = 0; i < d; ++i) mse += qr[i] * (double)Q->cent[code_at(cv, d, Q->bits, i)];
    double s = mse;
    if (Q->m > 0) {
        double qj = 0;
        for (int j = 0; j < Q->m; ++j) qj += p[j] * sign_at(sv, Q->m, j);
        s += tqref_half_to_double(g16) * sqrt(M_PI / 2.0) / Q->m * qj;
    }
    return tqref_half_to_double(n16) * s;
}

/* scores[qi][k] = estimated <q_qi, key_k> ([P2]: inner products from packed keys) */
void tqref_scores(const tqref_quantizer* Q, const uint32_t* codes, const uint32_t* signs,
                  const uint16_t* norm16, const uint16_t* rnorm16, int64_t n_keys,
                  const double* q, int64_t n_q, double* scores)
{
    int d = Q->d, m = Q->m, W = words_of(d), WS = words_of(m);
    double* qr = malloc(sizeof(double) * n_q * d);
    double* p = malloc(sizeof(double) * (n_q * m + 1));
    double* Sd = widen_S(Q);
    double* HD = build_HD(Q);
    for (int64_t a = 0; a < n_q; ++a) prep_query(Q, Sd, HD, q + a * d, qr + a * d, p + a * m);
    free(Sd); free(HD);
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < n_keys; ++k)
        for (int64_t a = 0; a < n_q; ++a)
            scores[a * n_keys + k] = score_one(Q, qr + a * d, p + a * m,
                                               codes + k * (int64_t)Q->bits * W,
                                               m ? signs + k * WS : NULL, norm16[k],
                                               m ? rnorm16[k] : 0);
    free(qr); free(p);
}

/* x_hat = n * D H (c + [qjl] gamma sqrt(pi/2)/m S^T sgn) / sqrt(d) */
void tqref_dequantize(const tqref_quantizer* Q, const uint32_t* codes, const uint32_t* signs,
                      const uint16_t* norm16, const uint16_t* rnorm16, int64_t n,
                      int include_qjl, double* out)
{
    int d = Q->d, m = Q->m, W = words_of(d), WS = words_of(m);
    double* Sd = widen_S(Q);
#pragma omp parallel
    {
        double* a = malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (int64_t v = 0; v < n; ++v) {
            const uint32_t* cv = codes + v * (int64_t)Q->bits * W;
            for (int i = 0; i < d; ++i) a[i] = Q->cent[code_at(cv, d, Q->bits, i)];
            if (m > 0 && include_qjl) {
                double g = tqref_half_to_double(rnorm16[v]) * sqrt(M_PI / 2.0) / m;
                for (int i = 0; i < d; ++i) {
                    double s = 0;
                    for (int j = 0; j < m; ++j)
                        s += Sd[(int64_t)j * d + i] * sign_at(signs + v * WS, m, j);
                    a[i] += g * s;
                }
            }
            double nv = tqref_half_to_double(norm16[v]);
            for (int j = 0; j < d; ++j) {
                double s = 0;
                for (int i = 0; i < d; ++i) s += had(j, i) * a[i];
                out[v * d + j] = nv * diag_sign(Q->diag, j) * s / sqrt((double)d);
            }
        }
        free(a);
    }
    free(Sd);
}

/*
 * Decode attention over compressed K/V: for each stream s and head h,
 * z_t = score(q_{s,h}, K_{s,t}) * scale, p = softmax_t(z),
 * o = sum_t p_t * V_hat_{s,t}, computed as D_v H (sum_t p_t n_t c_v(t)) / sqrt(d)
 * (V without QJL). Streams hold T consecutive packed vectors each; q and out
 * are [n_streams][G][d].
 */
void tqref_decode_attn(const tqref_quantizer* QK, const tqref_quantizer* QV,
                       const uint32_t* kcodes, const uint32_t* ksigns, const uint16_t* knorm,
                       const uint16_t* krnorm, const uint32_t* vcodes, const uint16_t* vnorm,
                       int64_t n_streams, int64_t T, int G, const double* q, double scale,
                       double* out)
{
    int d = QK->d, m = QK->m, W = words_of(d), WS = words_of(m), WV = words_of(QV->d);
    double* Sd = widen_S(QK);
    double* HD = build_HD(QK);
#pragma omp parallel
    {
        double* qr = malloc(sizeof(double) * d);
        double* p = malloc(sizeof(double) * (m + 1));
        double* z = malloc(sizeof(double) * (T + 1));
        double* acc = malloc(sizeof(double) * QV->d);
#pragma omp for schedule(dynamic, 1)
        for (int64_t sh = 0; sh < n_streams * G; ++sh) {
            int64_t s = sh / G;
            prep_query(QK, Sd, HD, q + sh * d, qr, p);
            double mx = -INFINITY;
            for (int64_t t = 0; t < T; ++t) {
                int64_t v = s * T + t;
                z[t] = scale * score_one(QK, qr, p, kcodes + v * (int64_t)QK->bits * W,
                                         m ? ksigns + v * WS : NULL, knorm[v],
                                         m ? krnorm[v] : 0);
                if (z[t] > mx) mx = z[t];
            }
            double l = 0;
            for (int i = 0; i < QV->d; ++i) acc[i] = 0;
            for (int64_t t = 0; t < T; ++t) {
                int64_t v = s * T + t;
                double w = exp(z[t] - mx);
                l += w;
                double wn = w * tqref_half_to_double(vnorm[v]);
                const uint32_t* cv = vcodes + v * (int64_t)QV->bits * WV;
                for (int i = 0; i < QV->d; ++i) acc[i] += wn * (double)QV->cent[code_at(cv, QV->d, QV->bits, i)];
            }
            for (int j = 0; j < QV->d; ++j) {
                double sacc = 0;
                for (int i = 0; i < QV->d; ++i) sacc += had(j, i) * acc[i];
                out[sh * QV->d + j] = diag_sign(QV->diag, j) * sacc / (sqrt((double)QV->d) * l);
            }
        }
        free(qr); free(p); free(z); free(acc);
    }
    free(Sd); free(HD);
}

int tqref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void tqref_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
