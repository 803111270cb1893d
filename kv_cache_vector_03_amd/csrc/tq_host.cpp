// Host side of the library: the codebook solver, argument validation and the
// thread-local error message. Pure C++ (no device code), so every check here
// can be exercised without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "tq.h"
#include "tq_internal.h"

namespace tq {

static thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = 0; }

// ---------------------------------------------------------------- codebook
//
// Lloyd-Max for N(0, sigma^2), sigma = 1/sqrt(d): alternate "boundaries at
// midpoints of neighbouring centroids" and "centroid = conditional mean of its
// cell" until the centroids move by less than tol * sigma. Initial centroids
// are the Gaussian quantiles at (l + 1/2) / L, found by bisection.

static double std_cdf_upper(double z) { return 0.5 * std::erfc(z / std::sqrt(2.0)); }

// P(a < Z <= b) for standard normal Z, computed from the nearer tail
static double std_mass(double a, double b)
{
    if (a >= 0) return std_cdf_upper(a) - std_cdf_upper(b);
    if (b <= 0) return std_cdf_upper(-b) - std_cdf_upper(-a);
    return 1.0 - std_cdf_upper(-a) - std_cdf_upper(b);
}

static double std_pdf(double z) { return std::isinf(z) ? 0.0 : std::exp(-0.5 * z * z) / std::sqrt(2.0 * M_PI); }

static double std_quantile(double p)
{
    double lo = -40, hi = 40;
    for (int i = 0; i < 200; ++i) {
        double mid = 0.5 * (lo + hi);
        if (1.0 - std_cdf_upper(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
}

// round a double to the nearest binary16 value (ties to even); returns it as double
static double round_to_half(double x)
{
    if (x == 0.0 || !std::isfinite(x)) return x;
    double ax = std::fabs(x);
    if (ax >= 65520.0) return std::copysign(INFINITY, x);
    int e = std::ilogb(ax);                 // ax in [2^e, 2^(e+1))
    int q = (e < -14 ? -14 : e) - 10;       // spacing 2^q (subnormals: 2^-24)
    double scaled = std::ldexp(ax, -q);     // exact
    double r = std::nearbyint(scaled);      // ties-to-even in the default mode
    return std::copysign(std::ldexp(r, q), x);
}

// analytic E[(Y - c(Y))^2] under N(0, sigma^2) for cells split at t
static double gauss_distortion(double sigma, int L, const double* c, const double* t)
{
    double D = 0;
    for (int l = 0; l < L; ++l) {
        double a = (l == 0) ? -INFINITY : t[l - 1] / sigma;
        double b = (l == L - 1) ? INFINITY : t[l] / sigma;
        double m0 = std_mass(a, b);
        double m1 = sigma * (std_pdf(a) - std_pdf(b));
        double ta = std::isinf(a) ? 0.0 : a * std_pdf(a);
        double tb = std::isinf(b) ? 0.0 : b * std_pdf(b);
        double m2 = sigma * sigma * (m0 + ta - tb);
        D += m2 - 2 * c[l] * m1 + c[l] * c[l] * m0;
    }
    return D;
}

// ---- the exact coordinate law of a random unit vector in R^d (TQ_LAW_SPHERE)
//
// With t = cos(theta) the density K (1 - t^2)^((d-3)/2) dt becomes
// K sin(theta)^(d-2) d(theta), smooth on [0, pi], so cell masses are
// integrated in theta by composite Gauss-Legendre rules (pieces narrower than
// the density's width, where a 24-point rule is exact to rounding). K is the
// inverse of the Wallis integral W(d-2) = int_0^pi sin^(d-2). The first moment
// has the closed form K (1 - t^2)^((d-1)/2) / (d - 1) between the cell ends.

struct GaussLegendre {
    double x[24], w[24];
    GaussLegendre()
    {
        const int n = 24;
        for (int i = 0; i < n; ++i) {
            double z = std::cos(M_PI * (i + 0.75) / (n + 0.5)), dp = 1.0;
            for (int it = 0; it < 100; ++it) {
                double p0 = 1.0, p1 = z;  // Legendre recurrence up to P_n
                for (int k = 2; k <= n; ++k) {
                    const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
                    p0 = p1;
                    p1 = p2;
                }
                dp = n * (z * p1 - p0) / (z * z - 1.0);
                const double dz = p1 / dp;
                z -= dz;
                if (std::fabs(dz) <= 1e-16) break;
            }
            x[i] = z;
            w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
        }
    }
};

static const GaussLegendre& gauss_legendre()
{
    static const GaussLegendre g;
    return g;
}

// int_{th0}^{th1} sin(th)^p cos(th)^k d(th), pieces no wider than h
static double sin_pow_integral(double th0, double th1, double p, int k, double h)
{
    if (th1 <= th0) return 0.0;
    const GaussLegendre& g = gauss_legendre();
    const int pieces = (int)std::ceil((th1 - th0) / h);
    const double wdt = (th1 - th0) / pieces;
    double sum = 0.0;
    for (int j = 0; j < pieces; ++j) {
        const double mid = th0 + (j + 0.5) * wdt;
        double part = 0.0;
        for (int i = 0; i < 24; ++i) {
            const double th = mid + 0.5 * wdt * g.x[i];
            const double sn = std::sin(th);
            double f = sn > 0 ? std::exp(p * std::log(sn)) : (p == 0 ? 1.0 : 0.0);
            if (k) f *= std::pow(std::cos(th), k);
            part += g.w[i] * f;
        }
        sum += 0.5 * wdt * part;
    }
    return sum;
}

struct SphereLaw {
    int d;
    double K, h;
    explicit SphereLaw(int dim) : d(dim)
    {
        double W = (dim - 2) % 2 ? 2.0 : M_PI;  // Wallis: W(n) = (n - 1) / n W(n - 2)
        for (int n = (dim - 2) % 2 ? 3 : 2; n <= dim - 2; n += 2) W *= (n - 1.0) / n;
        K = 1.0 / W;
        h = std::fmin(0.25, 1.5 / std::sqrt((double)dim));
    }
    double mass(double a, double b) const
    {
        a = std::fmax(a, -1.0);
        b = std::fmin(b, 1.0);
        return b > a ? K * sin_pow_integral(std::acos(b), std::acos(a), d - 2.0, 0, h) : 0.0;
    }
    double first(double a, double b) const
    {
        a = std::fmax(a, -1.0);
        b = std::fmin(b, 1.0);
        if (b <= a) return 0.0;
        const double e = 0.5 * (d - 1);
        return K / (d - 1) * (std::pow(1.0 - a * a, e) - std::pow(1.0 - b * b, e));
    }
    double second(double a, double b) const
    {
        a = std::fmax(a, -1.0);
        b = std::fmin(b, 1.0);
        return b > a ? K * sin_pow_integral(std::acos(b), std::acos(a), d - 2.0, 2, h) : 0.0;
    }
    // the p-quantile, by bisection on the mass below
    double quantile(double p) const
    {
        double lo = -1.0, hi = 1.0;
        for (int i = 0; i < 80; ++i) {
            const double mid = 0.5 * (lo + hi);
            if (mass(-1.0, mid) < p) lo = mid; else hi = mid;
        }
        return 0.5 * (lo + hi);
    }
};

static int codebook_sphere(int d, int bits, float* cent, float* bnd, double* dist)
{
    if (d < 2) return fail(TQ_ERR_UNSUPPORTED, "tq_codebook: the exact law needs d >= 2 (d=%d)", d);
    const int L = 1 << bits;
    const SphereLaw law(d);
    const double sigma = 1.0 / std::sqrt((double)d);
    double c[256], t[256], cn[256];
    for (int l = 0; l < L; ++l) c[l] = law.quantile((l + 0.5) / L);
    const double tol = (bits <= 4 ? 1e-13 : 1e-12) * sigma;
    bool done = false;
    for (int it = 0; it < 200000 && !done; ++it) {
        for (int l = 0; l + 1 < L; ++l) t[l] = 0.5 * (c[l] + c[l + 1]);
        for (int l = 0; l < L; ++l) {
            const double a = l == 0 ? -1.0 : t[l - 1], b = l == L - 1 ? 1.0 : t[l];
            const double m0 = law.mass(a, b);
            cn[l] = m0 > 0 ? law.first(a, b) / m0 : c[l];
        }
        for (int l = 0; l < L / 2; ++l) {  // symmetric law: keep the solution antisymmetric
            const double v = 0.5 * (cn[L - 1 - l] - cn[l]);
            cn[l] = -v;
            cn[L - 1 - l] = v;
        }
        double move = 0;
        for (int l = 0; l < L; ++l) {
            move = std::fmax(move, std::fabs(cn[l] - c[l]));
            c[l] = cn[l];
        }
        done = move < tol;
    }
    if (!done) return fail(TQ_ERR_NOCONV, "tq_codebook: no convergence for d=%d bits=%d (exact law)", d, bits);
    double cs[256], ts[256];
    for (int l = 0; l < L; ++l) {
        cs[l] = round_to_half(c[l]);
        cent[l] = (float)cs[l];
    }
    for (int l = 0; l + 1 < L; ++l) {
        bnd[l] = (float)(0.5 * (cs[l] + cs[l + 1]));
        ts[l] = (double)bnd[l];
    }
    if (dist) {
        double D = 0;
        for (int l = 0; l < L; ++l) {
            const double a = l == 0 ? -1.0 : ts[l - 1], b = l == L - 1 ? 1.0 : ts[l];
            D += law.second(a, b) - 2 * cs[l] * law.first(a, b) + cs[l] * cs[l] * law.mass(a, b);
        }
        *dist = D;
    }
    return TQ_OK;
}

int codebook(int d, int bits, int law, float* cent, float* bnd, double* dist)
{
    if (!cent || !bnd) return fail(TQ_ERR_INVALID, "tq_codebook: null output");
    if (law != TQ_LAW_GAUSSIAN && law != TQ_LAW_SPHERE)
        return fail(TQ_ERR_UNSUPPORTED, "tq_codebook: law %d unsupported", law);
    if (d < 1 || d > 65536) return fail(TQ_ERR_UNSUPPORTED, "tq_codebook: d=%d outside 1..65536", d);
    if (bits < 1 || bits > 8) return fail(TQ_ERR_UNSUPPORTED, "tq_codebook: bits=%d outside 1..8", bits);
    if (law == TQ_LAW_SPHERE) return codebook_sphere(d, bits, cent, bnd, dist);
    const int L = 1 << bits;
    const double sigma = 1.0 / std::sqrt((double)d);
    double c[256], t[256], cn[256];
    for (int l = 0; l < L; ++l) c[l] = sigma * std_quantile((l + 0.5) / L);
    const double tol = (bits <= 4 ? 1e-15 : 1e-12) * sigma;
    bool done = false;
    for (int it = 0; it < 4000000 && !done; ++it) {
        for (int l = 0; l + 1 < L; ++l) t[l] = 0.5 * (c[l] + c[l + 1]);
        for (int l = 0; l < L; ++l) {
            double a = (l == 0) ? -INFINITY : t[l - 1] / sigma;
            double b = (l == L - 1) ? INFINITY : t[l] / sigma;
            double m0 = std_mass(a, b);
            cn[l] = m0 > 0 ? sigma * (std_pdf(a) - std_pdf(b)) / m0 : c[l];
        }
        // the law is symmetric: keep the solution exactly antisymmetric
        for (int l = 0; l < L / 2; ++l) {
            double v = 0.5 * (cn[L - 1 - l] - cn[l]);
            cn[l] = -v;
            cn[L - 1 - l] = v;
        }
        double move = 0;
        for (int l = 0; l < L; ++l) {
            move = std::fmax(move, std::fabs(cn[l] - c[l]));
            c[l] = cn[l];
        }
        done = move < tol;
    }
    if (!done) return fail(TQ_ERR_NOCONV, "tq_codebook: no convergence for d=%d bits=%d", d, bits);
    double cs[256], ts[256];
    for (int l = 0; l < L; ++l) {
        cs[l] = round_to_half(c[l]);
        cent[l] = (float)cs[l];
    }
    for (int l = 0; l + 1 < L; ++l) {
        bnd[l] = (float)(0.5 * (cs[l] + cs[l + 1]));   // exact midpoint, then RNE to fp32
        ts[l] = (double)bnd[l];
    }
    if (dist) *dist = gauss_distortion(sigma, L, cs, ts);
    return TQ_OK;
}

// ---------------------------------------------------------------- validation

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_quantizer(const tq_quantizer* q, const char* who, const char* role)
{
    if (!q) return fail(TQ_ERR_INVALID, "%s: %s quantizer is NULL", who, role);
    if (q->d != 64 && q->d != 128 && q->d != 256)
        return fail(TQ_ERR_UNSUPPORTED, "%s: %s d=%d not in {64,128,256}", who, role, q->d);
    if (q->mse_bits < 1 || q->mse_bits > 8)
        return fail(TQ_ERR_UNSUPPORTED, "%s: %s mse_bits=%d not in 1..8", who, role, q->mse_bits);
    if (q->qjl_m != 0 && q->qjl_m != q->d)
        return fail(TQ_ERR_UNSUPPORTED, "%s: %s qjl_m=%d must be 0 or d", who, role, q->qjl_m);
    if (!q->centroids || !q->boundaries || !q->diag_signs)
        return fail(TQ_ERR_INVALID, "%s: %s quantizer has a NULL table", who, role);
    if (!aligned(q->centroids, 16) || !aligned(q->boundaries, 16) || !aligned(q->diag_signs, 16))
        return fail(TQ_ERR_INVALID, "%s: %s quantizer tables must be 16-byte aligned", who, role);
    if (q->qjl_m) {
        if (!q->S) return fail(TQ_ERR_INVALID, "%s: %s S is NULL with qjl_m=%d", who, role, q->qjl_m);
        if (!aligned(q->S, 16)) return fail(TQ_ERR_INVALID, "%s: %s S must be 16-byte aligned", who, role);
    }
    return TQ_OK;
}

int check_packed(const tq_quantizer* q, const tq_packed* p, const char* who, const char* role)
{
    if (!p) return fail(TQ_ERR_INVALID, "%s: %s packed descriptor is NULL", who, role);
    if (!p->codes || !p->norm) return fail(TQ_ERR_INVALID, "%s: %s codes/norm NULL", who, role);
    if (!aligned(p->codes, 16)) return fail(TQ_ERR_INVALID, "%s: %s codes must be 16-byte aligned", who, role);
    if (!aligned(p->norm, 2)) return fail(TQ_ERR_INVALID, "%s: %s norm must be 2-byte aligned", who, role);
    if (q->qjl_m) {
        if (!p->signs || !p->rnorm) return fail(TQ_ERR_INVALID, "%s: %s signs/rnorm NULL with qjl_m>0", who, role);
        if (!aligned(p->signs, 16)) return fail(TQ_ERR_INVALID, "%s: %s signs must be 16-byte aligned", who, role);
        if (!aligned(p->rnorm, 2)) return fail(TQ_ERR_INVALID, "%s: %s rnorm must be 2-byte aligned", who, role);
    }
    return TQ_OK;
}

int check_dense(const void* p, int dtype, const char* who, const char* what)
{
    if (!p) return fail(TQ_ERR_INVALID, "%s: %s is NULL", who, what);
    if (dtype != TQ_F32 && dtype != TQ_F16) return fail(TQ_ERR_INVALID, "%s: %s dtype %d unknown", who, what, dtype);
    if (!aligned(p, 16)) return fail(TQ_ERR_INVALID, "%s: %s must be 16-byte aligned", who, what);
    return TQ_OK;
}

// workspace layout helpers (sizes in bytes, each region 256-byte aligned)
static size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t scores_frag_bytes(const tq_quantizer* q, int64_t n_q)
{
    // d = 128: per tile of 8 queries, d/32 code and (QJL) d/32 sign k-steps of
    // 64 lanes x 16 bytes
    const size_t ksteps = (size_t)(q->d / 32) * (q->qjl_m ? 2 : 1);
    return up256((size_t)((n_q + 7) / 8) * ksteps * 64 * 16);
}

size_t scores_ws(const tq_quantizer* q, int64_t n_q)
{
    // d = 128: MFMA query fragments; else prepared queries: fp32 q' [n_q][d]
    // and p = S q' [n_q][m]
    if (q->d == 128) return scores_frag_bytes(q, n_q);
    return up256((size_t)n_q * q->d * 4) + up256((size_t)n_q * (q->qjl_m ? q->qjl_m : 1) * 4);
}

DecodePlan decode_plan(const tq_quantizer* qk, int64_t n_streams, int64_t T, int G, bool wide, bool append)
{
    DecodePlan p{};
    p.mfma = qk->d == 128 && G <= 8 && !wide;
    p.fused_append = p.mfma && append;
    // with the fused append the blocks scan the T - 1 cached tokens (at least
    // one block per stream, which also quantizes the new token)
    const int64_t Ts = p.fused_append ? (T - 1 > 1 ? T - 1 : 1) : T;
    if (p.mfma) {
        // spread the n_streams * T tokens over at most kDecodeSlots equal chunks
        // (multiples of 128 tokens: four waves of 32-token steps). With more
        // streams than slots, the chunks per stream (up to 8) that fill whole
        // rounds of slots best: 640 streams take 4 (2560 blocks, 5 full rounds)
        // rather than 1 (640 blocks, the second round a quarter full).
        int64_t per = kDecodeSlots / n_streams;
        if (per < 1) {
            double best = 0;
            for (int64_t c = 1; c <= 8; ++c) {
                const int64_t rounds = (n_streams * c + kDecodeSlots - 1) / kDecodeSlots;
                const double cost = (double)rounds / (double)c;
                if (c == 1 || cost < best - 1e-9) {
                    best = cost;
                    per = c;
                }
            }
        }
        int64_t tc = (Ts + per - 1) / per;
        tc = (tc + 127) / 128 * 128;
        p.tc = tc;
    } else {
        p.tc = 256;  // the scalar kernel handles one token per thread
    }
    p.n_chunks = (int)((Ts + p.tc - 1) / p.tc);
    p.pchunks = p.n_chunks + (p.fused_append ? 1 : 0);
    const size_t nq = (size_t)n_streams * G;
    // prepared queries (scalar kernels; the MFMA kernel prepares its own), then partials
    p.off_qr = 0;
    p.off_p = p.mfma ? 0 : up256(nq * qk->d * 4);
    p.off_parts = p.off_p + (p.mfma ? 0 : up256(nq * (qk->qjl_m ? qk->qjl_m : 1) * 4));
    p.total = p.off_parts + up256((size_t)n_streams * p.pchunks * G * part_stride(qk->d) * 4);
    return p;
}

}  // namespace tq

extern "C" {

int tq_codebook(int d, int bits, int law, float* centroids, float* boundaries, double* distortion)
{
    tq::clear_error();
    return tq::codebook(d, bits, law, centroids, boundaries, distortion);
}

size_t tq_workspace_size(int op, const tq_quantizer* qk, int64_t n_a, int64_t n_b, int G)
{
    if (!qk || n_a < 0 || n_b < 0) return 0;
    if (qk->d != 64 && qk->d != 128 && qk->d != 256) return 0;
    if (qk->qjl_m != 0 && qk->qjl_m != qk->d) return 0;
    if (op == TQ_OP_SCORES) return tq::scores_ws(qk, n_a);
    if (op == TQ_OP_DECODE_ATTN) {
        if (G < 1 || G > 16 || n_b < 1) return 0;
        // the value width is not an argument: enough for either kernel family
        // also the decode step's plan (n_b tokens with the new one)
        const size_t a = tq::decode_plan(qk, n_a, n_b, G, false).total;
        const size_t b = tq::decode_plan(qk, n_a, n_b, G, true).total;
        const size_t c = tq::decode_plan(qk, n_a, n_b, G, false, true).total;
        const size_t ab = a > b ? a : b;
        return ab > c ? ab : c;
    }
    return 0;
}

const char* tq_last_error(void) { return tq::g_err; }

}  // extern "C"
