// GPU twin of synth/__init__.py: the same counter-based SplitMix64 draws and
// Box-Muller normals, evaluated with the same sequence of IEEE double
// operations (this file is built with -ffp-contraction off, divisions and
// square roots use the correctly rounded intrinsics), so element i has the
// same bits on the host and on the device. No arithmetic of the compression
// method lives here.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline double uniform(uint64_t key, uint64_t i)
{
    uint64_t d = mix(key + (i + 1) * kGolden);
    return (double)(d >> 11) * 0x1.0p-53;
}

constexpr double kLn2 = 0.6931471805599453;
constexpr double kSqrt2 = 1.4142135623730951;
constexpr double kHalfPi = 1.5707963267948966;

struct Tables {
    double inv_odd[12];
    double inv_fact[25];
};

__device__ inline void make_tables(Tables& t)
{
    for (int j = 0; j < 12; ++j) t.inv_odd[j] = __ddiv_rn(1.0, (double)(2 * j + 1));
    double c = 1.0;
    t.inv_fact[0] = 1.0;
    for (int k = 1; k <= 24; ++k) {
        c = __ddiv_rn(c, (double)k);
        t.inv_fact[k] = c;
    }
}

// ln x for x in (0, 1]: x = f 2^e with f in [1, 2), folded to [1/sqrt2, sqrt2]
__device__ inline double ln01(double x, const Tables& t)
{
    uint64_t b = (uint64_t)__double_as_longlong(x);
    double e = (double)((int)((b >> 52) & 0x7FF) - 1023);
    double f = __longlong_as_double((long long)((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull));
    if (f > kSqrt2) {
        f = f * 0.5;
        e = e + 1.0;
    }
    double s = __ddiv_rn(f - 1.0, f + 1.0);
    double s2 = s * s;
    double p = t.inv_odd[11];
    for (int j = 10; j >= 0; --j) p = p * s2 + t.inv_odd[j];
    double tt = 2.0 * s;
    tt = tt * p;
    return e * kLn2 + tt;
}

__device__ inline void sincos_2pi(double u, const Tables& t, double* sn, double* cs)
{
    double v = u * 4.0;
    double q = floor(v);
    double f = v - q;
    double a = f * kHalfPi;
    double a2 = a * a;
    double ps = t.inv_fact[21];
    for (int k = 9; k >= 0; --k) ps = t.inv_fact[2 * k + 1] - ps * a2;
    double s = a * ps;
    double pc = t.inv_fact[22];
    for (int k = 10; k >= 0; --k) pc = t.inv_fact[2 * k] - pc * a2;
    int qi = (int)q;
    double so, co;
    if (qi == 0) { so = s; co = pc; }
    else if (qi == 1) { so = pc; co = -s; }
    else if (qi == 2) { so = -s; co = -pc; }
    else { so = -pc; co = s; }
    *sn = so;
    *cs = co;
}

__device__ inline double normal(uint64_t key, int64_t e, const Tables& t)
{
    uint64_t j = (uint64_t)(e / 2);
    double u1 = 1.0 - uniform(key, 2 * j);
    double u2 = uniform(key, 2 * j + 1);
    double r = __dsqrt_rn(-2.0 * ln01(u1, t));
    double sn, cs;
    sincos_2pi(u2, t, &sn, &cs);
    return (e % 2 == 0) ? r * cs : r * sn;
}

__global__ void k_fill_f16(uint64_t key, int64_t first, int64_t n, int d, int64_t tokens,
                           const double* __restrict__ scales, uint16_t* __restrict__ out)
{
    Tables t;
    make_tables(t);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t e = first + i;
        double z = normal(key, e, t);
        if (scales) {
            int64_t vec = e / d;
            z = z * scales[(vec / tokens) * d + (e % d)];
        }
        float f = (float)z;
        out[i] = __half_as_ushort(__float2half_rn(f));
    }
}

__global__ void k_fill_f32(uint64_t key, int64_t first, int64_t n, float* __restrict__ out)
{
    Tables t;
    make_tables(t);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = (float)normal(key, first + i, t);
}

// normalised N(0, I) vectors, norm summed in index order (one thread per vector)
__global__ void k_unit_f32(uint64_t key, int64_t first_vec, int64_t nvec, int d, float* __restrict__ out)
{
    Tables t;
    make_tables(t);
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * blockDim.x) {
        int64_t e0 = (first_vec + v) * d;
        double acc = 0.0;
        for (int i = 0; i < d; ++i) {
            double z = normal(key, e0 + i, t);
            acc = acc + z * z;
        }
        double nrm = __dsqrt_rn(acc);
        for (int i = 0; i < d; ++i) out[v * d + i] = (float)__ddiv_rn(normal(key, e0 + i, t), nrm);
    }
}

inline uint64_t stream_key(uint64_t seed, int role) { return mix(seed + (uint64_t)(role + 1) * kGolden); }

inline unsigned grid_of(int64_t n, int per)
{
    int64_t b = (n + per - 1) / per;
    return (unsigned)(b < 16384 ? b : 16384);
}

}  // namespace

extern "C" {

// out[i] = fp16(fp32(normal(first + i) * scales[group][channel])), group = vector / tokens
int synth_fill_f16(uint64_t seed, int role, int64_t first, int64_t n, int d, int64_t tokens,
                   const double* scales, uint16_t* out, void* stream)
{
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_fill_f16, dim3(grid_of(n, 256)), dim3(256), 0, (hipStream_t)stream,
                       stream_key(seed, role), first, n, d, tokens > 0 ? tokens : 1, scales, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int synth_fill_f32(uint64_t seed, int role, int64_t first, int64_t n, float* out, void* stream)
{
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_fill_f32, dim3(grid_of(n, 256)), dim3(256), 0, (hipStream_t)stream,
                       stream_key(seed, role), first, n, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

int synth_unit_f32(uint64_t seed, int role, int64_t first_vec, int64_t nvec, int d, float* out,
                   void* stream)
{
    if (nvec <= 0) return 0;
    hipLaunchKernelGGL(k_unit_f32, dim3(grid_of(nvec, 128)), dim3(128), 0, (hipStream_t)stream,
                       stream_key(seed, role), first_vec, nvec, d, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
