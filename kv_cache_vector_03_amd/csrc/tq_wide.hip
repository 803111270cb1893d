// Wide codes: MSE code widths of 5 to 8 bits (up to 256 Lloyd-Max levels)
// for any d in {64, 128, 256}, with the width a run-time argument.
//
// The method is the same as for the narrow widths ("[Benchmark] TurboQuant
// 實測：KV Cache 3-bit 壓縮，真的零損失？", section "TurboQuant 是什麼：30 秒懶人包":
// random rotation, stored norm, per-coordinate Lloyd-Max codes, for keys a
// 1-bit sketch of the residual plus its norm; wider caches such as the 8-bit
// key / 4-bit value split are among the modes measured in the vLLM benchmark
// summary, section "vLLM 工程師的實測", table of quantization modes). The
// packed layout is the group-major stream the
// narrow kernels write: group c (coordinates c + (d/8) t, t = 0..7) occupies
// stream bits [8 b c, 8 b c + 8 b), code t at bits [b t, b t + b).
//
// These kernels favour plainness over speed (the narrow kernels carry the
// hot configurations): one wave per vector for quantize and dequantize, the
// code of a coordinate found by binary search over the boundaries held in
// LDS, and scalar score and decode kernels that read each code straight from
// its (at most two) stream words.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWaves = 4;      // waves per block (one vector each)
constexpr int kMaxL = 256;     // levels of an 8-bit codebook
constexpr int kQT = 16;        // queries per LDS tile in the score kernel
constexpr int kTC = 256;       // tokens per decode chunk (one per thread)
constexpr int kMaxG = 16;

// Code of coordinate i (b-bit codes, group-major stream cv of d/32 * b words).
__device__ __forceinline__ int wide_code(const uint32_t* cv, int d, int b, int i)
{
    const int g = d / 8;
    const int start = 8 * b * (i % g) + b * (i / g);
    const int w = start >> 5, off = start & 31;
    uint32_t v = cv[w] >> off;
    if (off + b > 32) v |= cv[w + 1] << (32 - off);
    return (int)(v & ((1u << b) - 1u));
}

// #{l : t_l < y} over the L - 1 ascending boundaries t (L = 2^b): a
// branch-free binary search, the count the codebook's strict comparison
// defines.
__device__ __forceinline__ int wide_index(const float* t, int b, float y)
{
    int k = 0;
    for (int step = 1 << (b - 1); step >= 1; step >>= 1) k += t[k + step - 1] < y ? step : 0;
    return k;
}

// One wave per vector: rotation, norm, codes (binary search), group-major
// packing (one lane per group), and for keys the residual, its norm and the
// sign sketch u = S r (one projection row per lane and pass).
template <int D, bool QJL, bool F16>
__global__ __launch_bounds__(64 * kWaves) void k_quantize_wide(const void* __restrict__ x, int64_t n, int b,
                                                              const float* __restrict__ cent,
                                                              const float* __restrict__ bnd,
                                                              const uint32_t* __restrict__ diag,
                                                              const uint16_t* __restrict__ S,
                                                              uint32_t* __restrict__ codes,
                                                              uint32_t* __restrict__ signs,
                                                              uint16_t* __restrict__ norm,
                                                              uint16_t* __restrict__ rnorm)
{
    constexpr int R = D / 64, G = D / 8;
    __shared__ float tb[kMaxL], cb[kMaxL];
    __shared__ float res[kWaves][D];
    __shared__ unsigned char cidx[kWaves][D];
    extern __shared__ uint16_t st[];  // QJL: S transposed, st[i * D + j] = S[j][i]
    const int L = 1 << b;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int l = threadIdx.x; l < L; l += blockDim.x) {
        cb[l] = cent[l];
        tb[l] = l < L - 1 ? bnd[l] : INFINITY;
    }
    constexpr bool ST = QJL && D <= 128;  // S^T in LDS (d = 256: 128 KiB, too much; rows read from S)
    if constexpr (ST)
        for (int e = threadIdx.x; e < D * D; e += blockDim.x) st[(e % D) * D + e / D] = S[e];
    __syncthreads();
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);
    const int cw = b * D / 32;  // code words per vector

    for (int64_t base = (int64_t)blockIdx.x * kWaves; base < n; base += (int64_t)gridDim.x * kWaves) {
        const int64_t v = base + wid;
        const bool active = v < n;
        float y[R];
        float ss = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            y[r] = active ? load_elem<F16>(x, v * D + 64 * r + lane) : 0.f;
            ss += y[r] * y[r];
        }
        const float nrm = sqrtf(wave_sum(ss));
#pragma unroll
        for (int r = 0; r < R; ++r) y[r] = flip(y[r], dm[r]);
        fwht_wave<R>(y, lane);
        const float sc = nrm > 0.f ? 1.0f / (sqrtf((float)D) * nrm) : 0.f;
        float g2 = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float yr = y[r] * sc;
            const int k = wide_index(tb, b, yr);
            cidx[wid][64 * r + lane] = (unsigned char)k;
            if constexpr (QJL) {
                const float rr = yr - cb[k];
                g2 += rr * rr;
                res[wid][64 * r + lane] = rr;
            }
        }
        __syncthreads();
        if (active && lane < G) {
            uint64_t f = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) f |= (uint64_t)cidx[wid][lane + G * t] << (b * t);
            unsigned char* dst = reinterpret_cast<unsigned char*>(codes + v * cw) + b * lane;
            for (int k = 0; k < b; ++k) dst[k] = (unsigned char)(f >> (8 * k));
        }
        if (active && lane == 0) norm[v] = f2h(nrm);
        if constexpr (QJL) {
            g2 = wave_sum(g2);
            uint32_t sb[R];
            // row j = 64 k + lane of S r: consecutive lanes read consecutive
            // entries of a row of S^T, the residual entry is a broadcast
            float u[R];
#pragma unroll
            for (int k = 0; k < R; ++k) u[k] = 0.f;
            if constexpr (ST) {
                for (int i = 0; i < D; ++i) {
                    const float ri = res[wid][i];
#pragma unroll
                    for (int k = 0; k < R; ++k) u[k] = fmaf(h2f(st[i * D + 64 * k + lane]), ri, u[k]);
                }
            } else {
                // each lane walks its own rows of S, 16 bytes (8 entries) per load
#pragma unroll
                for (int k = 0; k < R; ++k) {
                    const uint4* Sj = reinterpret_cast<const uint4*>(S + (int64_t)(64 * k + lane) * D);
                    for (int i8 = 0; i8 < D / 8; ++i8) {
                        const uint4 w = Sj[i8];
                        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            u[k] = fmaf(h2f((uint16_t)(ww[e >> 1] >> (16 * (e & 1)))), res[wid][8 * i8 + e], u[k]);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < R; ++k) sb[k] = u[k] >= 0.f ? 1u : 0u;
            __syncthreads();
#pragma unroll
            for (int k = 0; k < R; ++k) cidx[wid][64 * k + lane] = (unsigned char)sb[k];
            __syncthreads();
            if (active && lane < G) {
                uint32_t f = 0;
#pragma unroll
                for (int t = 0; t < 8; ++t) f |= (uint32_t)cidx[wid][lane + G * t] << t;
                reinterpret_cast<unsigned char*>(signs + v * (D / 32))[lane] = (unsigned char)f;
            }
            if (active && lane == 0) rnorm[v] = f2h(sqrtf(g2));
        }
        __syncthreads();
    }
}

// x_hat = n D H (c[idx] + [qjl] g sqrt(pi/2)/m S^T s) / sqrt(d), one wave per vector.
template <int D, bool QJL, bool F16OUT>
__global__ __launch_bounds__(64 * kWaves) void k_dequantize_wide(const uint32_t* __restrict__ codes,
                                                                const uint32_t* __restrict__ signs,
                                                                const uint16_t* __restrict__ norm,
                                                                const uint16_t* __restrict__ rnorm, int64_t n,
                                                                int b, const float* __restrict__ cent,
                                                                const uint32_t* __restrict__ diag,
                                                                const uint16_t* __restrict__ S,
                                                                void* __restrict__ out)
{
    constexpr int R = D / 64;
    __shared__ float cb[kMaxL];
    const int L = 1 << b;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int l = threadIdx.x; l < L; l += blockDim.x) cb[l] = cent[l];
    __syncthreads();
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);
    const int cw = b * D / 32;
    for (int64_t base = (int64_t)blockIdx.x * kWaves; base < n; base += (int64_t)gridDim.x * kWaves) {
        const int64_t v = base + wid;
        if (v >= n) continue;  // no block-level synchronisation below
        const uint32_t* cv = codes + v * cw;
        float a[R];
#pragma unroll
        for (int r = 0; r < R; ++r) a[r] = cb[wide_code(cv, D, b, 64 * r + lane)];
        if constexpr (QJL) {
            const float g = h2f(rnorm[v]) * (kSqrtHalfPi / (float)D);
            const uint32_t* sv = signs + v * (D / 32);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = 64 * r + lane;
                float acc = 0.f;
                for (int j = 0; j < D; ++j) {
                    const int P = sign_bit<D>(j);
                    const float sg = ((sv[P >> 5] >> (P & 31)) & 1u) ? 1.f : -1.f;
                    acc += h2f(S[(int64_t)j * D + i]) * sg;
                }
                a[r] += g * acc;
            }
        }
        fwht_wave<R>(a, lane);
        const float sc = h2f(norm[v]) / sqrtf((float)D);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float o = flip(a[r], dm[r]) * sc;
            const int64_t e = v * D + 64 * r + lane;
            if constexpr (F16OUT) static_cast<uint16_t*>(out)[e] = f2h(o);
            else static_cast<float*>(out)[e] = o;
        }
    }
}

// Scores from prepared queries (q' and p = S q', fp32, as the narrow scalar
// path prepares them): one key per thread, kQT queries per LDS tile, double
// accumulation (scores reach |n||q| ~ 10^2-10^3).
template <int D, bool QJL>
__global__ __launch_bounds__(256) void k_scores_wide(const uint32_t* __restrict__ codes,
                                                     const uint32_t* __restrict__ signs,
                                                     const uint16_t* __restrict__ norm,
                                                     const uint16_t* __restrict__ rnorm, int64_t n_keys, int b,
                                                     const float* __restrict__ qr, const float* __restrict__ p,
                                                     int64_t n_q, const float* __restrict__ cent,
                                                     float* __restrict__ scores)
{
    constexpr int W = D / 32;
    __shared__ float sq[kQT][D];
    __shared__ float sp[QJL ? kQT : 1][D];
    __shared__ float cb[kMaxL];
    const int L = 1 << b;
    for (int l = threadIdx.x; l < L; l += blockDim.x) cb[l] = cent[l];
    const int64_t key = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool act = key < n_keys;
    const uint32_t* cv = codes + (act ? key : 0) * (int64_t)(b * W);
    uint32_t sw[W];
#pragma unroll
    for (int w = 0; w < W; ++w) sw[w] = (QJL && act) ? signs[key * W + w] : 0u;
    double nk = 0.0, gk = 0.0;
    if (act) {
        nk = (double)h2f(norm[key]);
        if (QJL) gk = (double)h2f(rnorm[key]) * (1.2533141373155003 / D);
    }
    for (int64_t q0 = (int64_t)blockIdx.y * kQT; q0 < n_q; q0 += (int64_t)gridDim.y * kQT) {
        __syncthreads();
        for (int e = threadIdx.x; e < kQT * D; e += 256) {
            const int qi = e / D, i = e % D;
            const bool ok = q0 + qi < n_q;
            sq[qi][i] = ok ? qr[(q0 + qi) * D + i] : 0.f;
            if (QJL) sp[qi][i] = ok ? p[(q0 + qi) * D + i] : 0.f;
        }
        __syncthreads();
        double am[kQT], aj[kQT];
#pragma unroll
        for (int qi = 0; qi < kQT; ++qi) am[qi] = aj[qi] = 0.0;
        for (int i = 0; i < D; ++i) {
            const double c = act ? (double)cb[wide_code(cv, D, b, i)] : 0.0;
            const int SP = sign_bit<D>(i);
            const bool pos = (sw[SP >> 5] >> (SP & 31)) & 1u;
#pragma unroll
            for (int qi = 0; qi < kQT; ++qi) {
                am[qi] += (double)sq[qi][i] * c;
                if (QJL) aj[qi] += pos ? (double)sp[qi][i] : -(double)sp[qi][i];
            }
        }
        if (act) {
            const int nq = (int)((n_q - q0) < kQT ? (n_q - q0) : kQT);
#pragma unroll
            for (int qi = 0; qi < kQT; ++qi)
                if (qi < nq) scores[(q0 + qi) * n_keys + key] = (float)(nk * (am[qi] + gk * aj[qi]));
        }
    }
}

// Decode attention over one chunk of kTC tokens of one stream (grid: chunks x
// streams), any key width bk and value width bv in 1..8. The chunk's key and
// value code rows are staged in LDS with coalesced loads (key rows padded to
// an odd word stride, so the per-token reads of phase A do not collide).
// Phase A scores this thread's token for the G heads, four coordinates per
// query read; phase B takes the chunk-local softmax per head and folds the
// value norms into the weights; phase C gives each thread one coordinate and
// a set of heads, so one code lookup serves all of them, and accumulates
// sum_t w_t n_t c_v[idx] in the rotated value domain. Each chunk writes a
// partial (max, sum, accumulator) that the combine kernel merges.
template <int D, bool QJL>
__global__ __launch_bounds__(256) void k_decode_wide(const uint32_t* __restrict__ kcodes,
                                                     const uint32_t* __restrict__ ksigns,
                                                     const uint16_t* __restrict__ knorm,
                                                     const uint16_t* __restrict__ krnorm, int bk,
                                                     const uint32_t* __restrict__ vcodes,
                                                     const uint16_t* __restrict__ vnorm, int bv, int64_t T,
                                                     int64_t stride, int G, const float* __restrict__ qr,
                                                     const float* __restrict__ p,
                                                     const float* __restrict__ kcent,
                                                     const float* __restrict__ vcent, float scale,
                                                     float* __restrict__ parts, int n_chunks, int64_t s0)
{
    constexpr int W = D / 32;
    constexpr int KROW = 8 * W + 1;          // staged key row stride (words)
    constexpr int TPC = 256 / D;             // phase C threads per coordinate
    constexpr int HPT = (kMaxG + TPC - 1) / TPC;  // heads per phase C thread (at most)
    // dynamic LDS, sized for the call's G: queries q' [G][D], projections p
    // [G][D] (QJL), scores then weights times value norms z [G][kTC]
    extern __shared__ __align__(16) float dsm[];
    float(*sq)[D] = reinterpret_cast<float(*)[D]>(dsm);
    float(*sp)[D] = reinterpret_cast<float(*)[D]>(dsm + G * D);
    float(*z)[kTC] = reinterpret_cast<float(*)[kTC]>(dsm + (QJL ? 2 : 1) * G * D);
    __shared__ uint32_t ks[kTC * KROW];      // key code rows (phase A), value code rows (phase C)
    __shared__ float kc[kMaxL], vc[kMaxL];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t s = s0 + blockIdx.y;  // launches cover at most 65535 streams each
    const int chunk = blockIdx.x;
    const int64_t t0 = (int64_t)chunk * kTC;
    const int64_t row0 = s * stride + t0;     // first vector of the chunk
    const int nt = (int)(T - t0 < kTC ? T - t0 : kTC);  // tokens in this chunk
    const int kw = bk * W, vwn = bv * W;  // code words per key / value
    for (int l = tid; l < (1 << bk); l += 256) kc[l] = kcent[l];
    for (int l = tid; l < (1 << bv); l += 256) vc[l] = vcent[l];
    for (int e = tid; e < G * D; e += 256) {
        const int h = e / D, i = e % D;
        sq[h][i] = qr[(s * G + h) * D + i];
        if (QJL) sp[h][i] = p[(s * G + h) * D + i];
    }
    for (int e = tid; e < nt * kw; e += 256) ks[(e / kw) * KROW + e % kw] = kcodes[row0 * kw + e];
    __syncthreads();

    // phase A: scores of this thread's token for all heads
    if (tid < nt) {
        float am[kMaxG], aj[kMaxG];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) am[h] = aj[h] = 0.f;
        const int64_t v = row0 + tid;
        const uint32_t* cv = ks + tid * KROW;
        uint32_t sw[W];
#pragma unroll
        for (int w = 0; w < W; ++w) sw[w] = QJL ? ksigns[v * W + w] : 0u;
#pragma unroll 2
        for (int i0 = 0; i0 < D; i0 += 4) {
            float c[4], sg[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[k] = kc[wide_code(cv, D, bk, i0 + k)];
                const int SP = sign_bit<D>(i0 + k);
                sg[k] = ((sw[SP >> 5] >> (SP & 31)) & 1u) ? 1.f : -1.f;
            }
#pragma unroll
            for (int h = 0; h < kMaxG; ++h)
                if (h < G) {
                    const float4 q4 = *reinterpret_cast<const float4*>(&sq[h][i0]);
                    am[h] += q4.x * c[0] + q4.y * c[1] + q4.z * c[2] + q4.w * c[3];
                    if (QJL) {
                        const float4 p4 = *reinterpret_cast<const float4*>(&sp[h][i0]);
                        aj[h] += p4.x * sg[0] + p4.y * sg[1] + p4.z * sg[2] + p4.w * sg[3];
                    }
                }
        }
        const float nk = h2f(knorm[v]);
        const float gk = QJL ? h2f(krnorm[v]) * (kSqrtHalfPi / (float)D) : 0.f;
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
            if (h < G) z[h][tid] = nk * (am[h] + gk * aj[h]) * scale;
    } else {
#pragma unroll
        for (int h = 0; h < kMaxG; ++h)
            if (h < G) z[h][tid] = -INFINITY;
    }
    __syncthreads();  // the key rows are no longer read: the buffer takes the value rows

    for (int e = tid; e < nt * vwn; e += 256) ks[(e / vwn) * KROW + e % vwn] = vcodes[row0 * vwn + e];
    // phase B: chunk-local softmax per head (one wave per head, round robin);
    // the weights are stored times the token's value norm
    for (int h = wid; h < G; h += 4) {
        float m = -INFINITY;
        for (int tt = lane; tt < kTC; tt += 64) m = fmaxf(m, z[h][tt]);
        m = wave_max(m);
        float l = 0.f;
        for (int tt = lane; tt < kTC; tt += 64) {
            const float w = (z[h][tt] == -INFINITY) ? 0.f : exp2f(z[h][tt] - m);
            z[h][tt] = tt < nt ? w * h2f(vnorm[row0 + tt]) : 0.f;
            l += w;
        }
        l = wave_sum(l);
        if (lane == 0) {
            float* part = parts + (((int64_t)s * n_chunks + chunk) * G + h) * part_stride(D);
            part[0] = m;
            part[1] = l;
        }
    }
    __syncthreads();

    // phase C: coordinate i = tid % D, heads tid / D, tid / D + TPC, ...
    {
        const int i = tid % D, h0 = tid / D;
        const int start = 8 * bv * (i % (D / 8)) + bv * (i / (D / 8));  // code bit of coordinate i
        const int w = start >> 5, off = start & 31;
        const bool two = off + bv > 32;
        const uint32_t mask = (1u << bv) - 1u;
        float acc[HPT];
#pragma unroll
        for (int k = 0; k < HPT; ++k) acc[k] = 0.f;
#pragma unroll 4
        for (int tt = 0; tt < nt; ++tt) {
            const uint32_t* row = ks + tt * KROW;
            uint32_t cw = row[w] >> off;
            if (two) cw |= row[w + 1] << (32 - off);
            const float c = vc[cw & mask];
#pragma unroll
            for (int k = 0; k < HPT; ++k)
                if (h0 + TPC * k < G) acc[k] = fmaf(z[h0 + TPC * k][tt], c, acc[k]);
        }
#pragma unroll
        for (int k = 0; k < HPT; ++k) {
            const int h = h0 + TPC * k;
            if (h < G) parts[(((int64_t)s * n_chunks + chunk) * G + h) * part_stride(D) + kPartAcc + i] = acc[k];
        }
    }
}

int wide_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "%s: %s", who, hipGetErrorString(e));
    return TQ_OK;
}

unsigned wide_grid(int64_t units, int per_block)
{
    const int64_t b = (units + per_block - 1) / per_block;
    return (unsigned)(b < 65536 ? b : 65536);
}

// Launch with the dynamic LDS the kernel needs (S^T for keys) and a grid of
// resident blocks (each block stages S^T once and loops over vectors).
template <typename Kern>
void launch_wide_q(Kern kern, size_t lds, int64_t n, const void* x, int b, const tq_quantizer* q,
                   const tq_packed* o, hipStream_t s)
{
    static int cap = 0;  // resident blocks of this instance (same device for the process's launches)
    if (!cap) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
        int per = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kern, 64 * kWaves, lds) != hipSuccess || per < 1)
            per = 1;
        cap = per * device_cus();
    }
    int64_t want = (n + kWaves - 1) / kWaves;
    const unsigned grid = (unsigned)(want < cap ? want : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kWaves), lds, s, x, n, b, q->centroids, q->boundaries,
                       q->diag_signs, q->S, o->codes, o->signs, o->norm, o->rnorm);
}

template <int D>
void quantize_wide_d(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* o, hipStream_t s)
{
    const dim3 grid(wide_grid(n, kWaves)), block(64 * kWaves);
    const int b = q->mse_bits;
    if (q->qjl_m) {
        constexpr size_t lds = D <= 128 ? (size_t)D * D * 2 : 0;  // S^T for d <= 128
        if (dtype == TQ_F16) launch_wide_q(k_quantize_wide<D, true, true>, lds, n, x, b, q, o, s);
        else launch_wide_q(k_quantize_wide<D, true, false>, lds, n, x, b, q, o, s);
    } else {
        if (dtype == TQ_F16)
            hipLaunchKernelGGL((k_quantize_wide<D, false, true>), grid, block, 0, s, x, n, b, q->centroids,
                               q->boundaries, q->diag_signs, q->S, o->codes, o->signs, o->norm, o->rnorm);
        else
            hipLaunchKernelGGL((k_quantize_wide<D, false, false>), grid, block, 0, s, x, n, b, q->centroids,
                               q->boundaries, q->diag_signs, q->S, o->codes, o->signs, o->norm, o->rnorm);
    }
}

template <int D>
void dequantize_wide_d(const tq_quantizer* q, const tq_packed* in, int64_t n, int qjl, void* out, int dtype,
                       hipStream_t s)
{
    const dim3 grid(wide_grid(n, kWaves)), block(64 * kWaves);
    const int b = q->mse_bits;
    if (qjl) {
        if (dtype == TQ_F16)
            hipLaunchKernelGGL((k_dequantize_wide<D, true, true>), grid, block, 0, s, in->codes, in->signs, in->norm,
                               in->rnorm, n, b, q->centroids, q->diag_signs, q->S, out);
        else
            hipLaunchKernelGGL((k_dequantize_wide<D, true, false>), grid, block, 0, s, in->codes, in->signs,
                               in->norm, in->rnorm, n, b, q->centroids, q->diag_signs, q->S, out);
    } else {
        if (dtype == TQ_F16)
            hipLaunchKernelGGL((k_dequantize_wide<D, false, true>), grid, block, 0, s, in->codes, in->signs,
                               in->norm, in->rnorm, n, b, q->centroids, q->diag_signs, q->S, out);
        else
            hipLaunchKernelGGL((k_dequantize_wide<D, false, false>), grid, block, 0, s, in->codes, in->signs,
                               in->norm, in->rnorm, n, b, q->centroids, q->diag_signs, q->S, out);
    }
}

template <int D>
void scores_wide_d(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const float* qr, const float* p,
                   int64_t n_q, float* scores, hipStream_t s)
{
    const int64_t qt = (n_q + kQT - 1) / kQT;
    const dim3 grid((unsigned)((n_keys + 255) / 256), (unsigned)(qt < 65535 ? qt : 65535)), block(256);
    if (q->qjl_m)
        hipLaunchKernelGGL((k_scores_wide<D, true>), grid, block, 0, s, k->codes, k->signs, k->norm, k->rnorm, n_keys,
                           q->mse_bits, qr, p, n_q, q->centroids, scores);
    else
        hipLaunchKernelGGL((k_scores_wide<D, false>), grid, block, 0, s, k->codes, k->signs, k->norm, k->rnorm,
                           n_keys, q->mse_bits, qr, p, n_q, q->centroids, scores);
}

template <int D>
void decode_wide_d(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k, const tq_packed* v,
                   int64_t n_streams, int64_t T, int64_t stride, int G, const float* qr, const float* p,
                   float zscale, float* parts, int n_chunks, hipStream_t s)
{
    const size_t lds = ((size_t)(qk->qjl_m ? 2 : 1) * G * D + (size_t)G * kTC) * sizeof(float);
    // allow each instance the dynamic LDS of the largest G (d = 256 with the sketch and
    // G = 16 needs 48 KiB beside 65 KiB of static LDS)
    static bool sized[2] = {false, false};
    if (!sized[qk->qjl_m ? 1 : 0]) {
        const int most = (int)(((qk->qjl_m ? 2 : 1) * kMaxG * D + kMaxG * kTC) * sizeof(float));
        if (qk->qjl_m)
            (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_decode_wide<D, true>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, most);
        else
            (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_decode_wide<D, false>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, most);
        sized[qk->qjl_m ? 1 : 0] = true;
    }
    // grid.y is limited to 65535: streams go in launches of at most that many
    for (int64_t s0 = 0; s0 < n_streams; s0 += 65535) {
        const int64_t ns = n_streams - s0 < 65535 ? n_streams - s0 : 65535;
        const dim3 grid((unsigned)n_chunks, (unsigned)ns), block(256);
        if (qk->qjl_m)
            hipLaunchKernelGGL((k_decode_wide<D, true>), grid, block, lds, s, k->codes, k->signs, k->norm,
                               k->rnorm, qk->mse_bits, v->codes, v->norm, qv->mse_bits, T, stride, G, qr, p,
                               qk->centroids, qv->centroids, zscale, parts, n_chunks, s0);
        else
            hipLaunchKernelGGL((k_decode_wide<D, false>), grid, block, lds, s, k->codes, k->signs, k->norm,
                               k->rnorm, qk->mse_bits, v->codes, v->norm, qv->mse_bits, T, stride, G, qr, p,
                               qk->centroids, qv->centroids, zscale, parts, n_chunks, s0);
    }
}

}  // namespace

int launch_quantize_wide(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* out,
                         hipStream_t s)
{
    switch (q->d) {
        case 64: quantize_wide_d<64>(q, x, dtype, n, out, s); break;
        case 128: quantize_wide_d<128>(q, x, dtype, n, out, s); break;
        default: quantize_wide_d<256>(q, x, dtype, n, out, s); break;
    }
    return wide_status("tq_quantize");
}

int launch_dequantize_wide(const tq_quantizer* q, const tq_packed* in, int64_t n, int include_qjl, void* out,
                           int dtype, hipStream_t s)
{
    switch (q->d) {
        case 64: dequantize_wide_d<64>(q, in, n, include_qjl, out, dtype, s); break;
        case 128: dequantize_wide_d<128>(q, in, n, include_qjl, out, dtype, s); break;
        default: dequantize_wide_d<256>(q, in, n, include_qjl, out, dtype, s); break;
    }
    return wide_status("tq_dequantize");
}

int launch_scores_wide(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const float* qr, const float* p,
                       int64_t n_q, float* scores, hipStream_t s)
{
    switch (q->d) {
        case 64: scores_wide_d<64>(q, k, n_keys, qr, p, n_q, scores, s); break;
        case 128: scores_wide_d<128>(q, k, n_keys, qr, p, n_q, scores, s); break;
        default: scores_wide_d<256>(q, k, n_keys, qr, p, n_q, scores, s); break;
    }
    return wide_status("tq_scores");
}

int launch_decode_wide(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k, const tq_packed* v,
                       int64_t n_streams, int64_t T, int64_t stride, int G, const float* qr, const float* p,
                       float zscale, float* parts, int n_chunks, hipStream_t s)
{
    switch (qk->d) {
        case 64: decode_wide_d<64>(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, parts, n_chunks, s); break;
        case 128: decode_wide_d<128>(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, parts, n_chunks, s); break;
        default: decode_wide_d<256>(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, parts, n_chunks, s); break;
    }
    return wide_status("tq_decode_attn");
}

}  // namespace tq
