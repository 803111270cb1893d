// Quantize, query preparation and dequantize kernels.
//
// Quantize (one wave per vector; lane l, slot r holds coordinate 64 r + l):
//   norm by a wave reduction -> sign flips of the random diagonal -> wave
//   FWHT -> scale by 1/(sqrt(d) n) -> code index by counting boundaries below
//   each coordinate -> one ballot per bit plane and slot gives two packed
//   words directly (bit k of the ballot is coordinate 64 r + k) -> with QJL:
//   residual r = y - c[idx], its norm, projections S r (one row per lane),
//   and a ballot of the signs.
// The method is the two-stage quantizer of "[Benchmark] TurboQuant 實測：KV
// Cache 3-bit 壓縮，真的零損失？", section "TurboQuant 是什麼：30 秒懶人包".
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWavesPerBlock = 4;

template <int D, int B, bool QJL, bool F16>
__global__ __launch_bounds__(256) void k_quantize(const void* __restrict__ x, int64_t n,
                                                  const float* __restrict__ cent,
                                                  const float* __restrict__ bnd,
                                                  const uint32_t* __restrict__ diag,
                                                  const uint16_t* __restrict__ S,
                                                  uint32_t* __restrict__ codes,
                                                  uint32_t* __restrict__ signs,
                                                  uint16_t* __restrict__ norm,
                                                  uint16_t* __restrict__ rnorm)
{
    constexpr int R = D / 64, L = 1 << B, W = D / 32;
    __shared__ float res[kWavesPerBlock][D];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float t[L - 1], c[L];
#pragma unroll
    for (int l = 0; l < L - 1; ++l) t[l] = bnd[l];
#pragma unroll
    for (int l = 0; l < L; ++l) c[l] = cent[l];
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);

    for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < n;
         base += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t v = base + wid;
        const bool active = v < n;
        float y[R];
        int idx[R];
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
        uint32_t myword = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            y[r] *= sc;
            int k = 0;
#pragma unroll
            for (int l = 0; l < L - 1; ++l) k += (t[l] < y[r]) ? 1 : 0;
            idx[r] = k;
#pragma unroll
            for (int p = 0; p < B; ++p) {
                const uint64_t m = __ballot((k >> p) & 1);
                if (lane == p * W + 2 * r) myword = (uint32_t)m;
                if (lane == p * W + 2 * r + 1) myword = (uint32_t)(m >> 32);
            }
        }
        if (active) {
            if (lane < B * W) codes[v * (B * W) + lane] = myword;
            if (lane == 0) norm[v] = f2h(nrm);
        }
        if constexpr (QJL) {
            float g2 = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float rr = y[r] - pick<L>(c, idx[r]);
                g2 += rr * rr;
                res[wid][64 * r + lane] = rr;
            }
            g2 = wave_sum(g2);
            __syncthreads();
            uint32_t sword = 0;
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int j = 64 * k + lane;
                const uint16_t* Sj = S + (int64_t)j * D;
                float u = 0.f;
                for (int i = 0; i < D; ++i) u += h2f(Sj[i]) * res[wid][i];
                const uint64_t m = __ballot(u >= 0.f);
                if (lane == 2 * k) sword = (uint32_t)m;
                if (lane == 2 * k + 1) sword = (uint32_t)(m >> 32);
            }
            if (active) {
                if (lane < W) signs[v * W + lane] = sword;
                if (lane == 0) rnorm[v] = f2h(sqrtf(g2));
            }
            __syncthreads();
        }
    }
}

// q' = H (D .* q) / sqrt(d) and p = S q' (one wave per query). Queries are
// few, so this runs in double and stores fp32 results rounded once, which
// keeps the rotation and projection error far below the score tolerance.
template <int D, bool QJL, bool F16>
__global__ __launch_bounds__(256) void k_qprep(const void* __restrict__ q, int64_t nq,
                                               const uint32_t* __restrict__ diag,
                                               const uint16_t* __restrict__ S,
                                               float* __restrict__ qr, float* __restrict__ p)
{
    constexpr int R = D / 64;
    __shared__ double sq[kWavesPerBlock][D];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);
    for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < nq;
         base += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t a = base + wid;
        const bool active = a < nq;
        double y[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float x = active ? load_elem<F16>(q, a * D + 64 * r + lane) : 0.f;
            y[r] = (double)flip(x, dm[r]);
        }
        fwht_wave<R>(y, lane);
        const double sc = 1.0 / sqrt((double)D);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            y[r] *= sc;
            if (active) qr[a * D + 64 * r + lane] = (float)y[r];
            sq[wid][64 * r + lane] = y[r];
        }
        if constexpr (QJL) {
            __syncthreads();
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int j = 64 * k + lane;
                const uint16_t* Sj = S + (int64_t)j * D;
                double u = 0.0;
                for (int i = 0; i < D; ++i) u += (double)h2f(Sj[i]) * sq[wid][i];
                if (active) p[a * D + j] = (float)u;
            }
            __syncthreads();
        }
    }
}

// x_hat = n D H (c[idx] + [qjl] g sqrt(pi/2)/m S^T s) / sqrt(d)  (one wave per vector)
template <int D, int B, bool QJL, bool F16OUT>
__global__ __launch_bounds__(256) void k_dequantize(const uint32_t* __restrict__ codes,
                                                    const uint32_t* __restrict__ signs,
                                                    const uint16_t* __restrict__ norm,
                                                    const uint16_t* __restrict__ rnorm, int64_t n,
                                                    const float* __restrict__ cent,
                                                    const uint32_t* __restrict__ diag,
                                                    const uint16_t* __restrict__ S,
                                                    void* __restrict__ out)
{
    constexpr int R = D / 64, W = D / 32, L = 1 << B;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float c[L];
#pragma unroll
    for (int l = 0; l < L; ++l) c[l] = cent[l];
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);
    for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < n;
         base += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t v = base + wid;
        if (v >= n) continue;  // no block-level synchronisation below
        const uint32_t* cv = codes + v * (B * W);
        float a[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = 64 * r + lane;
            int k = 0;
#pragma unroll
            for (int p = 0; p < B; ++p) k |= (int)((cv[p * W + (i >> 5)] >> (i & 31)) & 1u) << p;
            a[r] = pick<L>(c, k);
        }
        if constexpr (QJL) {
            const float g = h2f(rnorm[v]) * (kSqrtHalfPi / (float)D);
            const uint32_t* sv = signs + v * W;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = 64 * r + lane;
                float acc = 0.f;
                for (int j = 0; j < D; ++j) {
                    const float s = ((sv[j >> 5] >> (j & 31)) & 1u) ? 1.f : -1.f;
                    acc += h2f(S[(int64_t)j * D + i]) * s;
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

int grid_for(int64_t units, int per_block)
{
    int64_t b = (units + per_block - 1) / per_block;
    return (int)(b < 65536 ? b : 65536);
}

int device_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "%s: %s", who, hipGetErrorString(e));
    return TQ_OK;
}

// ---------------------------------------------------------------- dispatch

template <int D, int B, bool QJL>
void quantize_d_b(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* o,
                  hipStream_t s)
{
    dim3 grid(grid_for(n, kWavesPerBlock)), block(256);
    if (dtype == TQ_F16)
        hipLaunchKernelGGL((k_quantize<D, B, QJL, true>), grid, block, 0, s, x, n, q->centroids,
                           q->boundaries, q->diag_signs, q->S, o->codes, o->signs, o->norm, o->rnorm);
    else
        hipLaunchKernelGGL((k_quantize<D, B, QJL, false>), grid, block, 0, s, x, n, q->centroids,
                           q->boundaries, q->diag_signs, q->S, o->codes, o->signs, o->norm, o->rnorm);
}

template <int D>
void quantize_d(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* o,
                hipStream_t s)
{
    const bool qjl = q->qjl_m != 0;
    switch (q->mse_bits) {
        case 1: qjl ? quantize_d_b<D, 1, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 1, false>(q, x, dtype, n, o, s); break;
        case 2: qjl ? quantize_d_b<D, 2, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 2, false>(q, x, dtype, n, o, s); break;
        case 3: qjl ? quantize_d_b<D, 3, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 3, false>(q, x, dtype, n, o, s); break;
        default: qjl ? quantize_d_b<D, 4, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 4, false>(q, x, dtype, n, o, s); break;
    }
}

template <int D>
void qprep_d(const tq_quantizer* q, const void* queries, int dtype, int64_t nq, float* qr, float* p,
             hipStream_t s)
{
    dim3 grid(grid_for(nq, kWavesPerBlock)), block(256);
    const bool qjl = q->qjl_m != 0;
    if (dtype == TQ_F16) {
        if (qjl) hipLaunchKernelGGL((k_qprep<D, true, true>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
        else hipLaunchKernelGGL((k_qprep<D, false, true>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
    } else {
        if (qjl) hipLaunchKernelGGL((k_qprep<D, true, false>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
        else hipLaunchKernelGGL((k_qprep<D, false, false>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
    }
}

template <int D, int B, bool QJL>
void dequant_d_b(const tq_quantizer* q, const tq_packed* in, int64_t n, void* out, int dtype, hipStream_t s)
{
    dim3 grid(grid_for(n, kWavesPerBlock)), block(256);
    if (dtype == TQ_F16)
        hipLaunchKernelGGL((k_dequantize<D, B, QJL, true>), grid, block, 0, s, in->codes, in->signs,
                           in->norm, in->rnorm, n, q->centroids, q->diag_signs, q->S, out);
    else
        hipLaunchKernelGGL((k_dequantize<D, B, QJL, false>), grid, block, 0, s, in->codes, in->signs,
                           in->norm, in->rnorm, n, q->centroids, q->diag_signs, q->S, out);
}

template <int D>
void dequant_d(const tq_quantizer* q, const tq_packed* in, int64_t n, int qjl, void* out, int dtype,
               hipStream_t s)
{
    switch (q->mse_bits) {
        case 1: qjl ? dequant_d_b<D, 1, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 1, false>(q, in, n, out, dtype, s); break;
        case 2: qjl ? dequant_d_b<D, 2, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 2, false>(q, in, n, out, dtype, s); break;
        case 3: qjl ? dequant_d_b<D, 3, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 3, false>(q, in, n, out, dtype, s); break;
        default: qjl ? dequant_d_b<D, 4, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 4, false>(q, in, n, out, dtype, s); break;
    }
}

}  // namespace

int launch_quantize(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* out,
                    hipStream_t s)
{
    switch (q->d) {
        case 64: quantize_d<64>(q, x, dtype, n, out, s); break;
        case 128: quantize_d<128>(q, x, dtype, n, out, s); break;
        default: quantize_d<256>(q, x, dtype, n, out, s); break;
    }
    return device_status("tq_quantize");
}

int launch_qprep(const tq_quantizer* q, const void* queries, int dtype, int64_t nq, float* qr, float* p,
                 hipStream_t s)
{
    switch (q->d) {
        case 64: qprep_d<64>(q, queries, dtype, nq, qr, p, s); break;
        case 128: qprep_d<128>(q, queries, dtype, nq, qr, p, s); break;
        default: qprep_d<256>(q, queries, dtype, nq, qr, p, s); break;
    }
    return device_status("query preparation");
}

int launch_dequantize(const tq_quantizer* q, const tq_packed* in, int64_t n, int include_qjl, void* out,
                      int dtype, hipStream_t s)
{
    switch (q->d) {
        case 64: dequant_d<64>(q, in, n, include_qjl, out, dtype, s); break;
        case 128: dequant_d<128>(q, in, n, include_qjl, out, dtype, s); break;
        default: dequant_d<256>(q, in, n, include_qjl, out, dtype, s); break;
    }
    return device_status("tq_dequantize");
}

}  // namespace tq
