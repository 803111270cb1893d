// Single-vector quantizer for the decode step's append of a new token.
//
// Same method as the tensor quantizers ("[Benchmark] TurboQuant 實測：KV Cache
// 3-bit 壓縮，真的零損失？", section "TurboQuant 是什麼：30 秒懶人包": random
// rotation, stored norm, per-coordinate Lloyd-Max codes, and for keys a 1-bit
// sketch of the residual plus its norm), written for one vector per block of
// 256 threads in plain fp32: n = ||x||; y = H (D x) / (sqrt(d) n) through an
// in-LDS Walsh-Hadamard transform (y = 0 when n = 0); code = the number of
// boundaries strictly below y; with QJL r = y - c(code), rnorm = ||r|| and the
// signs of S r. Output in the group-major layout of the packed cache.
#ifndef TQ_APPEND_H
#define TQ_APPEND_H

#include "tq_device.h"

namespace tq {

// Sum over the block (every thread receives it); red: 4 floats of LDS.
__device__ __forceinline__ float block_sum256(float v, float* red)
{
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// LDS floats quantize_one needs for vector length D.
__host__ __device__ constexpr int append_smem_floats(int D) { return 4 * D + 8; }

// Quantize row `row` of x (TQ_F16 or TQ_F32, [rows][D]) with q into vector
// `slot` of o. Called by all 256 threads of a block; ends with a barrier.
template <int D>
__device__ void quantize_one(const tq_quantizer& q, const tq_packed& o, const void* __restrict__ x, int dtype,
                             int64_t row, int64_t slot, float* sm)
{
    float* xs = sm;                                 // [D] rotated coordinates
    float* rr = sm + D;                             // [D] residual
    int* ci = reinterpret_cast<int*>(sm + 2 * D);   // [D] codes
    int* sb = reinterpret_cast<int*>(sm + 3 * D);   // [D] sign bits
    float* red = sm + 4 * D;                        // [8] reductions
    const int tid = threadIdx.x;
    const int B = q.mse_bits, L = 1 << B;
    const bool qjl = q.qjl_m != 0;

    float v = 0.f;
    if (tid < D) {
        v = dtype == TQ_F16 ? h2f(static_cast<const uint16_t*>(x)[row * D + tid])
                            : static_cast<const float*>(x)[row * D + tid];
        if ((q.diag_signs[tid >> 5] >> (tid & 31)) & 1u) v = -v;
        xs[tid] = v;
    }
    const float ss = block_sum256(v * v, red);
    for (int h = 1; h < D; h <<= 1) {
        __syncthreads();
        if (tid < D / 2) {
            const int i = (tid / h) * 2 * h + tid % h;
            const float a = xs[i], b = xs[i + h];
            xs[i] = a + b;
            xs[i + h] = a - b;
        }
    }
    __syncthreads();
    const float nrm = sqrtf(ss);
    const float inv = nrm > 0.f ? 1.0f / (sqrtf((float)D) * nrm) : 0.f;
    float r2 = 0.f;
    if (tid < D) {
        const float y = xs[tid] * inv;
        int idx = 0;
        for (int j = 0; j < L - 1; ++j) idx += q.boundaries[j] < y ? 1 : 0;
        ci[tid] = idx;
        if (qjl) {
            const float r = y - q.centroids[idx];
            rr[tid] = r;
            r2 = r * r;
        }
    }
    const float g2 = block_sum256(r2, red + 4);  // also publishes ci and rr
    // codes: stream bit k = 8 B c + B t + p holds bit p of the code of coordinate c + (D/8) t
    const int CW = B * D / 32;
    if (tid < CW) {
        uint32_t w = 0;
        for (int k = 0; k < 32; ++k) {
            const int kk = 32 * tid + k;
            const int c = kk / (8 * B), t = (kk % (8 * B)) / B, p = kk % B;
            w |= (uint32_t)((ci[c + (D / 8) * t] >> p) & 1) << k;
        }
        o.codes[slot * CW + tid] = w;
    }
    if (qjl) {
        if (tid < D) {
            const uint16_t* srow = q.S + (int64_t)tid * D;
            float u = 0.f;
            for (int i = 0; i < D; ++i) u = fmaf(h2f(srow[i]), rr[i], u);
            sb[tid] = u >= 0.f ? 1 : 0;
        }
        __syncthreads();
        // signs: stream bit k = 8 j0 + t holds the sign of row j0 + (D/8) t
        if (tid < D / 32) {
            uint32_t w = 0;
            for (int k = 0; k < 32; ++k) {
                const int kk = 32 * tid + k;
                w |= (uint32_t)sb[kk / 8 + (D / 8) * (kk % 8)] << k;
            }
            o.signs[slot * (D / 32) + tid] = w;
        }
    }
    if (tid == 0) {
        o.norm[slot] = f2h(nrm);
        if (qjl) o.rnorm[slot] = f2h(sqrtf(g2));
    }
    __syncthreads();
}

}  // namespace tq

#endif
