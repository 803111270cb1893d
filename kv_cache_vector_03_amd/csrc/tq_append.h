// Single-vector quantizer for the decode step's append of a new token.
//
// Same method as the tensor quantizers ("[Benchmark] TurboQuant 實測：KV Cache
// 3-bit 壓縮，真的零損失？", section "TurboQuant 是什麼：30 秒懶人包": random
// rotation, stored norm, per-coordinate Lloyd-Max codes, and for keys a 1-bit
// sketch of the residual plus its norm), written for one vector per block of
// 256 threads in plain fp32: n = ||x||; y = H (D x) / (sqrt(d) n) through a
// one-wave Walsh-Hadamard transform (y = 0 when n = 0); code = the number of
// boundaries strictly below y; with QJL r = y - c(code), rnorm = ||r|| and the
// signs of S r. Output in the group-major layout of the packed cache.
#ifndef TQ_APPEND_H
#define TQ_APPEND_H

#include "tq_device.h"

namespace tq {

// LDS floats quantize_one needs for vector length D: the codebook (256 + 256),
// the residual (D), codes and sign bits (D bytes each).
__host__ __device__ constexpr int append_smem_floats(int D) { return 512 + D + D / 2; }

// Quantize row `row` of x (TQ_F16 or TQ_F32, [rows][D]) with q into vector
// `slot` of o. Called by all 256 threads of a block; ends with a barrier.
// The codebook, the input and (keys) each thread's row of S are fetched at
// once, so the block waits for one round of loads. Wave 0 then rotates and
// codes the vector in registers (lane l, slot r holds coordinate 64 r + l;
// cross-lane butterflies and sums by wave exchanges; boundaries and centroids
// from LDS); then all threads pack the code words and, for keys, take one row
// of S each for the sketch.
template <int D>
__device__ void quantize_one(const tq_quantizer& q, const tq_packed& o, const void* __restrict__ x, int dtype,
                             int64_t row, int64_t slot, float* sm)
{
    constexpr int R = D / 64;
    float* bt = sm;                                                  // [256] boundaries (L - 1 used)
    float* ct = sm + 256;                                            // [256] centroids (L used)
    float* rr = sm + 512;                                            // [D] residual
    unsigned char* ci = reinterpret_cast<unsigned char*>(sm + 512 + D);  // [D] codes
    unsigned char* sb = ci + D;                                      // [D] sign bits
    const int tid = threadIdx.x, lane = tid & 63;
    const int B = q.mse_bits, L = 1 << B;
    const bool qjl = q.qjl_m != 0;
    if (tid < L - 1) bt[tid] = q.boundaries[tid];
    if (tid < L) ct[tid] = q.centroids[tid];

    // this thread's row of S (keys), fetched first so that it arrives during
    // the rotation (S is 16-byte aligned)
    uint4 srow[D / 8];
    if (qjl && tid < D) {
        const uint4* sp = reinterpret_cast<const uint4*>(q.S + (int64_t)tid * D);
#pragma unroll
        for (int c = 0; c < D / 8; ++c) srow[c] = sp[c];
    }

    float y[R];
    if (tid < 64) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int c = 64 * r + lane;
            float v = dtype == TQ_F16 ? h2f(static_cast<const uint16_t*>(x)[row * D + c])
                                      : static_cast<const float*>(x)[row * D + c];
            if ((q.diag_signs[c >> 5] >> (c & 31)) & 1u) v = -v;
            y[r] = v;
        }
    }
    __syncthreads();  // the codebook is in LDS
    if (tid < 64) {
        float ss = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) ss += y[r] * y[r];
        const float nrm = sqrtf(wave_sum(ss));
        fwht_wave<R>(y, lane);
        const float inv = nrm > 0.f ? 1.0f / (sqrtf((float)D) * nrm) : 0.f;
        float r2 = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float yy = y[r] * inv;
            int idx = 0;
            for (int j = 0; j < L - 1; ++j) idx += bt[j] < yy ? 1 : 0;
            ci[64 * r + lane] = (unsigned char)idx;
            if (qjl) {
                const float e = yy - ct[idx];
                rr[64 * r + lane] = e;
                r2 += e * e;
            }
        }
        const float g2 = wave_sum(r2);
        if (lane == 0) {
            o.norm[slot] = f2h(nrm);
            if (qjl) o.rnorm[slot] = f2h(sqrtf(g2));
        }
    }
    __syncthreads();
    // codes: group c (coordinates c + (D/8) t, code t at bit B t of an 8 B-bit
    // field) is bytes B c .. B c + B - 1 of the vector's stream
    if (tid < D / 8) {
        uint64_t f = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) f |= (uint64_t)ci[tid + (D / 8) * t] << (B * t);
        unsigned char* dst = reinterpret_cast<unsigned char*>(o.codes + slot * (B * D / 32)) + B * tid;
        for (int b = 0; b < B; ++b) dst[b] = (unsigned char)(f >> (8 * b));
    }
    if (qjl) {
        if (tid < D) {
            float u = 0.f;  // sum over i in order, as a plain dot product
#pragma unroll
            for (int c = 0; c < D / 8; ++c) {
                const uint32_t w4[4] = {srow[c].x, srow[c].y, srow[c].z, srow[c].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    u = fmaf(h2f((uint16_t)(w4[e >> 1] >> (16 * (e & 1)))), rr[8 * c + e], u);
            }
            sb[tid] = u >= 0.f ? 1 : 0;
        }
        __syncthreads();
        // signs: bit t of byte j0 is the sign of row j0 + (D/8) t
        if (tid < D / 8) {
            uint32_t w = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) w |= (uint32_t)sb[tid + (D / 8) * t] << t;
            reinterpret_cast<unsigned char*>(o.signs + slot * (D / 32))[tid] = (unsigned char)w;
        }
    }
    __syncthreads();
}

}  // namespace tq

#endif
