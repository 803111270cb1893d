// Score estimation and fused decode attention over packed keys and values.
//
// Estimator ("[Benchmark] TurboQuant 實測：KV Cache 3-bit 壓縮，真的零損失？",
// section "TurboQuant 是什麼：30 秒懶人包", QJL step): with q' = H D q / sqrt(d)
// and p = S q' prepared once per query,
//   score = n * ( sum_i q'_i c[idx_i] + rnorm * sqrt(pi/2)/m * sum_j p_j (2 s_j - 1) ).
//
// Decode attention is split over token chunks: each block scores its chunk
// for the G heads of one stream, takes a chunk-local softmax, accumulates
// sum_t w_t n_t c_v[idx] in the rotated value domain and writes a partial
// (max, sum, accumulator). A combine kernel merges the partials of a stream
// and applies the inverse value rotation D_v H / sqrt(d) once per head.
#include <float.h>

#include "tq_append.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kQT = 16;       // queries per LDS tile in the score kernel
constexpr int kTC = 256;      // tokens per decode chunk (one per thread)
constexpr int kMaxG = 16;

template <int D, int B, bool QJL>
__global__ __launch_bounds__(256) void k_scores(const uint32_t* __restrict__ codes,
                                                const uint32_t* __restrict__ signs,
                                                const uint16_t* __restrict__ norm,
                                                const uint16_t* __restrict__ rnorm, int64_t n_keys,
                                                const float* __restrict__ qr,
                                                const float* __restrict__ p, int64_t n_q,
                                                const float* __restrict__ cent,
                                                float* __restrict__ scores)
{
    constexpr int W = D / 32, L = 1 << B;
    __shared__ float sq[kQT][D];
    __shared__ float sp[QJL ? kQT : 1][D];
    __shared__ float sc[L];
    if (threadIdx.x < L) sc[threadIdx.x] = cent[threadIdx.x];
    const int64_t key = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool act = key < n_keys;
    uint32_t cw[B * W], sw[W];
    double nk = 0.0, gk = 0.0;
#pragma unroll
    for (int w = 0; w < B * W; ++w) cw[w] = act ? codes[key * (B * W) + w] : 0u;
#pragma unroll
    for (int w = 0; w < W; ++w) sw[w] = (QJL && act) ? signs[key * W + w] : 0u;
    if (act) {
        nk = (double)h2f(norm[key]);
        if (QJL) gk = (double)h2f(rnorm[key]) * (1.2533141373155003 / D);
    }
    // query tiles are spread over grid.y so that small key sets still fill the device
    for (int64_t q0 = (int64_t)blockIdx.y * kQT; q0 < n_q; q0 += (int64_t)gridDim.y * kQT) {
        __syncthreads();
        for (int e = threadIdx.x; e < kQT * D; e += 256) {
            const int qi = e / D, i = e % D;
            const bool ok = q0 + qi < n_q;
            sq[qi][i] = ok ? qr[(q0 + qi) * D + i] : 0.f;
            if (QJL) sp[qi][i] = ok ? p[(q0 + qi) * D + i] : 0.f;
        }
        __syncthreads();
        // double accumulators: scores reach |n||q| ~ 10^2-10^3, where fp32
        // summation of 2d terms alone would use up the 1e-4 tolerance
        double am[kQT], aj[kQT];
#pragma unroll
        for (int qi = 0; qi < kQT; ++qi) am[qi] = aj[qi] = 0.0;
#pragma unroll
        for (int i = 0; i < D; ++i) {
                int idx = 0;
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int P = code_bit<D, B>(i, b);
                    idx |= (int)((cw[P >> 5] >> (P & 31)) & 1u) << b;
                }
                const double c = (double)sc[idx];
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
                if (qi < nq)
                    scores[(q0 + qi) * n_keys + key] = (float)(nk * (am[qi] + gk * aj[qi]));
        }
    }
}

template <int D, int BK, bool QJL, int BV>
__global__ __launch_bounds__(256) void k_decode(const uint32_t* __restrict__ kcodes,
                                                const uint32_t* __restrict__ ksigns,
                                                const uint16_t* __restrict__ knorm,
                                                const uint16_t* __restrict__ krnorm,
                                                const uint32_t* __restrict__ vcodes,
                                                const uint16_t* __restrict__ vnorm, int64_t T, int64_t stride,
                                                int G, const float* __restrict__ qr,
                                                const float* __restrict__ p,
                                                const float* __restrict__ kcent,
                                                const float* __restrict__ vcent, float scale,
                                                float* __restrict__ parts, int n_chunks)
{
    constexpr int W = D / 32, LK = 1 << BK, LV = 1 << BV;
    __shared__ float sq[kMaxG][D];
    __shared__ float sp[QJL ? kMaxG : 1][D];
    __shared__ float z[kMaxG][kTC];
    __shared__ uint32_t vw[kTC][BV * W];
    __shared__ float vn[kTC];
    __shared__ float kc[LK], vc[LV];
    __shared__ float smax[kMaxG];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t s = blockIdx.y;
    const int chunk = blockIdx.x;
    const int64_t t0 = (int64_t)chunk * kTC;
    if (tid < LK) kc[tid] = kcent[tid];
    if (tid < LV) vc[tid] = vcent[tid];
    for (int e = tid; e < G * D; e += 256) {
        const int h = e / D, i = e % D;
        sq[h][i] = qr[(s * G + h) * D + i];
        if (QJL) sp[h][i] = p[(s * G + h) * D + i];
    }
    // stage this chunk's value codes and norms
    for (int e = tid; e < kTC * BV * W; e += 256) {
        const int tt = e / (BV * W), j = e % (BV * W);
        const int64_t t = t0 + tt;
        vw[tt][j] = t < T ? vcodes[(s * stride + t) * (BV * W) + j] : 0u;
    }
    {
        const int64_t t = t0 + tid;
        vn[tid] = t < T ? h2f(vnorm[s * stride + t]) : 0.f;
    }
    __syncthreads();

    // phase A: scores of this thread's token for all heads
    {
        const int64_t t = t0 + tid;
        float am[kMaxG], aj[kMaxG];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) am[h] = aj[h] = 0.f;
        if (t < T) {
            const int64_t v = s * stride + t;
            uint32_t cw[BK * W], sw[W];
#pragma unroll
            for (int w = 0; w < BK * W; ++w) cw[w] = kcodes[v * (BK * W) + w];
#pragma unroll
            for (int w = 0; w < W; ++w) sw[w] = QJL ? ksigns[v * W + w] : 0u;
#pragma unroll 8
            for (int i = 0; i < D; ++i) {
                int idx = 0;
#pragma unroll
                for (int b = 0; b < BK; ++b) {
                    const int P = code_bit<D, BK>(i, b);
                    idx |= (int)((cw[P >> 5] >> (P & 31)) & 1u) << b;
                }
                const float c = kc[idx];
                const int SP = sign_bit<D>(i);
                const float sg = ((sw[SP >> 5] >> (SP & 31)) & 1u) ? 1.f : -1.f;
#pragma unroll
                for (int h = 0; h < kMaxG; ++h)
                    if (h < G) {
                        am[h] += sq[h][i] * c;
                        if (QJL) aj[h] += sp[h][i] * sg;
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
    }
    __syncthreads();

    // phase B: chunk-local softmax per head (one wave per head, round robin)
    for (int h = wid; h < G; h += 4) {
        float m = -INFINITY;
        for (int tt = lane; tt < kTC; tt += 64) m = fmaxf(m, z[h][tt]);
        m = wave_max(m);
        float l = 0.f;
        for (int tt = lane; tt < kTC; tt += 64) {
            const float w = (z[h][tt] == -INFINITY) ? 0.f : exp2f(z[h][tt] - m);
            z[h][tt] = w;
            l += w;
        }
        l = wave_sum(l);
        if (lane == 0) {
            smax[h] = m;
            float* part = parts + (((int64_t)s * n_chunks + chunk) * G + h) * part_stride(D);
            part[0] = m;
            part[1] = l;
        }
    }
    __syncthreads();

    // phase C: rotated-domain value accumulation, one (head, coordinate) per step
    for (int e = tid; e < G * D; e += 256) {
        const int h = e / D, i = e % D;
        float acc = 0.f;
        for (int tt = 0; tt < kTC; ++tt) {
            int idx = 0;
#pragma unroll
            for (int b = 0; b < BV; ++b) {
                const int P = code_bit<D, BV>(i, b);
                idx |= (int)((vw[tt][P >> 5] >> (P & 31)) & 1u) << b;
            }
            acc += z[h][tt] * vn[tt] * vc[idx];
        }
        parts[(((int64_t)s * n_chunks + chunk) * G + h) * part_stride(D) + kPartAcc + i] = acc;
    }
}

// Merge the chunk partials of one (stream, head) and rotate back to the value
// domain. Partials hold (max, sum, accumulator) with max in log2 units.
// Thread (lane c, slot i) folds chunks c, c + CL, ... of float4 slot i into a
// running (max, sum, accumulator) in a single pass over the partials (the
// loop is unrolled so that many chunks' loads are in flight at once); wave 0
// then merges the CL running results.
template <int D>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ parts, int n_chunks, int G,
                                                 const uint32_t* __restrict__ vdiag,
                                                 float* __restrict__ out)
{
    constexpr int R = D / 64, NV = D / 4, CL = 256 / NV, PS = part_stride(D);
    __shared__ float4 om[CL][NV];
    __shared__ float ol[CL], omx[CL];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t sh = blockIdx.x;  // s * G + h
    const int64_t s = sh / G, h = sh % G;
    const int64_t stride = (int64_t)G * PS;
    const float* p0 = parts + ((s * n_chunks) * G + h) * PS;

    // one pass: thread (cl, i) folds chunks cl, cl + CL, ... into a running
    // (max, sum, accumulator) for coordinates 4 i .. 4 i + 3
    const int cl = tid / NV, i = tid % NV;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f, m = -INFINITY;
#pragma unroll 8
    for (int c = cl; c < n_chunks; c += CL) {
        const float* pc = p0 + c * stride;
        const float2 ml = *reinterpret_cast<const float2*>(pc);
        const float4 a = reinterpret_cast<const float4*>(pc + kPartAcc)[i];
        // branch-free, so that the unrolled iterations' loads issue together;
        // a chunk with no tokens (max -inf) contributes nothing
        const float nm = fmaxf(m, ml.x);
        const float fo = m == -INFINITY ? 0.f : exp2f(m - nm);
        const float fn = ml.x == -INFINITY ? 0.f : exp2f(ml.x - nm);
        acc.x = acc.x * fo + fn * a.x;
        acc.y = acc.y * fo + fn * a.y;
        acc.z = acc.z * fo + fn * a.z;
        acc.w = acc.w * fo + fn * a.w;
        l = l * fo + fn * ml.y;
        m = nm;
    }
    om[cl][i] = acc;
    if (i == 0) {
        ol[cl] = l;
        omx[cl] = m;
    }
    __syncthreads();
    if (wid != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < CL; ++q) M = fmaxf(M, omx[q]);
    float fq[CL];
#pragma unroll
    for (int q = 0; q < CL; ++q) fq[q] = omx[q] == -INFINITY ? 0.f : exp2f(omx[q] - M);
    const float* omf = reinterpret_cast<const float*>(&om[0][0]);
    float v[R];
    float L = 0.f;
#pragma unroll
    for (int q = 0; q < CL; ++q) L += fq[q] * ol[q];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        v[r] = 0.f;
#pragma unroll
        for (int q = 0; q < CL; ++q) v[r] += fq[q] * omf[q * D + 64 * r + lane];
    }
    fwht_wave<R>(v, lane);
    uint32_t dm[R];
    load_diag<R>(vdiag, lane, dm);
    const float sc = 1.0f / (sqrtf((float)D) * L);
#pragma unroll
    for (int r = 0; r < R; ++r) out[sh * D + 64 * r + lane] = flip(v[r], dm[r]) * sc;
}

// The decode step's append for the shapes without the MFMA path: block
// (s, 0) quantizes stream s's new key, block (s, 1) its new value.
template <int D>
__global__ __launch_bounds__(256) void k_append(tq_quantizer qk, tq_quantizer qv, tq_packed k, tq_packed v,
                                                const void* __restrict__ k_new, const void* __restrict__ v_new,
                                                int dtype, int64_t stride, int64_t pos)
{
    __shared__ float sm[append_smem_floats(D)];
    const int64_t s = blockIdx.x;
    const bool val = blockIdx.y == 1;
    quantize_one<D>(val ? qv : qk, val ? v : k, val ? v_new : k_new, dtype, s, s * stride + pos, sm);
}

int device_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "%s: %s", who, hipGetErrorString(e));
    return TQ_OK;
}

template <int D, int B, bool QJL>
void scores_d_b(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const float* qr,
                const float* p, int64_t n_q, float* scores, hipStream_t s)
{
    const int64_t qt = (n_q + kQT - 1) / kQT;
    dim3 grid((unsigned)((n_keys + 255) / 256), (unsigned)(qt < 65535 ? qt : 65535)), block(256);
    hipLaunchKernelGGL((k_scores<D, B, QJL>), grid, block, 0, s, k->codes, k->signs, k->norm,
                       k->rnorm, n_keys, qr, p, n_q, q->centroids, scores);
}

template <int D>
void scores_d(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const float* qr,
              const float* p, int64_t n_q, float* scores, hipStream_t s)
{
    const bool qjl = q->qjl_m != 0;
    switch (q->mse_bits) {
        case 1: qjl ? scores_d_b<D, 1, true>(q, k, n_keys, qr, p, n_q, scores, s) : scores_d_b<D, 1, false>(q, k, n_keys, qr, p, n_q, scores, s); break;
        case 2: qjl ? scores_d_b<D, 2, true>(q, k, n_keys, qr, p, n_q, scores, s) : scores_d_b<D, 2, false>(q, k, n_keys, qr, p, n_q, scores, s); break;
        case 3: qjl ? scores_d_b<D, 3, true>(q, k, n_keys, qr, p, n_q, scores, s) : scores_d_b<D, 3, false>(q, k, n_keys, qr, p, n_q, scores, s); break;
        default: qjl ? scores_d_b<D, 4, true>(q, k, n_keys, qr, p, n_q, scores, s) : scores_d_b<D, 4, false>(q, k, n_keys, qr, p, n_q, scores, s); break;
    }
}

template <int D, int BK, bool QJL, int BV>
void decode_kernel(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k, const tq_packed* v,
                   int64_t n_streams, int64_t T, int64_t stride, int G, const float* qr, const float* p,
                   float scale, float* parts, int n_chunks, hipStream_t s)
{
    dim3 grid((unsigned)n_chunks, (unsigned)n_streams), block(256);
    hipLaunchKernelGGL((k_decode<D, BK, QJL, BV>), grid, block, 0, s, k->codes, k->signs, k->norm,
                       k->rnorm, v->codes, v->norm, T, stride, G, qr, p, qk->centroids, qv->centroids,
                       scale, parts, n_chunks);
}

template <int D, int BK, bool QJL>
void decode_bv(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k, const tq_packed* v,
               int64_t n_streams, int64_t T, int64_t stride, int G, const float* qr, const float* p,
               float scale, float* parts, int n_chunks, hipStream_t s)
{
    switch (qv->mse_bits) {
        case 1: decode_kernel<D, BK, QJL, 1>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
        case 2: decode_kernel<D, BK, QJL, 2>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
        case 3: decode_kernel<D, BK, QJL, 3>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
        default: decode_kernel<D, BK, QJL, 4>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
    }
}

template <int D>
void decode_d(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k, const tq_packed* v,
              int64_t n_streams, int64_t T, int64_t stride, int G, const float* qr, const float* p,
              float scale, float* out, float* parts, int n_chunks, hipStream_t s)
{
    const bool qjl = qk->qjl_m != 0;
    switch (qk->mse_bits) {
        case 1: qjl ? decode_bv<D, 1, true>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s) : decode_bv<D, 1, false>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
        case 2: qjl ? decode_bv<D, 2, true>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s) : decode_bv<D, 2, false>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
        case 3: qjl ? decode_bv<D, 3, true>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s) : decode_bv<D, 3, false>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
        default: qjl ? decode_bv<D, 4, true>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s) : decode_bv<D, 4, false>(qk, qv, k, v, n_streams, T, stride, G, qr, p, scale, parts, n_chunks, s); break;
    }
    (void)out;
}

}  // namespace

int launch_scores(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const float* qr,
                  const float* p, int64_t n_q, float* scores, hipStream_t s)
{
    switch (q->d) {
        case 64: scores_d<64>(q, k, n_keys, qr, p, n_q, scores, s); break;
        case 128: scores_d<128>(q, k, n_keys, qr, p, n_q, scores, s); break;
        default: scores_d<256>(q, k, n_keys, qr, p, n_q, scores, s); break;
    }
    return device_status("tq_scores");
}

int launch_decode(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k,
                  const tq_packed* v, int64_t n_streams, int64_t T, int64_t stride, int G, const void* q,
                  int q_dtype, const DecodePlan& plan, void* ws, float scale, float* out,
                  const AppendArgs* app, hipStream_t s)
{
    float* qr = (float*)((char*)ws + plan.off_qr);
    float* p = (float*)((char*)ws + plan.off_p);
    float* parts = (float*)((char*)ws + plan.off_parts);
    const float zscale = scale * 1.4426950408889634f;  // scores in log2 units
    if (plan.mfma) {
        int rc = launch_decode_mfma(qk, qv, k, v, n_streams, T, stride, G, q, q_dtype, zscale,
                                    (char*)ws + plan.off_frag, parts, plan.n_chunks, (int)plan.tc, app, s);
        if (rc != TQ_OK) return rc;
    } else {
        if (app) {
            const dim3 ag((unsigned)n_streams, 2u);
            switch (qk->d) {
                case 64: hipLaunchKernelGGL((k_append<64>), ag, dim3(256), 0, s, *qk, *qv, *k, *v, app->k_new, app->v_new, app->dtype, stride, app->pos); break;
                case 128: hipLaunchKernelGGL((k_append<128>), ag, dim3(256), 0, s, *qk, *qv, *k, *v, app->k_new, app->v_new, app->dtype, stride, app->pos); break;
                default: hipLaunchKernelGGL((k_append<256>), ag, dim3(256), 0, s, *qk, *qv, *k, *v, app->k_new, app->v_new, app->dtype, stride, app->pos); break;
            }
        }
        int rc = launch_qprep(qk, q, q_dtype, n_streams * G, qr, p, s);
        if (rc != TQ_OK) return rc;
        if (qk->mse_bits > 4 || qv->mse_bits > 4) {
            rc = launch_decode_wide(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, parts, plan.n_chunks, s);
            if (rc != TQ_OK) return rc;
        } else switch (qk->d) {
            case 64: decode_d<64>(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, out, parts, plan.n_chunks, s); break;
            case 128: decode_d<128>(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, out, parts, plan.n_chunks, s); break;
            default: decode_d<256>(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, out, parts, plan.n_chunks, s); break;
        }
    }
    const dim3 cg((unsigned)(n_streams * G));
    switch (qk->d) {
        case 64: hipLaunchKernelGGL((k_combine<64>), cg, dim3(256), 0, s, parts, plan.n_chunks, G, qv->diag_signs, out); break;
        case 128: hipLaunchKernelGGL((k_combine<128>), cg, dim3(256), 0, s, parts, plan.n_chunks, G, qv->diag_signs, out); break;
        default: hipLaunchKernelGGL((k_combine<256>), cg, dim3(256), 0, s, parts, plan.n_chunks, G, qv->diag_signs, out); break;
    }
    return device_status(app ? "tq_decode_step" : "tq_decode_attn");
}

}  // namespace tq
