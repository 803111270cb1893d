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
// (max, sum, accumulator); the MFMA kernel (tq_decode.hip) or the scalar one
// (tq_wide.hip) does that. The combine kernel here merges the partials of a
// stream and applies the inverse value rotation D_v H / sqrt(d) once per head.
#include <float.h>

#include <mutex>

#include "tq_append.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

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
    fwht_wave_dpp<R>(v, lane);
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

}  // namespace

// The fixed scratch of tq_decode_attn_noalloc, one copy per device (zero at
// load, kept until the process ends). Host code never uses the array's name
// as an address: noalloc_scratch looks up the device address once per device
// with hipGetSymbolAddress and every launch takes that address.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

int noalloc_scratch(void** ptr)
{
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(TQ_ERR_DEVICE, "tq_decode_attn_noalloc: no current device");
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(TQ_ERR_DEVICE, "tq_decode_attn_noalloc: scratch address: %s", hipGetErrorString(e));
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return TQ_OK;
}

namespace {

int device_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "%s: %s", who, hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace

int launch_decode(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k,
                  const tq_packed* v, int64_t n_streams, int64_t T, int64_t stride, int G, const void* q,
                  int q_dtype, const DecodePlan& plan, void* ws, float scale, float* out,
                  const AppendArgs* app, hipStream_t s)
{
    float* qr = (float*)((char*)ws + plan.off_qr);
    float* p = (float*)((char*)ws + plan.off_p);
    float* parts = (float*)((char*)ws + plan.off_parts);
    const float zscale = scale * 1.4426950408889634f;  // scores in log2 units
    // the decode step's append: inside the MFMA decode kernel, else first, as its
    // own launch (one block per stream and tensor)
    if (app && !plan.fused_append) {
        const dim3 ag((unsigned)n_streams, 2u);
        switch (qk->d) {
            case 64: hipLaunchKernelGGL((k_append<64>), ag, dim3(256), 0, s, *qk, *qv, *k, *v, app->k_new, app->v_new, app->dtype, stride, app->pos); break;
            case 128: hipLaunchKernelGGL((k_append<128>), ag, dim3(256), 0, s, *qk, *qv, *k, *v, app->k_new, app->v_new, app->dtype, stride, app->pos); break;
            default: hipLaunchKernelGGL((k_append<256>), ag, dim3(256), 0, s, *qk, *qv, *k, *v, app->k_new, app->v_new, app->dtype, stride, app->pos); break;
        }
    }
    if (plan.mfma) {
        // the MFMA kernel prepares its stream's queries itself; with the fused
        // append it scans the app->pos cached tokens and adds the new one
        AppendIn ap{};
        int64_t Ts = T;
        if (plan.fused_append) {
            ap = AppendIn{app->k_new, app->v_new, app->dtype == TQ_F16 ? 1 : 0, app->pos, qv->diag_signs,
                          qk->boundaries, qv->boundaries, k->codes, k->signs, k->norm, k->rnorm, v->codes, v->norm};
            Ts = app->pos;
        }
        int rc = launch_decode_mfma(qk, qv, k, v, n_streams, Ts, stride, G, q, q_dtype, zscale, parts, plan.n_chunks,
                                    plan.pchunks, (int)plan.tc, ap, s);
        if (rc != TQ_OK) return rc;
    } else {
        // every other shape and width pair: prepared queries and the scalar
        // kernel with run-time widths
        int rc = launch_qprep(qk, q, q_dtype, n_streams * G, qr, p, s);
        if (rc != TQ_OK) return rc;
        rc = launch_decode_wide(qk, qv, k, v, n_streams, T, stride, G, qr, p, zscale, parts, plan.n_chunks, s);
        if (rc != TQ_OK) return rc;
    }
    const dim3 cg((unsigned)(n_streams * G));
    switch (qk->d) {
        case 64: hipLaunchKernelGGL((k_combine<64>), cg, dim3(256), 0, s, parts, plan.pchunks, G, qv->diag_signs, out); break;
        case 128: hipLaunchKernelGGL((k_combine<128>), cg, dim3(256), 0, s, parts, plan.pchunks, G, qv->diag_signs, out); break;
        default: hipLaunchKernelGGL((k_combine<256>), cg, dim3(256), 0, s, parts, plan.pchunks, G, qv->diag_signs, out); break;
    }
    return device_status(app ? "tq_decode_step" : "tq_decode_attn");
}

}  // namespace tq
