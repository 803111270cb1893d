// The extern "C" entry points: validate on the host, then enqueue kernels.
#include <cmath>

#include "tq.h"
#include "tq_internal.h"

using namespace tq;

namespace {

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

// Argument checks shared by the decode-attention entry points; on success
// fills the work split (plan) for a non-empty call.
int check_decode_args(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k, const tq_packed* v,
                      int64_t n_streams, int64_t T, int G, const void* q, int q_dtype, float scale,
                      const float* out, const char* who, DecodePlan* plan)
{
    int rc;
    if ((rc = check_quantizer(qk, who, "key")) != TQ_OK) return rc;
    if ((rc = check_quantizer(qv, who, "value")) != TQ_OK) return rc;
    if (qv->d != qk->d) return fail(TQ_ERR_UNSUPPORTED, "%s: key d=%d != value d=%d", who, qk->d, qv->d);
    if (qv->qjl_m != 0) return fail(TQ_ERR_UNSUPPORTED, "%s: value quantizer must be codes-only (qjl_m=0)", who);
    if (n_streams < 0) return fail(TQ_ERR_INVALID, "%s: n_streams < 0", who);
    if (G < 1 || G > 16) return fail(TQ_ERR_UNSUPPORTED, "%s: G=%d not in 1..16", who, G);
    if (n_streams == 0) return TQ_OK;
    if (T < 1) return fail(TQ_ERR_INVALID, "%s: T=%lld < 1", who, (long long)T);
    if (!std::isfinite(scale) || scale < 0) return fail(TQ_ERR_INVALID, "%s: bad scale", who);
    if ((rc = check_packed(qk, k, who, "k")) != TQ_OK) return rc;
    if ((rc = check_packed(qv, v, who, "v")) != TQ_OK) return rc;
    if ((rc = check_dense(q, q_dtype, who, "q")) != TQ_OK) return rc;
    if ((rc = check_dense(out, TQ_F32, who, "out")) != TQ_OK) return rc;
    *plan = decode_plan(qk, n_streams, T, G, !mfma_decode_widths(qk->mse_bits, qv->mse_bits));
    return TQ_OK;
}

}  // namespace

extern "C" {

int tq_quantize(const tq_quantizer* q, const void* x, int x_dtype, int64_t n,
                const tq_packed* out, void* stream)
{
    clear_error();
    int rc;
    if ((rc = check_quantizer(q, "tq_quantize", "")) != TQ_OK) return rc;
    if (n < 0) return fail(TQ_ERR_INVALID, "tq_quantize: n=%lld < 0", (long long)n);
    if (n == 0) return TQ_OK;
    if ((rc = check_dense(x, x_dtype, "tq_quantize", "x")) != TQ_OK) return rc;
    if ((rc = check_packed(q, out, "tq_quantize", "out")) != TQ_OK) return rc;
    return launch_quantize(q, x, x_dtype, n, out, (hipStream_t)stream);
}

int tq_scores(const tq_quantizer* q, const tq_packed* keys, int64_t n_keys,
              const void* queries, int q_dtype, int64_t n_q, float* scores,
              void* ws, size_t ws_bytes, void* stream)
{
    clear_error();
    int rc;
    if ((rc = check_quantizer(q, "tq_scores", "")) != TQ_OK) return rc;
    if (n_keys < 0 || n_q < 0) return fail(TQ_ERR_INVALID, "tq_scores: negative size");
    if (n_keys == 0 || n_q == 0) return TQ_OK;
    if ((rc = check_packed(q, keys, "tq_scores", "keys")) != TQ_OK) return rc;
    if ((rc = check_dense(queries, q_dtype, "tq_scores", "queries")) != TQ_OK) return rc;
    if ((rc = check_dense(scores, TQ_F32, "tq_scores", "scores")) != TQ_OK) return rc;
    size_t need = scores_ws(q, n_q);
    if (!ws || ws_bytes < need)
        return fail(TQ_ERR_WORKSPACE, "tq_scores: workspace %zu bytes < %zu", ws_bytes, need);
    if ((uintptr_t)ws % 256) return fail(TQ_ERR_INVALID, "tq_scores: workspace must be 256-byte aligned");
    if (q->d == 128) return launch_scores_mfma(q, keys, n_keys, queries, q_dtype, n_q, scores, ws, (hipStream_t)stream);
    float* qr = (float*)ws;
    float* p = (float*)((char*)ws + up256((size_t)n_q * q->d * 4));
    if ((rc = launch_qprep(q, queries, q_dtype, n_q, qr, p, (hipStream_t)stream)) != TQ_OK) return rc;
    return launch_scores_wide(q, keys, n_keys, qr, p, n_q, scores, (hipStream_t)stream);
}

int tq_dequantize(const tq_quantizer* q, const tq_packed* in, int64_t n, int include_qjl,
                  void* out, int out_dtype, void* stream)
{
    clear_error();
    int rc;
    if ((rc = check_quantizer(q, "tq_dequantize", "")) != TQ_OK) return rc;
    if (n < 0) return fail(TQ_ERR_INVALID, "tq_dequantize: n=%lld < 0", (long long)n);
    if (n == 0) return TQ_OK;
    if (q->qjl_m == 0) include_qjl = 0;
    if (include_qjl) {
        if ((rc = check_packed(q, in, "tq_dequantize", "in")) != TQ_OK) return rc;
    } else {
        tq_quantizer q0 = *q;
        q0.qjl_m = 0;
        if ((rc = check_packed(&q0, in, "tq_dequantize", "in")) != TQ_OK) return rc;
    }
    if ((rc = check_dense(out, out_dtype, "tq_dequantize", "out")) != TQ_OK) return rc;
    return launch_dequantize(q, in, n, include_qjl ? 1 : 0, out, out_dtype, (hipStream_t)stream);
}

int tq_decode_attn(const tq_quantizer* qk, const tq_quantizer* qv,
                   const tq_packed* k, const tq_packed* v,
                   int64_t n_streams, int64_t T, int G,
                   const void* q, int q_dtype, float scale, float* out,
                   void* ws, size_t ws_bytes, void* stream)
{
    clear_error();
    DecodePlan plan;
    int rc = check_decode_args(qk, qv, k, v, n_streams, T, G, q, q_dtype, scale, out, "tq_decode_attn", &plan);
    if (rc != TQ_OK || n_streams == 0) return rc;
    if (!ws || ws_bytes < plan.total)
        return fail(TQ_ERR_WORKSPACE, "tq_decode_attn: workspace %zu bytes < %zu", ws_bytes, plan.total);
    if ((uintptr_t)ws % 256) return fail(TQ_ERR_INVALID, "tq_decode_attn: workspace must be 256-byte aligned");
    if (scale == 0.0f) scale = 1.0f / std::sqrt((float)qk->d);
    return launch_decode(qk, qv, k, v, n_streams, T, T, G, q, q_dtype, plan, ws, scale, out, nullptr,
                         (hipStream_t)stream);
}

int tq_decode_attn_noalloc(const tq_quantizer* qk, const tq_quantizer* qv,
                           const tq_packed* k, const tq_packed* v,
                           int64_t n_streams, int64_t T, int G,
                           const void* q, int q_dtype, float scale, float* out, void* stream)
{
    clear_error();
    DecodePlan plan;
    int rc = check_decode_args(qk, qv, k, v, n_streams, T, G, q, q_dtype, scale, out, "tq_decode_attn_noalloc",
                               &plan);
    if (rc != TQ_OK || n_streams == 0) return rc;
    if (plan.total > kNoallocScratchBytes)
        return fail(TQ_ERR_WORKSPACE, "tq_decode_attn_noalloc: the call needs %zu bytes of scratch, more than the "
                    "library's fixed %zu", plan.total, kNoallocScratchBytes);
    void* ws = nullptr;
    if ((rc = noalloc_scratch(&ws)) != TQ_OK) return rc;
    if (scale == 0.0f) scale = 1.0f / std::sqrt((float)qk->d);
    return launch_decode(qk, qv, k, v, n_streams, T, T, G, q, q_dtype, plan, ws, scale, out, nullptr,
                         (hipStream_t)stream);
}

int tq_decode_step(const tq_quantizer* qk, const tq_quantizer* qv,
                   const tq_packed* k, const tq_packed* v,
                   int64_t n_streams, int64_t T, int64_t cap, int G,
                   const void* k_new, const void* v_new, int new_dtype,
                   const void* q, int q_dtype, float scale, float* out,
                   void* ws, size_t ws_bytes, void* stream)
{
    clear_error();
    int rc;
    if ((rc = check_quantizer(qk, "tq_decode_step", "key")) != TQ_OK) return rc;
    if ((rc = check_quantizer(qv, "tq_decode_step", "value")) != TQ_OK) return rc;
    if (qv->d != qk->d) return fail(TQ_ERR_UNSUPPORTED, "tq_decode_step: key d=%d != value d=%d", qk->d, qv->d);
    if (qv->qjl_m != 0)
        return fail(TQ_ERR_UNSUPPORTED, "tq_decode_step: value quantizer must be codes-only (qjl_m=0)");
    if (n_streams < 0) return fail(TQ_ERR_INVALID, "tq_decode_step: n_streams < 0");
    if (G < 1 || G > 16) return fail(TQ_ERR_UNSUPPORTED, "tq_decode_step: G=%d not in 1..16", G);
    if (n_streams == 0) return TQ_OK;
    if (T < 0 || cap <= T)
        return fail(TQ_ERR_INVALID, "tq_decode_step: need 0 <= T < cap (T=%lld, cap=%lld)", (long long)T,
                    (long long)cap);
    if (!std::isfinite(scale) || scale < 0) return fail(TQ_ERR_INVALID, "tq_decode_step: bad scale");
    if ((rc = check_packed(qk, k, "tq_decode_step", "k")) != TQ_OK) return rc;
    if ((rc = check_packed(qv, v, "tq_decode_step", "v")) != TQ_OK) return rc;
    if ((rc = check_dense(k_new, new_dtype, "tq_decode_step", "k_new")) != TQ_OK) return rc;
    if ((rc = check_dense(v_new, new_dtype, "tq_decode_step", "v_new")) != TQ_OK) return rc;
    if ((rc = check_dense(q, q_dtype, "tq_decode_step", "q")) != TQ_OK) return rc;
    if ((rc = check_dense(out, TQ_F32, "tq_decode_step", "out")) != TQ_OK) return rc;
    const DecodePlan plan =
        decode_plan(qk, n_streams, T + 1, G, !mfma_decode_widths(qk->mse_bits, qv->mse_bits), true);
    if (!ws || ws_bytes < plan.total)
        return fail(TQ_ERR_WORKSPACE, "tq_decode_step: workspace %zu bytes < %zu", ws_bytes, plan.total);
    if ((uintptr_t)ws % 256) return fail(TQ_ERR_INVALID, "tq_decode_step: workspace must be 256-byte aligned");
    if (scale == 0.0f) scale = 1.0f / std::sqrt((float)qk->d);
    const AppendArgs app{k_new, v_new, new_dtype, T};
    return launch_decode(qk, qv, k, v, n_streams, T + 1, cap, G, q, q_dtype, plan, ws, scale, out, &app,
                         (hipStream_t)stream);
}

}  // extern "C"
