/*
 * tq.h -- C ABI of the TurboQuant KV-cache hot path for AMD MI355X (gfx950).
 *
 * What the library computes (sources are the benchmark pages; see each entry):
 *  - a data-oblivious codebook per (d, bits): Lloyd-Max scalar quantizer for
 *    the law of one coordinate after a random rotation ("[Benchmark]
 *    TurboQuant 實測：KV Cache 3-bit 壓縮，真的零損失？", section
 *    "TurboQuant 是什麼：30 秒懶人包", step one; section "Lloyd-Max Codebook");
 *  - a quantizer: random +-1 diagonal and normalised Walsh-Hadamard rotation,
 *    stored norm, per-coordinate codes, and for keys a 1-bit QJL sketch of
 *    the residual with the residual norm (same section, step two);
 *  - scores q.k estimated directly from packed keys, unbiased with QJL
 *    (same section; "MSE-Only vs QJL：bias 差異確認");
 *  - reconstruction of vectors (the "dequantize back to BF16" path of the
 *    vLLM summary page, section "延遲：dequantization 是隱藏成本");
 *  - a fused decode-attention step over compressed K and V: the logits are
 *    computed on the compressed form instead of dequantizing the cache to
 *    BF16 first, which the vLLM summary page names as the hidden cost
 *    ("延遲：dequantization 是隱藏成本"), and the GB10 page attributes its slow
 *    estimated inner products to the missing fused kernel ("GB10 速度").
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller owns every buffer. The library never allocates
 *    device memory and keeps no state between calls except the thread-local
 *    error message and the fixed scratch array of tq_decode_attn_noalloc.
 *  - Device pointers are plain HIP device addresses on the current device;
 *    "stream" is a hipStream_t (NULL = the default stream). GPU work is
 *    enqueued asynchronously on that stream; nothing synchronises.
 *  - Argument errors are detected on the host before any launch and return a
 *    non-zero status; tq_last_error() then describes the problem. Launch
 *    failures return TQ_ERR_DEVICE. n == 0 is a no-op returning TQ_OK.
 *  - Alignment: every device buffer must be 16-byte aligned, except norm and
 *    rnorm arrays (2-byte aligned).
 *  - Supported shapes: d in {64, 128, 256}; mse_bits in 1..8 (widths 5..8,
 *    such as the 8-bit key / 4-bit value split measured in the vLLM benchmark
 *    summary, section "vLLM 工程師的實測", run on plain wide-code kernels;
 *    widths 1..4 on the tuned ones); qjl_m in {0, d}.
 *  - Inputs with ||x|| >= 65504 overflow the fp16 norm and are out of
 *    contract (stored norm becomes inf); non-finite inputs likewise.
 *
 * Packed layout of one vector (the contract tests are bit-exact on). The
 * layout is group-major: the d rotated coordinates form d/8 groups, group c
 * holding coordinates c + (d/8) t for t = 0..7.
 *  - codes: a little-endian bit stream of mse_bits * d bits stored as uint32
 *    words (stream bit k = bit k%32 of word k/32). Group c occupies stream
 *    bits [8 b c, 8 b c + 8 b) (b = mse_bits); inside it, code t occupies
 *    bits [b t, b t + b), least significant bit first. The code of a
 *    coordinate y is the number of boundaries strictly below y.
 *  - signs: a stream of qjl_m bits grouped the same way over the projection
 *    rows: bit t of byte j0 is 1 iff row j0 + (qjl_m/8) t of S applied to the
 *    residual is >= 0.
 *  - norm: fp16 (RNE) of ||x||; rnorm: fp16 (RNE) of the residual norm of the
 *    rotated unit vector.
 *  Vector v of an array of n vectors starts at codes + v*mse_bits*d/32,
 *  signs + v*qjl_m/32, norm + v, rnorm + v.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TQ_OK 0
#define TQ_ERR_INVALID 1      /* null / misaligned pointer, negative size, bad dtype */
#define TQ_ERR_UNSUPPORTED 2  /* d, bits, m or law outside the supported set */
#define TQ_ERR_WORKSPACE 3    /* workspace missing or too small */
#define TQ_ERR_DEVICE 4       /* HIP launch or runtime error */
#define TQ_ERR_NOCONV 5       /* codebook iteration did not converge */

/* element types of dense inputs / outputs */
#define TQ_F32 0
#define TQ_F16 1

/* workspace query operations */
#define TQ_OP_SCORES 1
#define TQ_OP_DECODE_ATTN 2

/* codebook laws */
#define TQ_LAW_GAUSSIAN 0     /* N(0, 1/d) */
#define TQ_LAW_SPHERE 1       /* exact law of one coordinate of a random unit vector in R^d */

/* Quantizer state. All pointers are device pointers owned by the caller. */
typedef struct tq_quantizer {
    int d;                       /* vector length: 64, 128 or 256 */
    int mse_bits;                /* bits of the scalar codes: 1..8 */
    int qjl_m;                   /* 0: codes only (values); d: codes + QJL signs (keys) */
    const float* centroids;      /* [2^mse_bits], ascending, from tq_codebook */
    const float* boundaries;     /* [2^mse_bits - 1], from tq_codebook */
    const uint32_t* diag_signs;  /* [d/32]; bit i set: coordinate i is negated before H */
    const uint16_t* S;           /* fp16 [qjl_m][d] row-major JL matrix; NULL if qjl_m == 0 */
} tq_quantizer;

/* Packed vectors (device pointers owned by the caller; layout above). */
typedef struct tq_packed {
    uint32_t* codes;             /* [n][mse_bits * d / 32] */
    uint32_t* signs;             /* [n][qjl_m/32]; NULL if qjl_m == 0 */
    uint16_t* norm;              /* [n] fp16 */
    uint16_t* rnorm;             /* [n] fp16; NULL if qjl_m == 0 */
} tq_packed;

/*
 * tq_codebook -- host only, synchronous.
 * Lloyd-Max quantizer with 2^bits levels for the coordinate law N(0, 1/d)
 * (the law that reproduces the distortions printed in the "Lloyd-Max
 * Codebook" section: 0.000270 at d=128, bits=3; 0.000135 at d=256).
 * Writes centroids (host float[2^bits]; each value is fp16-representable,
 * the fp16 RNE rounding of the exact solution, and the set is symmetric) and
 * boundaries (host float[2^bits - 1]; fp32 RNE of the exact midpoints of the
 * stored centroids). distortion (nullable) receives the analytic mean squared
 * error per coordinate of the stored codebook under the law.
 * law TQ_LAW_SPHERE instead solves for the exact law of one coordinate of a
 * uniformly random unit vector in R^d, density proportional to
 * (1 - t^2)^((d-3)/2) on [-1, 1] (Y^2 ~ Beta(1/2, (d-1)/2): the Beta law that
 * "TurboQuant 是什麼：30 秒懶人包" on the vLLM benchmark summary names; N(0, 1/d)
 * is its large-d limit); d >= 2 for it.
 * Supports d in 1..65536, bits in 1..8.
 * Returns TQ_OK, TQ_ERR_INVALID (null output), TQ_ERR_UNSUPPORTED, or
 * TQ_ERR_NOCONV.
 */
int tq_codebook(int d, int bits, int law, float* centroids, float* boundaries,
                double* distortion);

/*
 * tq_quantize -- quantize n vectors x[n][d] (row-major, TQ_F32 or TQ_F16)
 * into out (layout above). For each vector: norm n = ||x||; rotated unit
 * vector y = H (D .* x) / (sqrt(d) n) (y = 0 when n = 0); codes; and with
 * qjl_m = d: residual r = y - c[code], rnorm = ||r||, signs of S r.
 * Asynchronous on stream.
 */
int tq_quantize(const tq_quantizer* q, const void* x, int x_dtype, int64_t n,
                const tq_packed* out, void* stream);

/*
 * tq_scores -- scores[n_q][n_keys] (fp32) of estimated <query, key> for
 * queries[n_q][d] (TQ_F32 or TQ_F16) against n_keys packed keys:
 *   s = n * ( <q', c[codes]> + rnorm * sqrt(pi/2) / m * sum_j (S q')_j (2 sign_j - 1) )
 * with q' = H (D .* q) / sqrt(d). With qjl_m = 0 only the first term is used.
 * ws: device workspace of at least tq_workspace_size(TQ_OP_SCORES, q, n_q, n_keys, 0)
 * bytes (query preparation). Asynchronous on stream.
 */
int tq_scores(const tq_quantizer* q, const tq_packed* keys, int64_t n_keys,
              const void* queries, int q_dtype, int64_t n_q, float* scores,
              void* ws, size_t ws_bytes, void* stream);

/*
 * tq_dequantize -- reconstruct out[n][d] (TQ_F32 or TQ_F16):
 *   x_hat = n * D H ( c[codes] + [include_qjl] rnorm sqrt(pi/2)/m S^T (2 sign - 1) ) / sqrt(d).
 * include_qjl is ignored when qjl_m = 0. The score of a query against x_hat
 * equals tq_scores' estimate. Asynchronous on stream.
 */
int tq_dequantize(const tq_quantizer* q, const tq_packed* in, int64_t n, int include_qjl,
                  void* out, int out_dtype, void* stream);

/*
 * tq_decode_attn -- one decode step of attention over compressed K/V, the
 * scores taken directly from the packed keys (the estimator of tq_scores)
 * rather than from a dequantized copy ("延遲：dequantization 是隱藏成本" on the
 * vLLM benchmark summary; "GB10 速度" on the GX10 page).
 * n_streams streams (one stream = one (layer, KV head) token sequence) of T
 * tokens each; stream s, token t is packed vector s*T + t of k and of v.
 * q: [n_streams][G][d] (TQ_F32 or TQ_F16), G query heads per KV head.
 * For each stream s and head h:
 *   z_t = score(q_{s,h}, K_{s,t}) * scale   (scale = 1/sqrt(d) when scale == 0)
 *   out_{s,h} = sum_t softmax(z)_t * v_hat_{s,t}   (v_hat as tq_dequantize)
 * out: fp32 [n_streams][G][d]. qk (keys) and qv (values) must have the same d.
 * T >= 1; G in 1..16. ws: at least
 * tq_workspace_size(TQ_OP_DECODE_ATTN, qk, n_streams, T, G) bytes.
 * Asynchronous on stream.
 */
int tq_decode_attn(const tq_quantizer* qk, const tq_quantizer* qv,
                   const tq_packed* k, const tq_packed* v,
                   int64_t n_streams, int64_t T, int G,
                   const void* q, int q_dtype, float scale, float* out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * tq_decode_attn_noalloc -- tq_decode_attn without a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that forbid allocation). Same arguments, semantics, kernels
 * and results as tq_decode_attn, minus ws and ws_bytes: the workspace is a
 * fixed scratch array of TQ_NOALLOC_SCRATCH_BYTES in the library, one per
 * device, held until the process ends (its address is looked up on the first
 * call on each device). The call allocates nothing. A call whose workspace
 * (tq_workspace_size(TQ_OP_DECODE_ATTN, ...)) would exceed the scratch returns
 * TQ_ERR_WORKSPACE before any launch. Every call on one device shares that
 * device's scratch: calls that overlap in time on one device (other streams,
 * other threads) race and must be serialised by the caller; calls on one
 * stream are ordered and safe. Asynchronous on stream.
 */
#define TQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int tq_decode_attn_noalloc(const tq_quantizer* qk, const tq_quantizer* qv,
                           const tq_packed* k, const tq_packed* v,
                           int64_t n_streams, int64_t T, int G,
                           const void* q, int q_dtype, float scale, float* out,
                           void* stream);

/*
 * tq_decode_step -- append one token to every stream's compressed cache, then
 * one decode step of attention over the grown caches: the per-token
 * quantization that generation pays ("Google把32B模型壓到5GB顯存，實測后我發現3個坑",
 * section "結果：省顯存是真的，慢也是真的") fused into the decode step.
 * The caches hold stream s at packed vectors s*cap .. s*cap + cap - 1, with
 * tokens 0..T-1 valid. k_new, v_new: [n_streams][d] (new_dtype TQ_F32 or
 * TQ_F16), the new token's key and value per stream; they are quantized
 * (as tq_quantize, with qk and qv) into vector s*cap + T of k and v, which is
 * the only cache memory written. Then, as tq_decode_attn, out_{s,h} is the
 * attention of q_{s,h} over tokens 0..T of stream s (T + 1 tokens, the new
 * one included). 0 <= T < cap; G in 1..16. ws: at least
 * tq_workspace_size(TQ_OP_DECODE_ATTN, qk, n_streams, T + 1, G) bytes.
 * Errors as tq_decode_attn (TQ_ERR_INVALID also for T < 0 or T >= cap).
 * Asynchronous on stream.
 */
int tq_decode_step(const tq_quantizer* qk, const tq_quantizer* qv,
                   const tq_packed* k, const tq_packed* v,
                   int64_t n_streams, int64_t T, int64_t cap, int G,
                   const void* k_new, const void* v_new, int new_dtype,
                   const void* q, int q_dtype, float scale, float* out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * tq_workspace_size -- device workspace bytes for op:
 *   TQ_OP_SCORES:      n_a = n_q, n_b = n_keys, G ignored;
 *   TQ_OP_DECODE_ATTN: n_a = n_streams, n_b = T, G = heads per stream; the
 *                      value quantizer is not an argument, so the size covers
 *                      every value width (the wide-code kernels split the
 *                      tokens into more chunks than the tuned ones).
 * Returns 0 for unknown ops or unsupported quantizers.
 */
size_t tq_workspace_size(int op, const tq_quantizer* qk, int64_t n_a, int64_t n_b, int G);

/* Thread-local description of the last error ("" if none). */
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
