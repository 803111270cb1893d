// Internal declarations shared by the host validation code and the kernels.
#ifndef TQ_INTERNAL_H
#define TQ_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#include "tq.h"

typedef struct ihipStream_t* hipStream_t;

namespace tq {

int fail(int code, const char* fmt, ...);
void clear_error();

int check_quantizer(const tq_quantizer* q, const char* who, const char* role);
int check_packed(const tq_quantizer* q, const tq_packed* p, const char* who, const char* role);
int check_dense(const void* p, int dtype, const char* who, const char* what);

size_t scores_ws(const tq_quantizer* q, int64_t n_q);
size_t scores_frag_bytes(const tq_quantizer* q, int64_t n_q);

// Decode-attention work split and workspace layout (offsets in bytes from
// the workspace base, each 256-byte aligned).
// One decode partial (per stream, chunk, head): max (log2 units), sum of
// weights, two pad words, then the d-float rotated-domain accumulator (16-byte
// aligned for vector loads).
constexpr int part_stride(int d) { return d + 4; }
constexpr int kPartAcc = 4;

// Blocks the MFMA decode plans for: two resident 256-thread blocks on each of
// the 256 compute units of an MI355X.
constexpr int kDecodeSlots = 512;

struct DecodePlan {
    bool mfma;          // MFMA kernel (d = 128, G <= 8, mfma_decode_widths); else a scalar kernel
    bool fused_append;  // decode step on the MFMA kernel: the new token is quantized inside it
    int64_t tc;         // tokens per block
    int n_chunks;       // blocks per stream
    int pchunks;        // partials per stream: n_chunks, plus the new token's with fused_append
    size_t off_qr, off_p, off_parts, total;
};
// Key and value code widths the MFMA decode kernel takes (d = 128, G <= 8):
// values of 1..4 bits with keys of 1..4 bits, values of 3, 4 or 8 bits with
// any key width. Other pairs run on the scalar kernels.
inline bool mfma_decode_widths(int bk, int bv) { return bv == 3 || bv == 4 || bv == 8 || (bk <= 4 && bv <= 4); }
// wide: a width pair the MFMA kernel does not take (mfma_decode_widths false).
// append: a decode step over T tokens whose last one is being appended; on the
// MFMA kernel the blocks then scan the T - 1 cached tokens and the new token
// becomes one more partial per stream.
DecodePlan decode_plan(const tq_quantizer* qk, int64_t n_streams, int64_t T, int G, bool wide,
                       bool append = false);

// Fixed scratch of tq_decode_attn_noalloc: a static device array of this many
// bytes per device, in place of a caller workspace.
constexpr size_t kNoallocScratchBytes = TQ_NOALLOC_SCRATCH_BYTES;
// Device address of the current device's scratch array (looked up once per
// device); TQ_ERR_DEVICE if the lookup fails.
int noalloc_scratch(void** ptr);

// compute units of the current device (cached per device)
int device_cus();

// kernel launchers (tq_*.hip); each returns TQ_OK or TQ_ERR_DEVICE
void launch_quantize_m128(const tq_quantizer* q, const void* x, int64_t n, const tq_packed* out,
                          hipStream_t s);
// d = 256 values (MSE codes, widths 1..4, fp16 or fp32 input) on MFMA
void launch_quantize_values_d256(const tq_quantizer* q, const void* x, int dtype, int64_t n,
                                 const tq_packed* out, hipStream_t s);
// d = 256 keys (MSE codes widths 1..4 plus the m = 256 sketch) on MFMA
void launch_quantize_keys_d256(const tq_quantizer* q, const void* x, int dtype, int64_t n,
                               const tq_packed* out, hipStream_t s);
int launch_quantize(const tq_quantizer* q, const void* x, int dtype, int64_t n,
                    const tq_packed* out, hipStream_t s);
int launch_qprep(const tq_quantizer* q, const void* queries, int dtype, int64_t nq,
                 float* qr, float* p, hipStream_t s);
int launch_dequantize(const tq_quantizer* q, const tq_packed* in, int64_t n, int include_qjl,
                      void* out, int dtype, hipStream_t s);
// The decode step's append: the new token of stream s (row s of k_new and
// v_new, [n_streams][d]) goes to vector s * stride + pos of the caches.
struct AppendArgs {
    const void* k_new;
    const void* v_new;
    int dtype;
    int64_t pos;
};

// decode over tokens 0..T-1 of each stream; stream s starts at vector s * stride;
// with app, the new tokens are quantized into the caches first (app->pos < T)
int launch_decode(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k,
                  const tq_packed* v, int64_t n_streams, int64_t T, int64_t stride, int G, const void* q,
                  int q_dtype, const DecodePlan& plan, void* ws, float scale, float* out,
                  const AppendArgs* app, hipStream_t s);
// d = 128: query fragments into `frags` (scores_frag_bytes(q, n_q)), then the MFMA score kernel
int launch_scores_mfma(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const void* queries,
                       int q_dtype, int64_t n_q, float* scores, void* frags, hipStream_t s);
// The MFMA decode kernel's in-kernel append (the decode step): the first
// block of each stream quantizes the stream's new key and value into slot
// `pos` and writes the new token's partial (index n_chunks of the stream).
struct AppendIn {
    const void* k_new;  // [n_streams][128] rows, or null: no append
    const void* v_new;
    int f16;            // rows are fp16 (else fp32)
    int64_t pos;
    const uint32_t* vdiag;
    const float* kbound;
    const float* vbound;
    uint32_t* kcodes;
    uint32_t* ksigns;
    uint16_t* knorm;
    uint16_t* krnorm;
    uint32_t* vcodes;
    uint16_t* vnorm;
};
// pchunks: partials per stream in `parts` (n_chunks, plus one with an append)
int launch_decode_mfma(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k,
                       const tq_packed* v, int64_t n_streams, int64_t T, int64_t stride, int G, const void* q,
                       int q_dtype, float zscale, float* parts, int n_chunks, int pchunks, int tc,
                       const AppendIn& ap, hipStream_t s);

// scalar kernels with run-time code widths 1..8 (tq_wide.hip): quantize and
// dequantize for widths 5..8 (and shapes the tuned kernels do not take), scores
// for d != 128, decode for shapes and width pairs the MFMA kernel does not
// take; scores and decode use prepared queries (launch_qprep)
int launch_quantize_wide(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* out,
                         hipStream_t s);
int launch_dequantize_wide(const tq_quantizer* q, const tq_packed* in, int64_t n, int include_qjl, void* out,
                           int dtype, hipStream_t s);
int launch_scores_wide(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const float* qr, const float* p,
                       int64_t n_q, float* scores, hipStream_t s);
int launch_decode_wide(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k, const tq_packed* v,
                       int64_t n_streams, int64_t T, int64_t stride, int G, const float* qr, const float* p,
                       float zscale, float* parts, int n_chunks, hipStream_t s);

}  // namespace tq

#endif
