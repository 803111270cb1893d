// Fused decode attention over compressed K/V on MFMA (d = 128, up to 8 query
// heads per KV head).
//
// The per-token work is three small dense contractions over the G heads of a
// KV stream: sum_i q'_i c(k_i), sum_j p_j (+-1)_j (the QJL correction of
// "[Benchmark] TurboQuant 實測：KV Cache 3-bit 壓縮，真的零損失？", section
// "TurboQuant 是什麼：30 秒懶人包"), and sum_t w_t n_t c(v_t). All of them run
// on 16x16x32 f16 MFMAs with exact operands: key and value codes expand to
// fp16 centroids (fp16-representable by construction) and signs to +-1 via
// small LDS tables; the fp32 side (rotated query, its projection, the softmax
// weights) is split into an fp16 hi part and an fp16 lo part carried in two
// halves of the 16 output columns (query side) or rows (weight side), so the
// products are exact and only the fp32 accumulation rounds.
//
// Work split: a block owns a chunk of one stream's tokens (one block per
// chunk), each of its four waves a contiguous quarter, processed 32 tokens at
// a time, after the block has prepared its stream's queries (rotation, S q'
// on MFMA, score fragments) and its lookup tables:
//   scores  16 tokens x 16 columns (8 heads x hi/lo) per MFMA tile, K = 256
//           (128 code slots + 128 sign slots, in group-major order);
//   softmax exact max per 32-token block; the running max moves (and the
//           accumulators are rescaled) only when a block beats it by 2^8;
//   values  16 rows (8 heads x hi/lo) x 16 coordinates per tile, K = 32 tokens.
// The four waves merge in LDS; one partial (max, sum, rotated-domain
// accumulator) per block goes to the workspace, and the combine kernel merges
// the partials of a stream and undoes the value rotation.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

__device__ __forceinline__ float xor8(float x)
{
    // lane i <-> lane i ^ 8 inside each row of 16 lanes (DPP row rotate by 8)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}

// Lanes of the upper half of each 16-lane row (bank_mask 0xC) or of the lower
// half (0x3) take the value of lane i ^ 8; the others keep their own.
// The same exchange with no old value: a row rotation reads a lane of every
// row, so no lane keeps its old value and none needs one.
__device__ __forceinline__ float ror8(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}

template <int BANKS>
__device__ __forceinline__ float take_xor8(float x)
{
    const int i = __float_as_int(x);
    return __int_as_float(__builtin_amdgcn_update_dpp(i, i, 0x128, 0xF, BANKS, false));
}

// Value of lane (lane & ~3) + R within each quad of lanes (DPP quad_perm).
template <int R>
__device__ __forceinline__ float quad_bcast(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), R * 0x55, 0xF, 0xF, false));
}

// Query preparation, grid (stream, k-step t < d/32). Every block rotates the
// stream's G <= 8 queries (q' = H D q / sqrt(d); rows at or past `total` of
// the query array count as zero); block t then projects them
// onto the d/4 rows of S with index = t (mod d/32), one dot product per thread
// (p = S q'), and writes two score-GEMM B fragments: code k-step t and sign
// k-step d/32 + t. Column c < 8 carries the fp16 rounding of head c's value,
// column c + 8 the fp16 rounding of the remainder. Lane (g, col) element e of
// k-step t maps to coordinate (or projection row) (4 g + t) + (d/8) e, the
// group-major order the key codes arrive in. Arithmetic is fp32: its relative
// error (~1e-7) is far below what the hi/lo operands carry into the scores.
// (The decode kernel prepares its queries itself, in the same layout.)
template <int D, bool QJL, bool F16>
__global__ __launch_bounds__(256) void k_qprep_frag(const void* __restrict__ q, int G, int64_t total,
                                                    const uint32_t* __restrict__ diag,
                                                    const uint16_t* __restrict__ S,
                                                    half8_t* __restrict__ frags)
{
    static_assert(D == 128, "fragment layout is laid out for d = 128");
    constexpr int R = D / 64, KS = D / 32, KSTEPS = KS * (QJL ? 2 : 1);
    __shared__ float qs[8][D];
    __shared__ float ps[QJL ? 8 : 1][32];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t s = blockIdx.x;
    const int tt = blockIdx.y;
    // thread (h, i) projects row j = tt + (d/32) i of S onto head h; the block's
    // 32 rows are copied to LDS first (coalesced, each row once), so the copy
    // overlaps the rotation
    const int ph = tid >> 5, pi = tid & 31;
    __shared__ uint4 srs[QJL ? 32 : 1][D / 8 + 1];
    if constexpr (QJL) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = tid + 256 * k, row = e >> 4, c = e & 15;
            srs[row][c] = reinterpret_cast<const uint4*>(S + (int64_t)(tt + KS * row) * D)[c];
        }
    }
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);
    const float inv_sqrt_d = 0.08838834764831845f;  // 1 / sqrt(128)
    // heads wid and wid + 4 of this wave, loaded together and rotated as two
    // independent chains (one transform over both slots' pairs)
    {
        float y[2 * R];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int h = wid + 4 * hh;
#pragma unroll
            for (int r = 0; r < R; ++r)
                y[R * hh + r] =
                    h < G && s * G + h < total ? flip(load_elem<F16>(q, (s * G + h) * D + 64 * r + lane), dm[r]) : 0.f;
        }
        float ya[R], yb[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ya[r] = y[r];
            yb[r] = y[R + r];
        }
        fwht_wave_dpp<R>(ya, lane);
        fwht_wave_dpp<R>(yb, lane);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            qs[wid][64 * r + lane] = ya[r] * inv_sqrt_d;
            qs[wid + 4][64 * r + lane] = yb[r] * inv_sqrt_d;
        }
    }
    __syncthreads();
    if constexpr (QJL) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            const uint4 sw = srs[pi][c];
            const uint32_t w4[4] = {sw.x, sw.y, sw.z, sw.w};
            const float4 qa = *reinterpret_cast<const float4*>(&qs[ph][8 * c]);
            const float4 qb = *reinterpret_cast<const float4*>(&qs[ph][8 * c + 4]);
            const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
            for (int k = 0; k < 8; ++k)
                acc[k & 3] = fmaf(h2f((uint16_t)(w4[k >> 1] >> (16 * (k & 1)))), qv[k], acc[k & 3]);
        }
        ps[ph][pi] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        __syncthreads();
    }
    if (tid < (QJL ? 128 : 64)) {
        const bool sgn = tid >= 64;
        const int l = tid & 63;
        const int col = l & 15, g = l >> 4, head = col & 7;
        const bool lo = col >= 8;
        half8_t f;
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) {
            // coordinate (row) 4 g + tt + (d/8) ee; as a row of this block: i = g + 4 ee
            float val = 0.f;
            if (head < G) val = sgn ? ps[QJL ? head : 0][(g + 4 * ee) & 31] : qs[head][KS * g + tt + (D / 8) * ee];
            const _Float16 hi = (_Float16)val;
            f[ee] = lo ? (_Float16)(val - (float)hi) : hi;
        }
        frags[(s * KSTEPS + (sgn ? KS + tt : tt)) * 64 + l] = f;
    }
}

// Entries of a block's key code table: a byte of four codes (widths 1, 2), a
// field of two codes (3, 4), or one code (5..8, where a two-code table would
// reach 256 KiB).
__host__ __device__ constexpr int key_lut_entries(int bk)
{
    return bk <= 2 ? 1 << (4 * bk) : (bk <= 4 ? 1 << (2 * bk) : 1 << bk);
}

// Key lookup tables of a block: for up to 2-bit codes one entry maps a byte of
// four codes to four fp16 centroids (klut4), for 3 and 4 bits a field of two
// codes to two (klut2), above 4 bits one code to its fp16 centroid in both
// halves (klut2); slut maps a byte of sign bits to eight fp16 +-1 values.
template <int BK, bool QJL>
__device__ void fill_key_luts(uint2* klut4, uint32_t* klut2, uint4* slut, const float* __restrict__ kcent)
{
    constexpr bool K4 = BK <= 2;
    constexpr int KLUT = key_lut_entries(BK);
    for (int i = threadIdx.x; i < KLUT; i += blockDim.x) {
        if constexpr (K4) {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = f2h(kcent[(i >> (BK * j)) & ((1 << BK) - 1)]);
            klut4[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else if constexpr (BK <= 4) {
            klut2[i] = (uint32_t)f2h(kcent[i & ((1 << BK) - 1)]) | ((uint32_t)f2h(kcent[i >> BK]) << 16);
        } else {
            klut2[i] = (uint32_t)f2h(kcent[i]) * 0x10001u;
        }
    }
    if constexpr (QJL)
        for (int i = threadIdx.x; i < 256; i += blockDim.x) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = (((i >> (2 * j)) & 1) ? 0x3C00u : 0xBC00u) | ((((i >> (2 * j + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
            slut[i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
}

// fill_key_luts from fp16 centroids already in LDS (kc16[code]), by the 256
// threads of a block (fixed trip counts, so the reads of an entry issue ahead
// of the writes).
template <int BK, bool QJL>
__device__ void fill_key_luts_lds(uint2* klut4, uint32_t* klut2, uint4* slut, const uint16_t* kc16, bool codes)
{
    constexpr bool K4 = BK <= 2;
    constexpr int KLUT = key_lut_entries(BK);
#pragma unroll
    for (int k = 0; k < (KLUT + 255) / 256; ++k) {
        const int i = (int)threadIdx.x + 256 * k;
        if (!codes || i >= KLUT) continue;
        if constexpr (K4) {
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = kc16[(i >> (BK * j)) & ((1 << BK) - 1)];
            klut4[i] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else if constexpr (BK <= 4) {
            klut2[i] = (uint32_t)kc16[i & ((1 << BK) - 1)] | ((uint32_t)kc16[i >> BK] << 16);
        } else {
            klut2[i] = (uint32_t)kc16[i] * 0x10001u;
        }
    }
    if constexpr (QJL) {
        const int i = (int)threadIdx.x;  // sign byte i
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (((i >> (2 * j)) & 1) ? 0x3C00u : 0xBC00u) | ((((i >> (2 * j + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
        slut[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// A operand of code group t of a key (8 codes, 8 BK bits at bit 8 BK t of
// the lane's BK code words) as fp16 centroids.
template <int BK>
__device__ __forceinline__ half8_t key_codes_a(const uint32_t (&kf)[BK], int t, const uint2* klut4,
                                               const uint32_t* klut2)
{
    constexpr bool K4 = BK <= 2;
    constexpr int FB = 8 * BK;
    const int bit = FB * t;
    if constexpr (BK > 4) {
        // a 40..64-bit field over two or three words; eight single-code lookups
        const int lo = bit >> 5, sh = bit & 31;
        uint64_t f = (((uint64_t)kf[lo + 1] << 32) | kf[lo]) >> sh;
        if (sh + FB > 64) f |= (uint64_t)kf[lo + 2] << (64 - sh);
        uint32_t wds[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t a = klut2[(uint32_t)(f >> (BK * 2 * j)) & ((1u << BK) - 1u)];
            const uint32_t b = klut2[(uint32_t)(f >> (BK * (2 * j + 1))) & ((1u << BK) - 1u)];
            wds[j] = __builtin_amdgcn_perm(b, a, 0x05040100u);  // low half of a, then low half of b
        }
        return __builtin_bit_cast(half8_t, wds);
    }
    uint32_t field;
    if constexpr (BK == 4) field = kf[t];
    else {
        const uint64_t cat = (bit >> 5) + 1 < BK ? ((uint64_t)kf[(bit >> 5) + 1] << 32) | kf[bit >> 5]
                                                 : (uint64_t)kf[bit >> 5];
        field = (uint32_t)(cat >> (bit & 31)) & ((1u << FB) - 1u);
    }
    if constexpr (K4) {
        const uint2 e0 = klut4[field & ((1u << (4 * BK)) - 1u)];
        const uint2 e1 = klut4[field >> (4 * BK)];
        const uint32_t wds[4] = {e0.x, e0.y, e1.x, e1.y};
        return __builtin_bit_cast(half8_t, wds);
    } else {
        uint32_t wds[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) wds[j] = klut2[(field >> (2 * BK * j)) & ((1u << (2 * BK)) - 1u)];
        return __builtin_bit_cast(half8_t, wds);
    }
}

// Table address (index byte k of y) * 256 + copy byte: one v_perm that puts
// byte k of y in bits 8..15 next to the low byte of `copy`.
template <int K>
__device__ __forceinline__ uint32_t row_addr(uint32_t y, uint32_t copy)
{
    return __builtin_amdgcn_perm(y, copy, 0x0C0C0000u | ((4u + K) << 8));
}

// max of three floats without NaN canonicalization (scores are never NaN)
__device__ __forceinline__ float max3f(float a, float b, float c)
{
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// One 32-token step's packed inputs for one lane (prefetched a step ahead).
template <int BK, int BV>
struct Step {
    uint32_t kf[2][BK];   // key code words of this lane's 4 groups, tiles 0 and 1
    uint32_t sf[2];       // key sign bytes of this lane's 4 groups
    uint32_t x0[8], x1[8];// value field words (x1: second word, 3- and 8-bit codes only)
    uint16_t nk[2], ng[2], nv[2];  // norms of token tb + 16 u + 4 g + (col & 3), u = 0, 1
};

// Loads of one step. Token indices are clamped to the last token of the
// wave's range (w1 - 1 >= tb), so every load is unconditional and in bounds;
// tokens past the range get a score of -inf and a weight of 0 later, so the
// values read for them never reach the result.
template <int D, int BK, bool QJL, int BV>
__device__ __forceinline__ void load_step(Step<BK, BV>& st, int64_t tb, int64_t w1, int64_t base, int lane,
                                          const uint32_t* __restrict__ kcodes,
                                          const uint32_t* __restrict__ ksigns,
                                          const uint16_t* __restrict__ knorm,
                                          const uint16_t* __restrict__ krnorm,
                                          const uint32_t* __restrict__ vcodes,
                                          const uint16_t* __restrict__ vnorm)
{
    constexpr int KW = BK * D / 32, VW = BV * D / 32, SWN = D / 32;
    const int col = lane & 15, g = lane >> 4;
    const int64_t last = w1 - 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t tA = base + min(tb + 16 * u + col, last);
#pragma unroll
        for (int w = 0; w < BK; ++w) st.kf[u][w] = kcodes[tA * KW + BK * g + w];
        st.sf[u] = QJL ? ksigns[tA * SWN + g] : 0u;
    }
    const int w = (8 * BV * col) >> 5;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t t = base + min(tb + 16 * (e >> 2) + 4 * g + (e & 3), last);
        const uint32_t* rec = vcodes + t * VW;
        st.x0[e] = rec[w];
        // 3-bit fields may straddle two words; the last field of a token does not
        if constexpr (BV == 3 || BV == 8) st.x1[e] = rec[w + 1 < VW ? w + 1 : w];
        else st.x1[e] = 0u;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t t = base + min(tb + 16 * u + 4 * g + (col & 3), last);
        st.nk[u] = knorm[t];
        st.ng[u] = QJL ? krnorm[t] : (uint16_t)0;
        st.nv[u] = vnorm[t];
    }
}

// Per-lane element offsets of a step's loads, relative to the step's first
// token (the same for every step).
struct LaneOff {
    int k, s, v, v1, n;
};

template <int D, int BK, int BV>
__device__ __forceinline__ LaneOff lane_offsets(int lane)
{
    constexpr int KW = BK * D / 32, VW = BV * D / 32, SWN = D / 32;
    const int col = lane & 15, g = lane >> 4;
    const int w = (8 * BV * col) >> 5;
    LaneOff o;
    o.k = col * KW + BK * g;
    o.s = col * SWN + g;
    o.v = 4 * g * VW + w;
    o.v1 = 4 * g * VW + (w + 1 < VW ? w + 1 : w);
    o.n = 4 * g + (col & 3);
    return o;
}

// Loads of a step whose 32 tokens all lie in the wave's range: wave-uniform
// row pointers (t0 = first token of the step) plus the fixed lane offsets, so
// no per-load address arithmetic. Same values as load_step.
template <int D, int BK, bool QJL, int BV>
__device__ __forceinline__ void load_full(Step<BK, BV>& st, int64_t t0, const LaneOff& lo,
                                          const uint32_t* __restrict__ kcodes,
                                          const uint32_t* __restrict__ ksigns,
                                          const uint16_t* __restrict__ knorm,
                                          const uint16_t* __restrict__ krnorm,
                                          const uint32_t* __restrict__ vcodes,
                                          const uint16_t* __restrict__ vnorm)
{
    constexpr int KW = BK * D / 32, VW = BV * D / 32, SWN = D / 32;
    const uint32_t* kc = kcodes + t0 * KW;
    const uint32_t* vc = vcodes + t0 * VW;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int w = 0; w < BK; ++w) st.kf[u][w] = kc[lo.k + 16 * u * KW + w];
        st.sf[u] = QJL ? ksigns[t0 * SWN + lo.s + 16 * u * SWN] : 0u;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        st.x0[e] = vc[lo.v + (16 * (e >> 2) + (e & 3)) * VW];
        if constexpr (BV == 3 || BV == 8) st.x1[e] = vc[lo.v1 + (16 * (e >> 2) + (e & 3)) * VW];
        else st.x1[e] = 0u;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        st.nk[u] = knorm[t0 + lo.n + 16 * u];
        st.ng[u] = QJL ? krnorm[t0 + lo.n + 16 * u] : (uint16_t)0;
        st.nv[u] = vnorm[t0 + lo.n + 16 * u];
    }
}

// The decode step's new token, coded inside the decode kernel: the code of a
// rotated unit coordinate y is the number of codebook boundaries strictly
// below it (the 2^B - 1 sorted boundaries, the same for every lane: up to 4
// bits a count over registers loaded once, above that a branch-free binary
// search over the boundaries in memory).
template <int B>
__device__ __forceinline__ int append_code(float y, const float (&br)[B <= 4 ? (1 << B) - 1 : 1],
                                           const float* __restrict__ bnd)
{
    constexpr int L = 1 << B;
    int idx = 0;
    if constexpr (B <= 4) {
#pragma unroll
        for (int j = 0; j < L - 1; ++j) idx += br[j] < y ? 1 : 0;
    } else {
#pragma unroll
        for (int step = L / 2; step >= 1; step >>= 1) idx += bnd[idx + step - 1] < y ? step : 0;
    }
    return idx;
}

// Store one vector's codes, held by a wave as lane l: coordinates l (code c0)
// and l + 64 (code c1), in the group-major stream: group c (coordinates
// c + 16 t) is an 8B-bit field with code t at bit B t, stream bytes
// B c .. B c + B - 1. Lanes c, c + 16, c + 32, c + 48 hold group c's codes;
// their shifted codes are OR-ed together and lane c stores the field.
template <int B>
__device__ __forceinline__ void append_store_codes(int c0, int c1, int lane, unsigned char* __restrict__ dst)
{
    const int q = lane >> 4;
    const uint64_t f = ((uint64_t)c0 << (B * q)) | ((uint64_t)c1 << (B * (4 + q)));
    uint32_t lo = (uint32_t)f, hi = (uint32_t)(f >> 32);
    lo |= (uint32_t)__shfl_xor((int)lo, 16);
    hi |= (uint32_t)__shfl_xor((int)hi, 16);
    lo |= (uint32_t)__shfl_xor((int)lo, 32);
    hi |= (uint32_t)__shfl_xor((int)hi, 32);
    if (lane < 16) {
        const uint64_t g = ((uint64_t)hi << 32) | lo;
#pragma unroll
        for (int b = 0; b < B; ++b) dst[B * lane + b] = (unsigned char)(g >> (8 * b));
    }
}

// Issue priority of a scanning wave from its progress (steps done of its
// range): 3 in the first quarter down to 0 in the last. Two blocks share a
// compute unit and the arbiter favours the older waves on ties; with these
// levels a wave that has fallen behind wins the ties instead (measured: the
// block dispatched second trailed the first by 5.3 us at the 128K shape
// without them, 2.4 us with them, and the call ended about 1 us earlier).
__device__ __forceinline__ void progress_prio(int64_t done, int64_t total)
{
    const int q = total > 0 ? (int)((4 * done) / total) : 4;
    if (q <= 0) __builtin_amdgcn_s_setprio(3);
    else if (q == 1) __builtin_amdgcn_s_setprio(2);
    else if (q == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

template <int D, int BK, bool QJL, int BV>
__global__ __launch_bounds__(256, 2) void k_decode_mfma(const uint32_t* __restrict__ kcodes,
                                                     const uint32_t* __restrict__ ksigns,
                                                     const uint16_t* __restrict__ knorm,
                                                     const uint16_t* __restrict__ krnorm,
                                                     const uint32_t* __restrict__ vcodes,
                                                     const uint16_t* __restrict__ vnorm, int64_t T,
                                                     int64_t stride, int G, const void* __restrict__ q,
                                                     int q_f16, const uint32_t* __restrict__ kdiag,
                                                     const uint16_t* __restrict__ S,
                                                     const float* __restrict__ kcent,
                                                     const float* __restrict__ vcent, float zscale,
                                                     float* __restrict__ parts, int n_chunks, int pchunks,
                                                     int tc, const AppendIn ap)
{
    static_assert(D == 128, "MFMA decode is laid out for d = 128");
    constexpr int KS = D / 32;                 // 4 code groups per lane per token
    constexpr int KSTEPS = KS * (QJL ? 2 : 1);
    constexpr int CT = D / 16;                 // value coordinate tiles
    constexpr bool K4 = BK <= 2;               // one key table entry = 4 codes (else 2, or 1 above 4 bits)
    constexpr int KLUT = key_lut_entries(BK);
    constexpr int VLUT = BV <= 4 ? 1 << (2 * BV) : 1 << BV;  // code pairs, or single codes above 4 bits
    constexpr float kappa = 1.2533141373155003f / D;  // sqrt(pi/2) / m

    // 2-bit keys and 4-bit values: tables in 256-byte rows, entry e's 32 value
    // copies (4 bytes, lane l reads copy l % 32) in bytes 0..127 and its 16 key
    // copies (8 bytes, copy l % 16) in 128..255. The index is a byte of the
    // packed codes, so an address is that byte next to the lane's copy byte (one
    // v_perm). The rows also hold the value table of other widths (first half),
    // and, after the scan, the merge buffers (rebuilt for a further item).
    // 3-bit values (V12): one table of 4096 entries indexed by two codes of each
    // of a token pair (6 bits each), giving the B-operand words of two value
    // tiles per lookup; the key table is then the plain one.
    constexpr bool V12 = BV == 3;
    constexpr bool PV = BV == 4, PK = BK == 2 && !V12, ROWS = PV || PK;
    __shared__ __align__(16) uint32_t rows[ROWS ? 256 : 1][64];
    __shared__ uint2 klut4[K4 && !PK ? KLUT : 1];
    __shared__ uint32_t klut2[K4 ? 1 : KLUT];
    __shared__ uint4 slut[QJL ? 256 : 1];
    __shared__ uint32_t vlut[ROWS || V12 ? 1 : VLUT][32];  // one copy per bank: lane l reads copy l % 32
    // even-tile words at [i], odd-tile words at [kV12Odd + i]: 16388 bytes apart, a
    // distance no paired LDS read spans, so each lands in its operand's register
    constexpr int kV12Odd = 4097;
    __shared__ __align__(16) uint32_t vlut12[V12 ? 2 * kV12Odd : 1];
    __shared__ float mrg_m[4][8], mrg_l[4][8], mrg_f[4][8], mrg_x[8];
    __shared__ __align__(16) float mrg_own[ROWS || V12 ? 1 : 4][8][D];
    float(*const mrg_o)[8][D] = ROWS ? reinterpret_cast<float(*)[8][D]>(&rows[0][0])
                                     : (V12 ? reinterpret_cast<float(*)[8][D]>(&vlut12[0]) : mrg_own);
    static_assert(!V12 || 2 * kV12Odd * 4 >= 4 * 8 * D * 4, "the merge buffers fit in the 3-bit value table");
    const char* const rowsb = reinterpret_cast<const char*>(&rows[0][0]);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int col = lane & 15, g = lane >> 4;
    const LaneOff loff = lane_offsets<D, BK, BV>(lane);
    const uint32_t vcopy = (lane & 31) * 4, kcopy = 128 + (lane & 15) * 8;  // copy bytes in a row
    // value table entry e, copy of this lane
    auto vl = [&](uint32_t e) -> uint32_t {
        if constexpr (ROWS) return rows[e][lane & 31];
        else return vlut[e][lane & 31];
    };

    // the two codebooks (one global load per thread) are the first loads in
    // flight, so they can be waited for while the first item's loads are not
    __shared__ __align__(16) uint16_t cb16[2][256];
    const float kc_v = kcent[min(tid, (1 << BK) - 1)];  // clamped: no branch around the loads
    const float vc_v = vcent[min(tid, (1 << BV) - 1)];

    const int64_t item = blockIdx.x;  // one work item (stream, chunk) per block

    // Decode step (ap.k_new set): the first block of each stream also quantizes
    // the stream's new key and value into slot ap.pos (wave 0 the key, wave 1
    // the value, as tq_quantize would) and writes the new token's partial,
    // index n_chunks of the stream; the blocks scan the ap.pos cached tokens.
    // Its inputs are the first loads in flight.
    const bool appb = ap.k_new != nullptr && (uint32_t)item % (uint32_t)n_chunks == 0u;
    const int64_t as = (int64_t)((uint32_t)item / (uint32_t)n_chunks);  // the stream (used by the append only)
    uint32_t axw[2] = {0u, 0u};  // new row words (fp32 bits, or the word holding the fp16 value)
    uint32_t dmv[2] = {0u, 0u};  // value rotation's sign flips
    float kbr[BK <= 4 ? (1 << BK) - 1 : 1], vbr[BV <= 4 ? (1 << BV) - 1 : 1];
    if (appb) {
        if (wid < 2) {
            const uint32_t* src = static_cast<const uint32_t*>(wid == 0 ? ap.k_new : ap.v_new);
            const int64_t row = as * D + lane;
#pragma unroll
            for (int r = 0; r < 2; ++r) axw[r] = src[ap.f16 ? (row + 64 * r) >> 1 : row + 64 * r];
        }
        if constexpr (BK <= 4)
#pragma unroll
            for (int j = 0; j < (1 << BK) - 1; ++j) kbr[j] = ap.kbound[j];
        if constexpr (BV <= 4)
#pragma unroll
            for (int j = 0; j < (1 << BV) - 1; ++j) vbr[j] = ap.vbound[j];
        load_diag<2>(ap.vdiag, lane, dmv);
    }

    // the current item's geometry and first loads: the first 512 value norms of
    // each wave's range (indices clamped into it), then the first two full steps
    // and the query fragments. Loads complete in order, so the norms, needed
    // first, are issued first.
    int64_t s, base, w0, w1, nfull;
    int chunk;
    uint16_t hv[8];
    Step<BK, BV> sa, sb;
    half8_t bq[KSTEPS];
    // query preparation inputs of the item's stream: heads wid and wid + 4 (two
    // coordinates per lane each; heads past G read as zero) and this wave's two
    // 16-row tiles of S for the projection (MFMA A operands, 8 per lane)
    // rows padded by 4 floats: the fragment reads take the same offset of eight
    // heads' rows at once, which then fall in eight different bank groups
    __shared__ __align__(16) float qs[8][D + 4];             // q' = H D q / sqrt(d), per head
    __shared__ __align__(16) float ps[QJL ? 8 : 1][D + 4];  // p = S q', per head
    uint32_t qw[2][2];  // raw query words (fp32 bits, or the 32-bit word holding the fp16 value)
    uint4 sA[QJL ? 2 : 1][4];
    uint32_t dm[2];
    load_diag<2>(kdiag, lane, dm);
    auto begin_item = [&]() {
        // items number fewer than 2^31 (streams times chunks): 32-bit division
        const uint32_t it = (uint32_t)item, nc = (uint32_t)n_chunks;
        s = it / nc;
        chunk = (int)(it - (uint32_t)s * nc);
        base = s * stride;
        const int64_t c0 = (int64_t)chunk * tc;
        const int64_t c1 = c0 + tc < T ? c0 + tc : T;
        w0 = c0 + (int64_t)wid * (tc / 4);
        w1 = w0 + tc / 4 < c1 ? w0 + tc / 4 : c1;
        nfull = w1 > w0 ? (w1 - w0) >> 5 : 0;  // a wave past the chunk's end has none
        // no branches around these loads, so that waiting for the codebooks does not
        // wait for them: indices are clamped to the range's last token, or to the
        // chunk's last one for a wave past its end
        // (a decode step on empty caches scans nothing: slot 0 is then read, and unused)
        const int64_t lim = w1 > w0 ? w1 : (c1 > 0 ? c1 : 1);
        // the query (clamped head index, zeroed past G) and S first: they are needed first
        // (32-bit word loads for both dtypes, no branch: the fp16 pair's word)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int64_t row = (s * G + min(wid + 4 * hh, G - 1)) * D + lane;
#pragma unroll
            for (int r = 0; r < 2; ++r)
                qw[hh][r] = static_cast<const uint32_t*>(q)[q_f16 ? (row + 64 * r) >> 1 : row + 64 * r];
        }
        if constexpr (QJL) {
            // A operand of tile 2 wid + u, k-step k: row j = 16 (2 wid + u) + col,
            // coordinates 32 k + 8 g .. + 7
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    sA[u][k] = *reinterpret_cast<const uint4*>(S + (16 * (2 * wid + u) + col) * D + 32 * k + 8 * g);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) hv[k] = vnorm[base + min(w0 + lane + 64 * k, lim - 1)];
        load_step<D, BK, QJL, BV>(sa, w0, lim, base, lane, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
        load_step<D, BK, QJL, BV>(sb, w0 + 32, lim, base, lane, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
    };
    begin_item();

    // fp16 parts of a pair of fp32 values for this lane's column half: fp16(x) for
    // col < 8, fp16(x - fp16(x)) for col >= 8; both are fp16(x + negsel fp16(x))
    const float negsel = col >= 8 ? -1.0f : 0.0f;
    // (each mixlo leaves its high half to the mixhi that follows, so it is an
    // output-only operand and needs no initial value)
    auto split2 = [&](float x0, float x1) -> uint32_t {
        uint32_t hw, ow;
        asm("v_fma_mixlo_f16 %0, %1, 1.0, 0" : "=v"(hw) : "v"(x0));
        asm("v_fma_mixhi_f16 %0, %1, 1.0, 0" : "+v"(hw) : "v"(x1));
        asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(ow) : "v"(hw), "v"(negsel), "v"(x0));
        asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(ow) : "v"(hw), "v"(negsel), "v"(x1));
        return ow;
    };
    const int head = col & 7;

    // ---- prologue, while the first steps' loads are in flight: lookup tables
    // (codes -> fp16 centroids, sign bytes -> +-1) and the query preparation
    // (q' by the rotation, p = S q' on MFMA, then the score B fragments bq). Lane
    // (g, col) element e of k-step t holds coordinate (or projection row)
    // 4 g + t + 16 e of head col & 7, split as split2 does, in the group-major
    // order the key codes arrive in. Arithmetic is fp32 (the products of fp16 S
    // and the fp16 parts of q' are exact). LDS-only barriers.

    // (1) the codebooks and q' = H D q / sqrt(d) to LDS. Every thread writes a
    // codebook slot (slots past the codebook repeat its last centroid and are
    // never read): no branch for the compiler to sink the loads into.
    cb16[0][tid] = f2h(kc_v);
    cb16[1][tid] = f2h(vc_v);
    {
        constexpr float inv_sqrt_d = 0.08838834764831845f;  // 1 / sqrt(128)
        float qv[2][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float v = q_f16 ? h2f((uint16_t)(qw[hh][r] >> (16 * (lane & 1)))) : __uint_as_float(qw[hh][r]);
                qv[hh][r] = wid + 4 * hh < G ? v : 0.f;  // heads past G are zero
            }
        float ya[2] = {flip(qv[0][0], dm[0]), flip(qv[0][1], dm[1])};
        float yb[2] = {flip(qv[1][0], dm[0]), flip(qv[1][1], dm[1])};
        fwht_wave_dpp<2>(ya, lane);
        fwht_wave_dpp<2>(yb, lane);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            qs[wid][64 * r + lane] = ya[r] * inv_sqrt_d;
            qs[wid + 4][64 * r + lane] = yb[r] * inv_sqrt_d;
        }
    }
    // the new key (wave 0) or value (wave 1): n = ||x||, H D x (unnormalised)
    float ay[2] = {0.f, 0.f}, anrm = 0.f;
    if (appb && wid < 2) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float v = ap.f16 ? h2f((uint16_t)(axw[r] >> (16 * (lane & 1)))) : __uint_as_float(axw[r]);
            ay[r] = flip(v, wid == 0 ? dm[r] : dmv[r]);
        }
        anrm = sqrtf(wave_sum_dpp(ay[0] * ay[0] + ay[1] * ay[1]));
        fwht_wave_dpp<2>(ay, lane);
    }
    lds_barrier();

    // (2) the tables from the codebooks, and p = S q' to LDS
    // value table entry e: a code pair, or one code above 4 bits in both halves
    auto ventry = [&](int e) -> uint32_t {
        if constexpr (BV <= 4) return (uint32_t)cb16[1][e & ((1 << BV) - 1)] | ((uint32_t)cb16[1][e >> BV] << 16);
        else return (uint32_t)cb16[1][e] * 0x10001u;
    };
    // Fixed trip counts throughout, so that the codebook reads of all of a
    // thread's entries issue ahead of its table writes.
    if constexpr (ROWS) {
        // the row tables: 16 uint4 per row, 8 of value copies and 8 of key copies;
        // thread t writes uint4 t % 8 of both halves of rows t / 8 + 32 k, a wave
        // eight half-rows per instruction
        const int qq = tid & 7;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int e = (tid >> 3) + 32 * k;
            if (e < VLUT) {
                const uint32_t v = ventry(e);
                reinterpret_cast<uint4*>(&rows[e][0])[qq] = make_uint4(v, v, v, v);
            }
        }
        if constexpr (PK) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = (tid >> 3) + 32 * k;
                uint32_t h[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) h[j] = cb16[0][(e >> (2 * j)) & 3];
                const uint32_t x = h[0] | (h[1] << 16), y = h[2] | (h[3] << 16);
                reinterpret_cast<uint4*>(&rows[e][0])[8 + qq] = make_uint4(x, y, x, y);
            }
        }
        fill_key_luts_lds<BK, QJL>(klut4, klut2, slut, cb16[0], !PK);
    } else {
        fill_key_luts_lds<BK, QJL>(klut4, klut2, slut, cb16[0], true);
        if constexpr (V12) {
            // entry aa | bb << 6: (codes aa & 7, bb & 7) for the even tile, (aa >> 3, bb >> 3) for the odd one
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = tid + 256 * k, aa = i & 63, bb = i >> 6;
                vlut12[i] = (uint32_t)cb16[1][aa & 7] | ((uint32_t)cb16[1][bb & 7] << 16);
                vlut12[kV12Odd + i] = (uint32_t)cb16[1][aa >> 3] | ((uint32_t)cb16[1][bb >> 3] << 16);
            }
        } else {
            // value table: entry e in all 32 copies; a wave writes 8 entries' 128-byte
            // rows per instruction
#pragma unroll
            for (int k = 0; k < (VLUT * 8 + 255) / 256; ++k) {
                const int i = tid + 256 * k;
                if (i < VLUT * 8) {
                    const uint32_t v = ventry(i >> 3);
                    reinterpret_cast<uint4*>(&vlut[i >> 3][0])[i & 7] = make_uint4(v, v, v, v);
                }
            }
        }
    }
    if constexpr (QJL) {
        // tiles 2 wid, 2 wid + 1 of p: rows j, columns = head col & 7's hi / lo parts
        float4_t pa[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float4 x0 = *reinterpret_cast<const float4*>(&qs[head][32 * k + 8 * g]);
            const float4 x1 = *reinterpret_cast<const float4*>(&qs[head][32 * k + 8 * g + 4]);
            const uint32_t bw[4] = {split2(x0.x, x0.y), split2(x0.z, x0.w), split2(x1.x, x1.y), split2(x1.z, x1.w)};
            const half8_t b = __builtin_bit_cast(half8_t, bw);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                pa[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, sA[u][k]), b, pa[u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pv = pa[u][r] + xor8(pa[u][r]);  // hi + lo columns
                if (col < 8) ps[head][16 * (2 * wid + u) + 4 * g + r] = pv;
            }
    }
    // the new token's codes against the codebook boundaries, its fp16 centroids
    // (ac) and, for the key, the residual r = y - c (ar) and its norm; norms and
    // codes go to the caches
    float ac[2] = {0.f, 0.f}, ar[2] = {0.f, 0.f}, arn = 0.f;
    if (appb && wid < 2) {
        const float inv = anrm > 0.f ? 1.0f / (11.313708498984761f * anrm) : 0.f;  // 1 / (sqrt(d) n)
        const int64_t slot = as * stride + ap.pos;
        int code[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float yy = ay[r] * inv;
            code[r] = wid == 0 ? append_code<BK>(yy, kbr, ap.kbound) : append_code<BV>(yy, vbr, ap.vbound);
            ac[r] = h2f(cb16[wid][code[r]]);
            ar[r] = yy - ac[r];
        }
        if (wid == 0) {
            if constexpr (QJL) arn = sqrtf(wave_sum_dpp(ar[0] * ar[0] + ar[1] * ar[1]));
            append_store_codes<BK>(code[0], code[1], lane,
                                   reinterpret_cast<unsigned char*>(ap.kcodes + slot * (BK * D / 32)));
            if (lane == 0) {
                ap.knorm[slot] = f2h(anrm);
                if constexpr (QJL) ap.krnorm[slot] = f2h(arn);
            }
        } else {
            append_store_codes<BV>(code[0], code[1], lane,
                                   reinterpret_cast<unsigned char*>(ap.vcodes + slot * (BV * D / 32)));
            if (lane == 0) ap.vnorm[slot] = f2h(anrm);
        }
    }
    lds_barrier();

    // (3) the score B fragments: element e of k-steps t = 0..3 is one float4 of
    // four consecutive coordinates
#pragma unroll
    for (int part = 0; part < (QJL ? 2 : 1); ++part) {
        const float* src = part ? &ps[QJL ? head : 0][4 * g] : &qs[head][4 * g];
        float4 x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = *reinterpret_cast<const float4*>(src + 16 * e);
        uint32_t w[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w[0][j] = split2(x[2 * j].x, x[2 * j + 1].x);
            w[1][j] = split2(x[2 * j].y, x[2 * j + 1].y);
            w[2][j] = split2(x[2 * j].z, x[2 * j + 1].z);
            w[3][j] = split2(x[2 * j].w, x[2 * j + 1].w);
        }
#pragma unroll
        for (int t = 0; t < KS; ++t) bq[KS * part + t] = __builtin_bit_cast(half8_t, w[t]);
    }

    if (appb) {
        // The new token's sketch and partial. The codebook area is free now; it
        // takes r (keys with the sketch: scaled by 2^10 so its fp16 lo part stays
        // normal, the signs unchanged), the 16 sign bytes, the key's stored norms
        // and its fp16 centroids in the order of the score A operand (coordinate
        // 4 g + t + 16 e at [4 g + t][e]).
        float* rr = reinterpret_cast<float*>(&cb16[0][0]);
        uint32_t* sgw = reinterpret_cast<uint32_t*>(&cb16[0][0]) + D;
        float* nkg = reinterpret_cast<float*>(&cb16[0][0]) + D + 4;
        uint16_t* ckg = &cb16[0][0] + 2 * (D + 8);  // 16-byte aligned
        if (wid == 0) {
            if constexpr (QJL) {
                rr[lane] = ar[0] * 1024.0f;
                rr[lane + 64] = ar[1] * 1024.0f;
                if (lane < 4) sgw[lane] = 0u;
            }
            if (lane == 0) {
                nkg[0] = h2f(f2h(anrm));
                nkg[1] = QJL ? h2f(f2h(arn)) : 0.f;
            }
            ckg[(lane & 15) * 8 + (lane >> 4)] = f2h(ac[0]);
            ckg[(lane & 15) * 8 + 4 + (lane >> 4)] = f2h(ac[1]);
        }
        lds_barrier();
        if constexpr (QJL) {
            // S r against the rows of S this wave holds; row 16 (2 wid + u) + 4 g + r
            // is bit 2 wid + u of sign byte 4 g + r (word g, byte r)
            float4_t pr[2] = {float4_t{0.f, 0.f, 0.f, 0.f}, float4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 x0 = *reinterpret_cast<const float4*>(&rr[32 * k + 8 * g]);
                const float4 x1 = *reinterpret_cast<const float4*>(&rr[32 * k + 8 * g + 4]);
                const uint32_t bw[4] = {split2(x0.x, x0.y), split2(x0.z, x0.w), split2(x1.x, x1.y), split2(x1.z, x1.w)};
                const half8_t b = __builtin_bit_cast(half8_t, bw);
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    pr[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, sA[u][k]), b, pr[u], 0, 0, 0);
            }
            uint32_t bits = 0u;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = pr[u][r] + xor8(pr[u][r]);
                    bits |= (v >= 0.f ? 1u : 0u) << (8 * r + 2 * wid + u);
                }
            if (col == 0) atomicOr(&sgw[g], bits);
            lds_barrier();
            if (wid == 0 && lane == 0)
                *reinterpret_cast<uint4*>(ap.ksigns + (as * stride + ap.pos) * (D / 32)) =
                    make_uint4(sgw[0], sgw[1], sgw[2], sgw[3]);
        }
        // partial of the new token (index n_chunks of the stream): its score for
        // every head from the same score MFMAs as a cached token (row 0 of the A
        // operands, the query fragments bq of this wave), weight sum 1 and
        // accumulator n_v c(v) in the rotated value domain
        float* pn = parts + ((as * pchunks + n_chunks) * G) * part_stride(D);
        if (wid == 3) {
            float4_t sa4 = float4_t{0.f, 0.f, 0.f, 0.f}, sq4 = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                const uint4 av = col == 0 ? *reinterpret_cast<const uint4*>(&ckg[(4 * g + t) * 8]) : make_uint4(0u, 0u, 0u, 0u);
                sa4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), bq[t], sa4, 0, 0, 0);
                if constexpr (QJL) {
                    const uint4 sv = col == 0 ? slut[(sgw[g] >> (8 * t)) & 0xFFu] : make_uint4(0u, 0u, 0u, 0u);
                    sq4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, sv), bq[KS + t], sq4, 0, 0, 0);
                }
            }
            // lanes 0..15 hold row 0: head col & 7's hi (col < 8) and lo parts
            const float a = sa4[0] + xor8(sa4[0]);
            const float fk = nkg[0] * zscale;
            float z = fk * a;
            if constexpr (QJL) z = fmaf(fk * (nkg[1] * kappa), sq4[0] + xor8(sq4[0]), z);
            if (lane < G) *reinterpret_cast<float2*>(pn + lane * part_stride(D)) = make_float2(z, 1.0f);
        } else if (wid == 1) {
            const float nv = h2f(f2h(anrm));
            for (int h = 0; h < G; ++h) {
                pn[h * part_stride(D) + kPartAcc + lane] = nv * ac[0];
                pn[h * part_stride(D) + kPartAcc + lane + 64] = nv * ac[1];
            }
        }
    }

    {
        // fixed weight scale for this wave: max weight * norm stays below 2^15 in fp16.
        // The norms of the wave's range, 512 at a time (the first 512 loaded above).
        float nmax = 0.f;
        if (w1 > w0)
#pragma unroll
            for (int k = 0; k < 8; ++k) nmax = fmaxf(nmax, h2f(hv[k]));
        for (int64_t t0 = w0 + 512; t0 < w1; t0 += 512) {
#pragma unroll
            for (int k = 0; k < 8; ++k) hv[k] = vnorm[base + min(t0 + lane + 64 * k, w1 - 1)];
#pragma unroll
            for (int k = 0; k < 8; ++k) nmax = fmaxf(nmax, h2f(hv[k]));
        }
        nmax = wave_max_dpp(nmax);
        int ex = 0;
        (void)frexpf(nmax, &ex);
        const float wscale = nmax > 0.f ? ldexpf(1.0f, 7 - ex) : 1.0f;

        float M = -INFINITY, lsum = 0.f;
        float4_t acc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};

        // Score MFMAs of one 32-token step (two 16-token tiles): code part am and
        // sign part aq per tile, raw (hi and lo columns not yet added).
        struct Raw {
            float4_t am[2], aq[2];
        };
        auto issue_scores = [&](const Step<BK, BV>& st, Raw& rw) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                rw.am[u] = float4_t{0.f, 0.f, 0.f, 0.f};
                rw.aq[u] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    half8_t a;
                    if constexpr (PK) {
                        // group t: bytes 2 (t & 1) and 2 (t & 1) + 1 of word t >> 1 index two entries
                        const uint32_t w = st.kf[u][t >> 1];
                        const uint2 e0 = *reinterpret_cast<const uint2*>(
                            rowsb + (t & 1 ? row_addr<2>(w, kcopy) : row_addr<0>(w, kcopy)));
                        const uint2 e1 = *reinterpret_cast<const uint2*>(
                            rowsb + (t & 1 ? row_addr<3>(w, kcopy) : row_addr<1>(w, kcopy)));
                        const uint32_t wds[4] = {e0.x, e0.y, e1.x, e1.y};
                        a = __builtin_bit_cast(half8_t, wds);
                    } else {
                        a = key_codes_a<BK>(st.kf[u], t, klut4, klut2);
                    }
                    rw.am[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[t], rw.am[u], 0, 0, 0);
                    if constexpr (QJL) {
                        const uint4 sv = slut[(st.sf[u] >> (8 * t)) & 0xFFu];
                        rw.aq[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, sv), bq[KS + t],
                                                                          rw.aq[u], 0, 0, 0);
                    }
                }
            }
        };
        // The score MFMAs give head col & 7's hi (col < 8) and lo (col >= 8) column
        // parts for both 16-token tiles. Each lane finishes the scores of one tile:
        // the lower half of a 16-lane row tile 0, the upper half tile 1 (own tile
        // `up`), so the softmax and weight work is done once per token and head.
        const bool up = col >= 8;
        // scores in log2 units: zz[r] is token tb + 16 up + 4 g + r for head
        // col & 7 (hi + lo columns added); MASK: -inf past the range
        auto finish_scores = [&](const Step<BK, BV>& st, const Raw& rw, int64_t tb, float (&zz)[4], auto MASK) {
            // per-token factors of the lane's quad (all four lanes of a quad lie in
            // one half): row 16 up + 4 g + r sits in quad lane r
            const float fk = h2f(up ? st.nk[1] : st.nk[0]) * zscale;
            const float fq = fk * (h2f(up ? st.ng[1] : st.ng[0]) * kappa);
            static_for<0, 4>([&](auto rr) {
                constexpr int r = decltype(rr)::value;
                const float a0 = rw.am[0][r] + xor8(rw.am[0][r]), a1 = rw.am[1][r] + xor8(rw.am[1][r]);
                float z = quad_bcast<r>(fk) * (up ? a1 : a0);
                if constexpr (QJL) {
                    const float q0 = rw.aq[0][r] + xor8(rw.aq[0][r]), q1 = rw.aq[1][r] + xor8(rw.aq[1][r]);
                    z = fmaf(quad_bcast<r>(fq), up ? q1 : q0, z);
                }
                if constexpr (decltype(MASK)::value) zz[r] = (tb + (up ? 16 : 0) + 4 * g + r < w1) ? z : -INFINITY;
                else zz[r] = z;
            });
        };
        // the block max per head column (the other tile's lane, then permlane swaps
        // across the row groups); rescale the running sums only when it beats the
        // running max by 2^8
        auto softmax_check = [&](const float (&zz)[4]) {
            float bm = max3f(zz[0], zz[1], max2nn(zz[2], zz[3]));
            bm = max2nn(bm, xor8(bm));
            bm = rows_max(bm);
            if (__builtin_expect(__ballot(bm > M + 8.0f) != 0, 0)) {
                const float nM = max2nn(M, bm);
                const float f = __builtin_amdgcn_exp2f(M - nM);
                lsum *= f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float fr = __shfl(f, (4 * g + r) & 7);
#pragma unroll
                    for (int c = 0; c < CT; ++c) acc[c][r] *= fr;
                }
                M = nM;
            }
        };
        // weights of one step (A operand: row = head column, K slot = token) times
        // its value centroids, accumulated in the rotated value domain
        auto accumulate = [&](const Step<BK, BV>& st, const float (&zz)[4]) {
            const float fv = h2f(up ? st.nv[1] : st.nv[0]) * wscale;
            float Wo[4];  // own tile's weights times value norms
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float w = __builtin_amdgcn_exp2f(zz[r] - M);
                lsum += w;
                Wo[r] = w;
            }
            Wo[0] *= quad_bcast<0>(fv);
            Wo[1] *= quad_bcast<1>(fv);
            Wo[2] *= quad_bcast<2>(fv);
            Wo[3] *= quad_bcast<3>(fv);
            // K slot 4 u + r is token 16 u + 4 g + r: tile 0's weights from the lower
            // lane of the pair, tile 1's from the upper one
            float W8[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                W8[r] = take_xor8<0xC>(Wo[r]);
                W8[4 + r] = take_xor8<0x3>(Wo[r]);
            }
            // head rows take fp16(W), remainder rows fp16(W - fp16(W))
            uint32_t awd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) awd[j] = split2(W8[2 * j], W8[2 * j + 1]);
            const half8_t aw = __builtin_bit_cast(half8_t, awd);

            // ---- value codes: lane column = code group, slot e = token 4g+e (tile 0) / 16+4g+e-4 (tile 1)
            uint32_t X[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (BV == 3) X[e] = __builtin_amdgcn_alignbit(st.x1[e], st.x0[e], (24 * col) & 31) & 0xFFFFFFu;
                else if constexpr (BV == 4 || BV == 8) X[e] = st.x0[e];
                else X[e] = (st.x0[e] >> ((8 * BV * col) & 31)) & ((1u << (8 * BV)) - 1u);
            }
            if constexpr (BV == 8) {
                // one byte per code: member c of the group is byte c of (x1:x0); single-code
                // table entries carry the centroid in both halves, so a bit-field insert
                // pairs two tokens
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    uint32_t bw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t wa = c < 4 ? X[2 * j] : st.x1[2 * j];
                        const uint32_t wb = c < 4 ? X[2 * j + 1] : st.x1[2 * j + 1];
                        const uint32_t a = vl((wa >> (8 * (c & 3))) & 0xFFu);
                        const uint32_t b = vl((wb >> (8 * (c & 3))) & 0xFFu);
                        bw[j] = (a & 0xFFFFu) | (b & 0xFFFF0000u);
                    }
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, bw), acc[c], 0, 0, 0);
                }
            } else if constexpr (BV == 3) {
                // tiles 2 cp and 2 cp + 1 from one lookup: codes 2 cp, 2 cp + 1 of each token
                // of pair j are bits 6 cp .. 6 cp + 5 of its field
#pragma unroll
                for (int cp = 0; cp < CT / 2; ++cp) {
                    uint32_t be[4], bo[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t aa = (X[2 * j] >> (6 * cp)) & 63u, bb = (X[2 * j + 1] >> (6 * cp)) & 63u;
                        const uint32_t ix = aa | (bb << 6);
                        be[j] = vlut12[ix];
                        bo[j] = vlut12[kV12Odd + ix];
                    }
                    acc[2 * cp] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, be), acc[2 * cp], 0, 0, 0);
                    acc[2 * cp + 1] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, bo), acc[2 * cp + 1], 0, 0, 0);
                }
            } else {
                // interleave the two tokens' fields: slot k of y0 (2*BV bits) is the index for
                // tile 2k, slot k of y1 the index for tile 2k+1
                constexpr uint32_t MSK = BV == 4 ? 0x0F0F0F0Fu : (BV == 2 ? 0x33333333u : 0x55555555u);
                uint32_t y0[4], y1[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t xa = X[2 * j], xb = X[2 * j + 1];
                    y0[j] = (xa & MSK) | ((xb << BV) & ~MSK);
                    y1[j] = ((xa >> BV) & MSK) | (xb & ~MSK);
                }
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    uint32_t bw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t y = (c & 1) ? y1[j] : y0[j];
                        if constexpr (PV) {
                            // 4-bit codes: the index of tile c is byte c >> 1 of y
                            uint32_t ad;
                            switch (c >> 1) {
                                case 0: ad = row_addr<0>(y, vcopy); break;
                                case 1: ad = row_addr<1>(y, vcopy); break;
                                case 2: ad = row_addr<2>(y, vcopy); break;
                                default: ad = row_addr<3>(y, vcopy); break;
                            }
                            bw[j] = *reinterpret_cast<const uint32_t*>(rowsb + ad);
                        } else {
                            bw[j] = vl((y >> (2 * BV * (c >> 1))) & ((1u << (2 * BV)) - 1u));
                        }
                    }
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, bw), acc[c], 0, 0, 0);
                }
            }
        };
        using Full = std::integral_constant<bool, false>;
        using Tail = std::integral_constant<bool, true>;

        // Full steps, software-pipelined: the next step's key lookups and score
        // MFMAs are issued before the current step's softmax check (whose rare
        // rescale is a branch), so they run under the current step's weight and
        // value work; loads run a step ahead of the scores. sa / sb alternate.
        float za[4], zb[4];
        Raw rw;
        int64_t i = 0;
        if (nfull > 0) {
            issue_scores(sa, rw);
            finish_scores(sa, rw, w0, za, Full{});
            // steady state: steps i (sa, za) and i + 1 (sb); steps i + 2 and i + 3 exist
            for (; i + 3 < nfull; i += 2) {
                const int64_t tb = w0 + 32 * i;
                progress_prio(i, nfull);
                issue_scores(sb, rw);
                softmax_check(za);
                accumulate(sa, za);
                finish_scores(sb, rw, tb + 32, zb, Full{});
                load_full<D, BK, QJL, BV>(sa, base + tb + 64, loff, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
                issue_scores(sa, rw);
                softmax_check(zb);
                accumulate(sb, zb);
                finish_scores(sa, rw, tb + 64, za, Full{});
                load_full<D, BK, QJL, BV>(sb, base + tb + 96, loff, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
            }
            // the last one to three full steps: i (sa, za), i + 1 (sb), i + 2 (into sa)
            const int64_t rem = nfull - i, tb = w0 + 32 * i;
            if (rem >= 2) issue_scores(sb, rw);
            softmax_check(za);
            accumulate(sa, za);
            if (rem >= 2) {
                finish_scores(sb, rw, tb + 32, zb, Full{});
                if (rem >= 3) {
                    load_full<D, BK, QJL, BV>(sa, base + tb + 64, loff, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
                    issue_scores(sa, rw);
                }
                softmax_check(zb);
                accumulate(sb, zb);
                if (rem >= 3) {
                    finish_scores(sa, rw, tb + 64, za, Full{});
                    softmax_check(za);
                    accumulate(sa, za);
                }
            }
        }
        // at most one partial step: clamped loads, masked scores
        const int64_t tt = w0 + 32 * nfull;
        if (tt < w1) {
            load_step<D, BK, QJL, BV>(sa, tt, w1, base, lane, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
            issue_scores(sa, rw);
            finish_scores(sa, rw, tt, za, Tail{});
            softmax_check(za);
            accumulate(sa, za);
        }

        __builtin_amdgcn_s_setprio(0);
        // ---- per-wave results: sum over the tile pair and the row groups, hi rows +
        // lo rows (permlane swaps)
        lsum += xor8(lsum);
        if constexpr (ROWS || V12) lds_barrier();  // every wave is done with the tables the merge buffers overwrite
        {
            float e_, o_;
            row_pair<16>(lsum, e_, o_);
            lsum = e_ + o_;
            row_pair<32>(lsum, e_, o_);
            lsum = e_ + o_;
        }
        const float inv = 1.0f / wscale;
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float e_, o_;
                row_pair<32>(acc[c][r], e_, o_);  // rows 4 g + r of the upper half are the lo rows
                const int h = 4 * g + r;
                if (g < 2 && h < G) mrg_o[wid][h][col + 16 * c] = (e_ + o_) * inv;
            }
        if (lane < 8) {
            mrg_m[wid][lane] = M;
            mrg_l[wid][lane] = lsum;
        }
        float* part0 = parts + ((s * pchunks + chunk) * G) * part_stride(D);
        lds_barrier();

        // ---- merge the four waves into one partial per head: the 32 factors
        // exp2(m_w - max) once, then float4 rows
        constexpr int PS = part_stride(D);
        if (tid < 32) {
            const int w = tid >> 3, h = tid & 7;
            float mx = -INFINITY;
#pragma unroll
            for (int v = 0; v < 4; ++v) mx = fmaxf(mx, mrg_m[v][h]);
            mrg_f[w][h] = (mx == -INFINITY || mrg_m[w][h] == -INFINITY) ? 0.f : exp2f(mrg_m[w][h] - mx);
            if (w == 0) mrg_x[h] = mx;
        }
        lds_barrier();
        for (int e = tid; e < G * (D / 4); e += 256) {
            const int h = e / (D / 4), i4 = e % (D / 4);
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = mrg_f[w][h];
                const float4 v = *reinterpret_cast<const float4*>(&mrg_o[w][h][4 * i4]);
                o.x += f * v.x;
                o.y += f * v.y;
                o.z += f * v.z;
                o.w += f * v.w;
            }
            *reinterpret_cast<float4*>(part0 + h * PS + kPartAcc + 4 * i4) = o;
            if (i4 == 0) {
                float l = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) l += mrg_f[w][h] * mrg_l[w][h];
                *reinterpret_cast<float2*>(part0 + h * PS) = make_float2(mrg_x[h], l);
            }
        }
    }
}

// Query rows as the kernel takes them: pointer and fp16 flag.
struct QueryIn {
    const void* q;
    int f16;
};

template <int D, int BK, bool QJL, int BV>
void launch_mfma(const tq_packed* k, const tq_packed* v, int64_t n_streams, int64_t T, int64_t stride, int G,
                 QueryIn fr, const tq_quantizer* qk, const tq_quantizer* qv, float zscale,
                 float* parts, int n_chunks, int pchunks, int tc, const AppendIn& ap, hipStream_t s)
{
    const int64_t n_items = n_streams * n_chunks;
    hipLaunchKernelGGL((k_decode_mfma<D, BK, QJL, BV>), dim3((unsigned)n_items), dim3(256), 0, s, k->codes, k->signs, k->norm,
                       k->rnorm, v->codes, v->norm, T, stride, G, fr.q, fr.f16, qk->diag_signs, qk->S,
                       qk->centroids, qv->centroids, zscale, parts, n_chunks, pchunks, tc, ap);
}

template <int D, int BK, bool QJL>
void launch_bv(int bv, const tq_packed* k, const tq_packed* v, int64_t ns, int64_t T, int64_t stride, int G,
               QueryIn fr,
               const tq_quantizer* qk, const tq_quantizer* qv, float zs, float* parts, int nc, int pc, int tc,
               const AppendIn& ap, hipStream_t s)
{
    // value widths 1..4 with keys of 1..4 bits, 3, 4 and 8 with any key width
    switch (bv) {
        case 1: if constexpr (BK <= 4) launch_mfma<D, BK, QJL, 1>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, pc, tc, ap, s); break;
        case 2: if constexpr (BK <= 4) launch_mfma<D, BK, QJL, 2>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, pc, tc, ap, s); break;
        case 3: launch_mfma<D, BK, QJL, 3>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, pc, tc, ap, s); break;
        case 4: launch_mfma<D, BK, QJL, 4>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, pc, tc, ap, s); break;
        default: launch_mfma<D, BK, QJL, 8>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, pc, tc, ap, s); break;
    }
}

// Score fragments of `tiles` groups of G query rows (rows at or past `total`
// count as zero).
void launch_qprep_frag(const tq_quantizer* qk, const void* q, int q_dtype, int64_t tiles, int G, int64_t total,
                       half8_t* frags, hipStream_t s)
{
    constexpr int D = 128;
    const bool qjl = qk->qjl_m != 0;
    const dim3 pg((unsigned)tiles, (unsigned)(D / 32)), pb(256);
    if (q_dtype == TQ_F16) {
        if (qjl) hipLaunchKernelGGL((k_qprep_frag<D, true, true>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags);
        else hipLaunchKernelGGL((k_qprep_frag<D, false, true>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags);
    } else {
        if (qjl) hipLaunchKernelGGL((k_qprep_frag<D, true, false>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags);
        else hipLaunchKernelGGL((k_qprep_frag<D, false, false>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags);
    }
}

// Estimated inner products (the score formula of "[Benchmark] TurboQuant
// 實測：KV Cache 3-bit 壓縮，真的零損失？", section "TurboQuant 是什麼：30 秒懶人包")
// for d = 128 on MFMA, with the same exact operands as the decode step: a
// 16-key tile (rows) against tiles of 8 queries whose fp32 rotated values and
// projections are split into fp16 hi and lo columns. A wave holds the
// fragments of kScoreQT query tiles and walks 16-key tiles, building each
// tile's key operands once for all of them and fetching the next tile's
// packed keys while it works. Grid (key-tile groups, query-tile groups);
// scores[q][key], fp32.
constexpr int kScoreQT = 4;

template <int D, int BK, bool QJL>
__global__ __launch_bounds__(256, 2) void k_scores_mfma(const uint32_t* __restrict__ kcodes,
                                                        const uint32_t* __restrict__ ksigns,
                                                        const uint16_t* __restrict__ knorm,
                                                        const uint16_t* __restrict__ krnorm, int64_t N,
                                                        const half8_t* __restrict__ frags, int64_t n_q,
                                                        const float* __restrict__ kcent,
                                                        float* __restrict__ scores)
{
    static_assert(D == 128, "MFMA scores are laid out for d = 128");
    constexpr int KS = D / 32, KSTEPS = KS * (QJL ? 2 : 1);
    constexpr int KW = BK * D / 32, SWN = D / 32;
    constexpr bool K4 = BK <= 2;
    constexpr int KLUT = key_lut_entries(BK);
    constexpr float kappa = 1.2533141373155003f / D;  // sqrt(pi/2) / m
    __shared__ uint2 klut4[K4 ? KLUT : 1];
    __shared__ uint32_t klut2[K4 ? 1 : KLUT];
    __shared__ uint4 slut[QJL ? 256 : 1];
    fill_key_luts<BK, QJL>(klut4, klut2, slut, kcent);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int64_t n_qt = (n_q + 7) / 8, n_qg = (n_qt + kScoreQT - 1) / kScoreQT, n_kt = (N + 15) / 16;
    // packed inputs of one key tile for this lane: A row k0 + col, norms of rows
    // k0 + 4 g + r. A tile inside the key range is read from a wave-uniform tile
    // base plus fixed 32-bit lane offsets; only the last, partial tile clamps.
    struct KT {
        uint32_t kf[BK];
        uint32_t sf;
        uint16_t nk[4], ng[4];
    };
    const int ko = col * KW + BK * g, so = col * SWN + g, no = 4 * g;
    auto load_kt = [&](KT& t, int64_t k0) {
        if (k0 + 16 <= N) {
            const uint32_t* kc = kcodes + k0 * KW;
#pragma unroll
            for (int w = 0; w < BK; ++w) t.kf[w] = kc[ko + w];
            t.sf = QJL ? ksigns[k0 * SWN + so] : 0u;
            const uint16_t* kn = knorm + k0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                t.nk[r] = kn[no + r];
                t.ng[r] = QJL ? krnorm[k0 + no + r] : (uint16_t)0;
            }
        } else {
            const int64_t ka = min(k0 + col, N - 1);
#pragma unroll
            for (int w = 0; w < BK; ++w) t.kf[w] = kcodes[ka * KW + BK * g + w];
            t.sf = QJL ? ksigns[ka * SWN + g] : 0u;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t kr = min(k0 + 4 * g + r, N - 1);
                t.nk[r] = knorm[kr];
                t.ng[r] = QJL ? krnorm[kr] : (uint16_t)0;
            }
        }
    };
    // the wave takes key tiles in adjacent pairs (2 pr, 2 pr + 1), so the two
    // 64-byte halves of each 128-byte line of a score row are written back to back
    const int64_t pstep = (int64_t)gridDim.x * 4;
    auto next_kt = [&](int64_t kt) { return (kt & 1) ? kt - 1 + 2 * pstep : kt + 1; };
    const bool vec4 = (N & 3) == 0;
    const int64_t lrow = (int64_t)(col & 7) * N + 4 * g;  // this lane's offset in a query tile's rows
    for (int64_t qg = blockIdx.y; qg < n_qg; qg += gridDim.y) {
        half8_t bq[kScoreQT][KSTEPS];
#pragma unroll
        for (int j = 0; j < kScoreQT; ++j) {
            const int64_t qt = min(qg * kScoreQT + j, n_qt - 1);  // past the end: repeat, not stored
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) bq[j][k] = frags[(qt * KSTEPS + k) * 64 + lane];
        }
        // the scores of one key tile against every query tile of the group
        auto tile = [&](const KT& cur, int64_t k0) {
            half8_t ac[KS], as[QJL ? KS : 1];
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                ac[t] = key_codes_a<BK>(cur.kf, t, klut4, klut2);
                if constexpr (QJL) as[t] = __builtin_bit_cast(half8_t, slut[(cur.sf >> (8 * t)) & 0xFFu]);
            }
            float fk[4], fq[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                fk[r] = h2f(cur.nk[r]);
                fq[r] = QJL ? fk[r] * h2f(cur.ng[r]) * kappa : 0.f;
            }
            const bool full = vec4 && k0 + 16 <= N;  // wave-uniform
#pragma unroll
            for (int j = 0; j < kScoreQT; ++j) {
                float4_t am = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    am = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[t], bq[j][t], am, 0, 0, 0);
                    if constexpr (QJL) aq = __builtin_amdgcn_mfma_f32_16x16x32_f16(as[t], bq[j][KS + t], aq, 0, 0, 0);
                }
                // hi + lo columns, then row (key) 4 g + r of query column col & 7
                float z[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    z[r] = fk[r] * (am[r] + ror8(am[r]));
                    if constexpr (QJL) z[r] = fmaf(fq[r], aq[r] + ror8(aq[r]), z[r]);
                }
                // query row (qg kScoreQT + j) 8 + col (lanes col < 8): a wave-uniform
                // tile base plus this lane's fixed offset
                const int64_t q0 = (qg * kScoreQT + j) * 8;
                if (col < 8 && q0 + col < n_q) {
                    float* dst = scores + q0 * N + lrow + k0;
                    if (full) {
                        // write-once output: streamed past the caches
                        __builtin_nontemporal_store(float4_t{z[0], z[1], z[2], z[3]}, reinterpret_cast<float4_t*>(dst));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (k0 + 4 * g + r < N) dst[r] = z[r];
                    }
                }
            }
        };
        // the next tile's loads go out before this one's work
        int64_t kt = 2 * ((int64_t)blockIdx.x * 4 + wid);
        KT cur;
        if (kt < n_kt) load_kt(cur, kt * 16);
        for (; kt < n_kt; kt = next_kt(kt)) {
            KT nxt;
            if (next_kt(kt) < n_kt) load_kt(nxt, next_kt(kt) * 16);
            tile(cur, kt * 16);
            cur = nxt;
        }
    }
}

template <int D, int BK, bool QJL>
void launch_scores_k(const tq_packed* k, int64_t n_keys, const half8_t* fr, int64_t n_q, const tq_quantizer* q,
                     float* scores, hipStream_t s)
{
    auto kern = k_scores_mfma<D, BK, QJL>;
    const int64_t n_kt = (n_keys + 15) / 16, n_qg = ((n_q + 7) / 8 + kScoreQT - 1) / kScoreQT;
    // about two resident 4-wave blocks per compute unit in all
    int64_t gx = (n_kt + 7) / 8;
    const int64_t want = (int64_t)device_cus() * 2;
    const int64_t per_q = (want + n_qg - 1) / n_qg;
    if (gx > per_q) gx = per_q < 1 ? 1 : per_q;
    const dim3 grid((unsigned)gx, (unsigned)(n_qg < 65535 ? n_qg : 65535));
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, k->codes, k->signs, k->norm, k->rnorm, n_keys, fr, n_q,
                       q->centroids, scores);
}

}  // namespace

int launch_decode_mfma(const tq_quantizer* qk, const tq_quantizer* qv, const tq_packed* k,
                       const tq_packed* v, int64_t n_streams, int64_t T, int64_t stride, int G, const void* q,
                       int q_dtype, float zscale, float* parts, int n_chunks, int pchunks, int tc,
                       const AppendIn& ap, hipStream_t s)
{
    constexpr int D = 128;
    const bool qjl = qk->qjl_m != 0;
    if (n_streams * n_chunks >= (int64_t)1 << 31)
        return fail(TQ_ERR_UNSUPPORTED, "tq_decode_attn: %lld streams x %d chunks is more work items than 2^31",
                    (long long)n_streams, n_chunks);
    const QueryIn fr{q, q_dtype == TQ_F16 ? 1 : 0};
    switch (qk->mse_bits) {
        case 1: qjl ? launch_bv<D, 1, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                    : launch_bv<D, 1, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
        case 2: qjl ? launch_bv<D, 2, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                    : launch_bv<D, 2, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
        case 3: qjl ? launch_bv<D, 3, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                    : launch_bv<D, 3, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
        case 4: qjl ? launch_bv<D, 4, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                    : launch_bv<D, 4, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
        case 5: qjl ? launch_bv<D, 5, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                    : launch_bv<D, 5, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
        case 6: qjl ? launch_bv<D, 6, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                    : launch_bv<D, 6, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
        case 7: qjl ? launch_bv<D, 7, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                    : launch_bv<D, 7, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
        default: qjl ? launch_bv<D, 8, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s)
                     : launch_bv<D, 8, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, pchunks, tc, ap, s); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "tq_decode_attn: %s", hipGetErrorString(e));
    return TQ_OK;
}

int launch_scores_mfma(const tq_quantizer* q, const tq_packed* k, int64_t n_keys, const void* queries,
                       int q_dtype, int64_t n_q, float* scores, void* frags, hipStream_t s)
{
    constexpr int D = 128;
    const int64_t n_qt = (n_q + 7) / 8;
    launch_qprep_frag(q, queries, q_dtype, n_qt, 8, n_q, (half8_t*)frags, s);
    const half8_t* fr = (const half8_t*)frags;
    const bool qjl = q->qjl_m != 0;
    switch (q->mse_bits) {
        case 1: qjl ? launch_scores_k<D, 1, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 1, false>(k, n_keys, fr, n_q, q, scores, s); break;
        case 2: qjl ? launch_scores_k<D, 2, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 2, false>(k, n_keys, fr, n_q, q, scores, s); break;
        case 3: qjl ? launch_scores_k<D, 3, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 3, false>(k, n_keys, fr, n_q, q, scores, s); break;
        case 4: qjl ? launch_scores_k<D, 4, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 4, false>(k, n_keys, fr, n_q, q, scores, s); break;
        case 5: qjl ? launch_scores_k<D, 5, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 5, false>(k, n_keys, fr, n_q, q, scores, s); break;
        case 6: qjl ? launch_scores_k<D, 6, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 6, false>(k, n_keys, fr, n_q, q, scores, s); break;
        case 7: qjl ? launch_scores_k<D, 7, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 7, false>(k, n_keys, fr, n_q, q, scores, s); break;
        default: qjl ? launch_scores_k<D, 8, true>(k, n_keys, fr, n_q, q, scores, s) : launch_scores_k<D, 8, false>(k, n_keys, fr, n_q, q, scores, s); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "tq_scores: %s", hipGetErrorString(e));
    return TQ_OK;
}

}  // namespace tq
