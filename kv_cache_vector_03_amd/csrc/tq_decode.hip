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
// Work split: a block owns a chunk of one stream's tokens, each of its four
// waves a contiguous quarter, processed 32 tokens at a time:
//   scores  16 tokens x 16 columns (8 heads x hi/lo) per MFMA tile, K = 256
//           (128 code slots + 128 sign slots, in group-major order);
//   softmax exact max per 32-token block; the running max moves (and the
//           accumulators are rescaled) only when a block beats it by 2^8;
//   values  16 rows (8 heads x hi/lo) x 16 coordinates per tile, K = 32 tokens.
// The four waves merge in LDS; one partial (max, sum, rotated-domain
// accumulator) per block goes to the workspace, and the combine kernel merges
// the partials of a stream and undoes the value rotation.
#include "tq_append.h"
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

__device__ __forceinline__ float xor8(float x)
{
    // lane i <-> lane i ^ 8 inside each row of 16 lanes (DPP row rotate by 8)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
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
//
// With the decode step's append, grid.y has two more blocks per stream: they
// quantize the stream's new key (y = d/32) and value (y = d/32 + 1) into the
// caches, beside the fragment blocks and in the same launch.
struct AppendDev {
    tq_quantizer qk, qv;
    tq_packed k, v;
    const void* k_new;
    const void* v_new;
    int dtype;
    int64_t stride, pos;
};

template <int D, bool QJL, bool F16>
__global__ __launch_bounds__(256) void k_qprep_frag(const void* __restrict__ q, int G, int64_t total,
                                                    const uint32_t* __restrict__ diag,
                                                    const uint16_t* __restrict__ S,
                                                    half8_t* __restrict__ frags, AppendDev app)
{
    static_assert(D == 128, "fragment layout is laid out for d = 128");
    static_assert(8 * D >= append_smem_floats(D), "append scratch reuses the query buffer");
    constexpr int R = D / 64, KS = D / 32, KSTEPS = KS * (QJL ? 2 : 1);
    __shared__ float qs[8][D];
    __shared__ float ps[QJL ? 8 : 1][32];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t s = blockIdx.x;
    const int tt = blockIdx.y;
    if (tt >= KS) {
        const bool val = tt == KS + 1;
        quantize_one<D>(val ? app.qv : app.qk, val ? app.v : app.k, val ? app.v_new : app.k_new, app.dtype, s,
                        s * app.stride + app.pos, &qs[0][0]);
        return;
    }
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
        fwht_wave<R>(ya, lane);
        fwht_wave<R>(yb, lane);
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

template <int D, int BK, bool QJL, int BV>
__global__ __launch_bounds__(256, 2) void k_decode_mfma(const uint32_t* __restrict__ kcodes,
                                                     const uint32_t* __restrict__ ksigns,
                                                     const uint16_t* __restrict__ knorm,
                                                     const uint16_t* __restrict__ krnorm,
                                                     const uint32_t* __restrict__ vcodes,
                                                     const uint16_t* __restrict__ vnorm, int64_t T,
                                                     int64_t stride, int G, const half8_t* __restrict__ frags,
                                                     const float* __restrict__ kcent,
                                                     const float* __restrict__ vcent, float zscale,
                                                     float* __restrict__ parts, int n_chunks, int tc,
                                                     int64_t n_items)
{
    static_assert(D == 128, "MFMA decode is laid out for d = 128");
    constexpr int KS = D / 32;                 // 4 code groups per lane per token
    constexpr int KSTEPS = KS * (QJL ? 2 : 1);
    constexpr int CT = D / 16;                 // value coordinate tiles
    constexpr bool K4 = BK <= 2;               // one key table entry = 4 codes (else 2, or 1 above 4 bits)
    constexpr int KLUT = key_lut_entries(BK);
    constexpr int VLUT = BV <= 4 ? 1 << (2 * BV) : 1 << BV;  // code pairs, or single codes above 4 bits
    constexpr float kappa = 1.2533141373155003f / D;  // sqrt(pi/2) / m

    __shared__ uint2 klut4[K4 ? KLUT : 1];
    __shared__ uint32_t klut2[K4 ? 1 : KLUT];
    __shared__ uint4 slut[QJL ? 256 : 1];
    __shared__ uint32_t vlut[VLUT][32];  // one copy per bank: lane l reads copy l % 32
    __shared__ float mrg_m[4][8], mrg_l[4][8];
    __shared__ float mrg_o[4][8][D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int col = lane & 15, g = lane >> 4;
    const LaneOff loff = lane_offsets<D, BK, BV>(lane);

    // ---- lookup tables: codes -> fp16 centroids, sign bytes -> +-1 (built once per block)
    fill_key_luts<BK, QJL>(klut4, klut2, slut, kcent);
    for (int i = tid; i < VLUT * 32; i += 256) {
        const int e = i >> 5;
        if constexpr (BV <= 4)
            vlut[e][i & 31] = (uint32_t)f2h(vcent[e & ((1 << BV) - 1)]) | ((uint32_t)f2h(vcent[e >> BV]) << 16);
        else
            vlut[e][i & 31] = (uint32_t)f2h(vcent[e]) * 0x10001u;  // one code, its centroid in both halves
    }
    __syncthreads();

    for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int64_t s = item / n_chunks;
        const int chunk = (int)(item % n_chunks);
        const int64_t base = s * stride;
        const int64_t c0 = (int64_t)chunk * tc;
        const int64_t c1 = c0 + tc < T ? c0 + tc : T;
        const int64_t w0 = c0 + (int64_t)wid * (tc / 4);
        const int64_t w1 = w0 + tc / 4 < c1 ? w0 + tc / 4 : c1;

        // the first full step's loads go out first, so that they are in flight
        // while the query fragments and the norms of the range arrive
        const int64_t nfull = w1 > w0 ? (w1 - w0) >> 5 : 0;  // a wave past the chunk's end has none
        Step<BK, BV> sa, sb;
        if (nfull > 0) load_full<D, BK, QJL, BV>(sa, base + w0, loff, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);

        half8_t bq[KSTEPS];
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) bq[k] = frags[(s * KSTEPS + k) * 64 + lane];

        // fixed weight scale for this wave: max weight * norm stays below 2^15 in fp16.
        // The norms of the wave's range are read 512 at a time with all loads in
        // flight together (indices clamped into the range, as for the steps).
        float nmax = 0.f;
        for (int64_t t0 = w0; t0 < w1; t0 += 512) {
            uint16_t hv[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) hv[k] = vnorm[base + min(t0 + lane + 64 * k, w1 - 1)];
#pragma unroll
            for (int k = 0; k < 8; ++k) nmax = fmaxf(nmax, h2f(hv[k]));
        }
        nmax = wave_max(nmax);
        int ex = 0;
        (void)frexpf(nmax, &ex);
        const float wscale = nmax > 0.f ? ldexpf(1.0f, 7 - ex) : 1.0f;

        float M = -INFINITY, lsum = 0.f;
        float4_t acc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};

        // one 32-token step from tb; MASK: the step runs past the wave's range
        auto compute = [&](const Step<BK, BV>& st, int64_t tb, auto MASK) {
            // per-token factors of this lane's quad: row 16 u + 4 g + r sits in quad lane r
            float fk[2], fq[2], fv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                fk[u] = h2f(st.nk[u]) * zscale;
                fq[u] = fk[u] * (h2f(st.ng[u]) * kappa);
                fv[u] = h2f(st.nv[u]) * wscale;
            }

            // ---- scores for two 16-token tiles
            float zz[8];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float4_t am = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    const half8_t a = key_codes_a<BK>(st.kf[u], t, klut4, klut2);
                    am = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[t], am, 0, 0, 0);
                    if constexpr (QJL) {
                        const uint4 sv = slut[(st.sf[u] >> (8 * t)) & 0xFFu];
                        aq = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, sv), bq[KS + t], aq,
                                                                    0, 0, 0);
                    }
                }
                static_for<0, 4>([&](auto rr) {
                    constexpr int r = decltype(rr)::value;
                    const int row = 16 * u + 4 * g + r;
                    const float zm = am[r] + xor8(am[r]);
                    float z = quad_bcast<r>(fk[u]) * zm;
                    if constexpr (QJL) z = fmaf(quad_bcast<r>(fq[u]), aq[r] + xor8(aq[r]), z);
                    if constexpr (decltype(MASK)::value) zz[4 * u + r] = (tb + row < w1) ? z : -INFINITY;
                    else zz[4 * u + r] = z;
                });
            }

            // ---- block max per head column; rescale only when it beats the running max by 2^8
            float bm = zz[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) bm = fmaxf(bm, zz[e]);
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            if (__ballot(bm > M + 8.0f)) {
                const float nM = fmaxf(M, bm);
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

            // ---- weights as the A operand (row = head column, K slot = token)
            uint32_t awd[4];
            static_for<0, 4>([&](auto jj) {
                constexpr int j = decltype(jj)::value;
                float W[2];
                static_for<0, 2>([&](auto hh) {
                    constexpr int e = 2 * j + decltype(hh)::value;
                    const float w = __builtin_amdgcn_exp2f(zz[e] - M);
                    lsum += w;
                    W[decltype(hh)::value] = w * quad_bcast<e & 3>(fv[e >> 2]);
                });
                // fp16(W) for head rows, fp16(W - fp16(W)) for remainder rows
                const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)W[0]);
                const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)W[1]);
                uint32_t lw = 0;
                asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "+v"(lw) : "v"(h0), "v"(W[0]));
                asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "+v"(lw) : "v"(h1), "v"(W[1]));
                awd[j] = col < 8 ? (h0 | (h1 << 16)) : lw;
            });
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
                        const uint32_t a = vlut[(wa >> (8 * (c & 3))) & 0xFFu][lane & 31];
                        const uint32_t b = vlut[(wb >> (8 * (c & 3))) & 0xFFu][lane & 31];
                        bw[j] = (a & 0xFFFFu) | (b & 0xFFFF0000u);
                    }
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, bw), acc[c], 0, 0, 0);
                }
            } else if constexpr (BV == 3) {
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    uint32_t bw[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t ia = (X[2 * j] >> (3 * c)) & 7u, ib = (X[2 * j + 1] >> (3 * c)) & 7u;
                        bw[j] = vlut[ia | (ib << 3)][lane & 31];
                    }
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, bw), acc[c], 0, 0, 0);
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
                        bw[j] = vlut[(y >> (2 * BV * (c >> 1))) & ((1u << (2 * BV)) - 1u)][lane & 31];
                    }
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw, __builtin_bit_cast(half8_t, bw), acc[c], 0, 0, 0);
                }
            }
        };
        // full steps (no masking, uniform-base loads, next step in flight),
        // then at most one partial step with clamped loads and masked scores
        using Full = std::integral_constant<bool, false>;
        using Tail = std::integral_constant<bool, true>;
        int64_t i = 0;
        for (; i + 2 <= nfull; i += 2) {
            const int64_t tb = w0 + 32 * i;
            load_full<D, BK, QJL, BV>(sb, base + tb + 32, loff, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
            compute(sa, tb, Full{});
            if (i + 2 < nfull)
                load_full<D, BK, QJL, BV>(sa, base + tb + 64, loff, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
            compute(sb, tb + 32, Full{});
        }
        if (i < nfull) compute(sa, w0 + 32 * i, Full{});
        const int64_t tt = w0 + 32 * nfull;
        if (tt < w1) {
            load_step<D, BK, QJL, BV>(sa, tt, w1, base, lane, kcodes, ksigns, knorm, krnorm, vcodes, vnorm);
            compute(sa, tt, Tail{});
        }

        // ---- per-wave results: sum over row groups, hi rows + lo rows
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        const float inv = 1.0f / wscale;
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float o = acc[c][r] + __shfl_xor(acc[c][r], 32);
                const int h = 4 * g + r;
                if (g < 2 && h < G) mrg_o[wid][h][col + 16 * c] = o * inv;
            }
        if (lane < 8) {
            mrg_m[wid][lane] = M;
            mrg_l[wid][lane] = lsum;
        }
        __syncthreads();

        // ---- merge the four waves into one partial per head
        constexpr int PS = part_stride(D);
        float* part0 = parts + ((s * n_chunks + chunk) * G) * PS;
        for (int e = tid; e < G * D; e += 256) {
            const int h = e / D, i = e % D;
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) mx = fmaxf(mx, mrg_m[w][h]);
            float o = 0.f;
            if (mx != -INFINITY)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    if (mrg_m[w][h] != -INFINITY) o += exp2f(mrg_m[w][h] - mx) * mrg_o[w][h][i];
            part0[h * PS + kPartAcc + i] = o;
            if (i == 0) {
                float l = 0.f;
                if (mx != -INFINITY)
#pragma unroll
                    for (int w = 0; w < 4; ++w)
                        if (mrg_m[w][h] != -INFINITY) l += exp2f(mrg_m[w][h] - mx) * mrg_l[w][h];
                part0[h * PS] = mx;
                part0[h * PS + 1] = l;
            }
        }
        __syncthreads();
    }
}

template <int D, int BK, bool QJL, int BV>
void launch_mfma(const tq_packed* k, const tq_packed* v, int64_t n_streams, int64_t T, int64_t stride, int G,
                 const half8_t* frags, const tq_quantizer* qk, const tq_quantizer* qv, float zscale,
                 float* parts, int n_chunks, int tc, hipStream_t s)
{
    const int64_t n_items = n_streams * n_chunks;
    const int64_t cap = (int64_t)device_cus() * 2;
    const unsigned grid = (unsigned)(n_items < cap ? n_items : cap);
    hipLaunchKernelGGL((k_decode_mfma<D, BK, QJL, BV>), dim3(grid), dim3(256), 0, s, k->codes, k->signs, k->norm,
                       k->rnorm, v->codes, v->norm, T, stride, G, frags, qk->centroids, qv->centroids, zscale, parts,
                       n_chunks, tc, n_items);
}

template <int D, int BK, bool QJL>
void launch_bv(int bv, const tq_packed* k, const tq_packed* v, int64_t ns, int64_t T, int64_t stride, int G,
               const half8_t* fr,
               const tq_quantizer* qk, const tq_quantizer* qv, float zs, float* parts, int nc, int tc,
               hipStream_t s)
{
    // value widths 1..4 with keys of 1..4 bits, 3, 4 and 8 with any key width
    switch (bv) {
        case 1: if constexpr (BK <= 4) launch_mfma<D, BK, QJL, 1>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, tc, s); break;
        case 2: if constexpr (BK <= 4) launch_mfma<D, BK, QJL, 2>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, tc, s); break;
        case 3: launch_mfma<D, BK, QJL, 3>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, tc, s); break;
        case 4: launch_mfma<D, BK, QJL, 4>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, tc, s); break;
        default: launch_mfma<D, BK, QJL, 8>(k, v, ns, T, stride, G, fr, qk, qv, zs, parts, nc, tc, s); break;
    }
}

// Score fragments of `tiles` groups of G query rows (rows at or past `total`
// count as zero); with app (one tile per stream), also the append blocks.
void launch_qprep_frag(const tq_quantizer* qk, const void* q, int q_dtype, int64_t tiles, int G, int64_t total,
                       half8_t* frags, const AppendDev* app, hipStream_t s)
{
    constexpr int D = 128;
    const bool qjl = qk->qjl_m != 0;
    AppendDev a{};
    if (app) a = *app;
    const dim3 pg((unsigned)tiles, (unsigned)(D / 32 + (app ? 2 : 0))), pb(256);
    if (q_dtype == TQ_F16) {
        if (qjl) hipLaunchKernelGGL((k_qprep_frag<D, true, true>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags, a);
        else hipLaunchKernelGGL((k_qprep_frag<D, false, true>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags, a);
    } else {
        if (qjl) hipLaunchKernelGGL((k_qprep_frag<D, true, false>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags, a);
        else hipLaunchKernelGGL((k_qprep_frag<D, false, false>), pg, pb, 0, s, q, G, total, qk->diag_signs, qk->S, frags, a);
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
    // packed inputs of one key tile for this lane: A row ka = k0 + col (clamped),
    // norms of rows k0 + 4 g + r (clamped)
    struct KT {
        uint32_t kf[BK];
        uint32_t sf;
        uint16_t nk[4], ng[4];
    };
    auto load_kt = [&](KT& t, int64_t k0) {
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
    };
    for (int64_t qg = blockIdx.y; qg < n_qg; qg += gridDim.y) {
        half8_t bq[kScoreQT][KSTEPS];
#pragma unroll
        for (int j = 0; j < kScoreQT; ++j) {
            const int64_t qt = min(qg * kScoreQT + j, n_qt - 1);  // past the end: repeat, not stored
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) bq[j][k] = frags[(qt * KSTEPS + k) * 64 + lane];
        }
        // the wave takes key tiles in adjacent pairs (2 pr, 2 pr + 1), so the two
        // 64-byte halves of each 128-byte line of a score row are written back to back
        const int64_t pstep = (int64_t)gridDim.x * 4;
        auto next_kt = [&](int64_t kt) { return (kt & 1) ? kt - 1 + 2 * pstep : kt + 1; };
        int64_t kt = 2 * ((int64_t)blockIdx.x * 4 + wid);
        KT cur;
        if (kt < n_kt) load_kt(cur, kt * 16);
        for (; kt < n_kt; kt = next_kt(kt)) {
            const int64_t k0 = kt * 16;
            KT nxt;
            if (next_kt(kt) < n_kt) load_kt(nxt, next_kt(kt) * 16);
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
                    z[r] = fk[r] * (am[r] + xor8(am[r]));
                    if constexpr (QJL) z[r] = fmaf(fq[r], aq[r] + xor8(aq[r]), z[r]);
                }
                const int64_t qrow = (qg * kScoreQT + j) * 8 + (col & 7);
                if (col < 8 && qrow < n_q) {
                    float* dst = scores + qrow * N + k0 + 4 * g;
                    if ((N & 3) == 0 && k0 + 4 * g + 3 < N) {
                        // write-once output: streamed past the caches
                        __builtin_nontemporal_store(float4_t{z[0], z[1], z[2], z[3]}, reinterpret_cast<float4_t*>(dst));
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (k0 + 4 * g + r < N) dst[r] = z[r];
                    }
                }
            }
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
                       int q_dtype, float zscale, void* frags, float* parts, int n_chunks, int tc,
                       const AppendArgs* app, hipStream_t s)
{
    constexpr int D = 128;
    const bool qjl = qk->qjl_m != 0;
    AppendDev ad{};
    if (app) ad = AppendDev{*qk, *qv, *k, *v, app->k_new, app->v_new, app->dtype, stride, app->pos};
    launch_qprep_frag(qk, q, q_dtype, n_streams, G, n_streams * G, (half8_t*)frags, app ? &ad : nullptr, s);
    const half8_t* fr = (const half8_t*)frags;
    switch (qk->mse_bits) {
        case 1: qjl ? launch_bv<D, 1, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                    : launch_bv<D, 1, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
        case 2: qjl ? launch_bv<D, 2, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                    : launch_bv<D, 2, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
        case 3: qjl ? launch_bv<D, 3, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                    : launch_bv<D, 3, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
        case 4: qjl ? launch_bv<D, 4, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                    : launch_bv<D, 4, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
        case 5: qjl ? launch_bv<D, 5, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                    : launch_bv<D, 5, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
        case 6: qjl ? launch_bv<D, 6, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                    : launch_bv<D, 6, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
        case 7: qjl ? launch_bv<D, 7, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                    : launch_bv<D, 7, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
        default: qjl ? launch_bv<D, 8, true>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s)
                     : launch_bv<D, 8, false>(qv->mse_bits, k, v, n_streams, T, stride, G, fr, qk, qv, zscale, parts, n_chunks, tc, s); break;
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
    launch_qprep_frag(q, queries, q_dtype, n_qt, 8, n_q, (half8_t*)frags, nullptr, s);
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
