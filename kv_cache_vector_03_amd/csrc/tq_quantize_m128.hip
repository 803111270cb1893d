// Quantizer for d = 128 with fp16 input: the rotation runs on MFMA.
//
// Same method as the quad kernel ("[Benchmark] TurboQuant 實測：KV Cache 3-bit
// 壓縮，真的零損失？", section "TurboQuant 是什麼：30 秒懶人包": random
// rotation, stored norm, per-coordinate Lloyd-Max codes, and for keys a 1-bit
// sketch of the residual plus its norm); only the data movement differs.
//
// Rotation. Sylvester's H_128 factors as H_4 (x) H_32 over the coordinate
// bits: H_128[i][j] = (-1)^popcount(i & j) = H_4[i >> 5][j >> 5] H_32[i & 31][j & 31].
// A wave takes 16 vectors at a time, four lanes per vector: lane (v, q) with
// v = lane % 16 and q = lane / 16. For each 32-coordinate chunk a' of the
// input the lane loads coordinates 32 a' + 8 q .. + 7 (sign-flipped by the
// random diagonal) -- the B operand of a 16x16x32 MFMA whose 16 columns are
// the vectors. The A operand is a constant 16-row slab of H_32 (two slabs,
// tau = 0, 1) or its negation, and output chunk a accumulates the four input
// chunks with the signs H_4[a][a'], so each accumulator holds finished
// rotated coordinates: row rho = 4 q + r of slab tau, output chunk a lands in
// lane (v, q), register r, as coordinate 32 a + 16 tau + 4 q + r -- group
// n = 4 q + r, member t = 2 a + tau of the group-major layout. Lane (v, q)
// thus holds the four complete groups 4 q .. 4 q + 3 of vector v, i.e. code
// words B q .. B q + B - 1. The next batch's input is fetched while the
// current one is processed.
//
// Codes follow the quad kernel (sign-bit arithmetic for 1- and 2-bit codes)
// or a lookup grid (3 and 4 bits). For keys the residual is formed, negated,
// directly in units of 1/(1024 s) (s = sqrt(d) ||x||, keeping it in fp16
// range), split into exact fp16 hi + lo operands and projected on MFMA against
// S, with the rows of S permuted so each ballot is two bytes of the sign
// stream. The
// projection's A operand is the residual with rows = vectors (lane % 16) and
// k-block q: k-step r, element t is coordinate 4 q + r + 16 t, which this
// lane holds.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kD = 128;
constexpr float kResUnit = 1024.0f;  // residual scale for the projection operands

// S row feeding column c of n-tile nu (sign stream bits 16 nu .. 16 nu + 15)
__host__ __device__ constexpr int m128_proj_row(int nu, int c) { return 2 * nu + c / 8 + 16 * (c % 8); }

// Codes of the 32 coordinates a lane holds by sign-bit arithmetic: with the
// symmetric codebook the top code bit is [Y > 0] and the lower bits are the
// count #{M_j s < |Y|} (XOR-folded from the signs of M_j s - |Y|), complemented
// for Y <= 0. Local stream bit 8 B r + B t + p is shifted in from the top. For
// keys, y is replaced by the negated scaled residual (c s - Y) * sc and its
// squared norm accumulates in g2 (Cq: centroid magnitudes times kResUnit).
template <int B, bool QJL, int K = (1 << B) / 2 - 1, typename Pre, typename Post>
__device__ __forceinline__ void codes_compare(float (&y)[8][4], const float (&Ms)[K > 0 ? K : 1],
                                              const float (&Cq)[K + 1], const float* __restrict__ ctab, float sc,
                                              uint32_t (&W)[B], float& g2, Pre&& pre, Post&& post)
{
#pragma unroll
    for (int w = 0; w < B; ++w) W[w] = 0;
#pragma unroll
    for (int r = 3; r >= 0; --r) {
        pre(r);
#pragma unroll
        for (int t = 7; t >= 0; --t) {
            const float Y = y[t][r];
            const float d2f = 0.0f - Y;  // sign bit = [Y > 0]
            const uint32_t d2 = __float_as_uint(d2f);
            const int P = 8 * B * r + B * t;
            float mag = Cq[0];
            if constexpr (K == 0) {
                W[P >> 5] = __builtin_amdgcn_alignbit(W[P >> 5], d2, 31);
            } else if constexpr (K == 1) {
                const bool outer = fabsf(Y) > Ms[0];
                // bit 0 = [|Y| > M s] for Y > 0, its complement otherwise
                const float b0 = outer ? d2f : -d2f;
                W[(P + 1) >> 5] = __builtin_amdgcn_alignbit(W[(P + 1) >> 5], d2, 31);
                W[P >> 5] = __builtin_amdgcn_alignbit(W[P >> 5], __float_as_uint(b0), 31);
                if constexpr (QJL) mag = outer ? Cq[1] : Cq[0];
            } else {
                uint32_t e[K];
#pragma unroll
                for (int j = 0; j < K; ++j) e[j] = __float_as_uint(Ms[j] - fabsf(Y));  // [|Y| > M_j s]
#pragma unroll
                for (int p = B - 1; p >= 0; --p) {
                    uint32_t val;
                    if (p == B - 1) {
                        val = d2;
                    } else {
                        uint32_t xq = 0;
#pragma unroll
                        for (int j = 1; j <= K; ++j)
                            if (j % (1 << p) == 0) xq ^= e[j - 1];
                        val = ~(xq ^ d2);
                    }
                    W[(P + p) >> 5] = __builtin_amdgcn_alignbit(W[(P + p) >> 5], val, 31);
                }
                if constexpr (QJL) {
                    // magnitude level from the comparison signs, value from the table
                    uint32_t cnt = 0;
#pragma unroll
                    for (int j = 0; j < K; ++j) cnt += e[j] >> 31;
                    mag = ctab[(1 << B) / 2 + cnt];
                }
            }
            if constexpr (QJL) {
                // c = +mag for Y > 0, -mag otherwise (y = 0 maps to the level just below 0)
                const float c = __uint_as_float(__float_as_uint(mag) ^ (~d2 & 0x80000000u));
                const float rn = fmaf(-Y, sc, c);  // negated scaled residual
                g2 = fmaf(rn, rn, g2);
                y[t][r] = rn;
            }
        }
        post(r);
    }
}

// Code lookup grid. Cell c of the table covers the rotated unit coordinate
// y in [(c - NC - 1/2) / NC, (c - NC + 1/2) / NC); its entry holds the number
// of boundaries below the cell start and the first boundary at or above it.
// The code of Y = sqrt(d) ||x|| y is then base + [Y > next * sqrt(d) ||x||],
// the same strict comparison the codebook defines, as long as no window of two
// cells holds two boundaries (the cell index itself may be off by one where
// rounding puts y on a cell edge). The table is checked for that when built.
constexpr int kLutCells = 256;
constexpr int kLutEntries = 2 * kLutCells + 2;
constexpr uint32_t kMagicBits = 0x4B000000u;  // bit pattern of 2^23

template <int B, bool QJL, typename Pre, typename Post>
__device__ __forceinline__ void codes_lut(float (&y)[8][4], const uint2* __restrict__ lut,
                                          const float* __restrict__ ctab, float s, float rs_cells, float sc,
                                          uint32_t (&W)[B], float& g2, Pre&& pre, Post&& post)
{
    constexpr float magic = 8388608.0f + kLutCells;  // 2^23 + NC: rounds to an integer index
    uint32_t Gr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        pre(r);
        uint32_t g = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float Y = y[t][r];
            uint32_t bits = __float_as_uint(fmaf(Y, rs_cells, magic));
            bits = min(max(bits, kMagicBits), kMagicBits + (uint32_t)(kLutEntries - 1));
            const uint2 ent = lut[bits - kMagicBits];
            const float e = fmaf(__uint_as_float(ent.x), s, -Y);  // < 0 iff Y > next boundary
            const uint32_t code = ent.y - (uint32_t)((int32_t)__float_as_uint(e) >> 31);
            g = __builtin_amdgcn_alignbit(code, g, B);  // code t ends at bits 32 - 8B + B t
            if constexpr (QJL) {
                const float rn = fmaf(-Y, sc, ctab[code & ((1u << B) - 1u)]);  // negated residual
                g2 = fmaf(rn, rn, g2);
                y[t][r] = rn;
            }
        }
        Gr[r] = g;  // group r in its top 8 B bits
        post(r);
    }
    if constexpr (B == 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) W[r] = Gr[r];
    } else if constexpr (B == 3) {
        W[0] = (Gr[0] >> 8) | (Gr[1] << 16);
        W[1] = (Gr[1] >> 16) | (Gr[2] << 8);
        W[2] = (Gr[2] >> 24) | Gr[3];
    } else if constexpr (B == 2) {
        W[0] = (Gr[0] >> 16) | (Gr[1] & 0xFFFF0000u);
        W[1] = (Gr[2] >> 16) | (Gr[3] & 0xFFFF0000u);
    } else {
        W[0] = (Gr[0] >> 24) | ((Gr[1] >> 16) & 0xFF00u) | ((Gr[2] >> 8) & 0xFF0000u) | (Gr[3] & 0xFF000000u);
    }
}

// Half H (0: low, 1: high) of two wave-uniform words packed into one:
// half H of a in bits 0..15, half H of b in bits 16..31 (one scalar op).
template <int H>
__device__ __forceinline__ uint32_t pack_half(uint32_t a, uint32_t b)
{
    uint32_t w;
    if constexpr (H == 0) asm("s_pack_ll_b32_b16 %0, %1, %2" : "=s"(w) : "s"(a), "s"(b));
    else asm("s_pack_hh_b32_b16 %0, %1, %2" : "=s"(w) : "s"(a), "s"(b));
    return w;
}

// Sign word of n-tiles (2p, 2p+1) for the 16 vectors of a batch, from the
// projection accumulators t0, t1 (values -(S r) in scaled units, so the sign
// bit [S r >= 0] is [t <= 0]). Output row 4 g + r4 is vector 4 g + r4; its 16
// bits in each ballot are bits 16 g .. 16 g + 15. Lane v < 16 receives the
// word of vector v.
__device__ __forceinline__ uint32_t sign_word(const float4_t& t0, const float4_t& t1)
{
    uint64_t m0[4], m1[4];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
        m0[r4] = __ballot(t0[r4] <= 0.f);
        m1[r4] = __ballot(t1[r4] <= 0.f);
    }
    uint32_t sw = 0;
    static_for<0, 16>([&](auto k) {
        constexpr int g = decltype(k)::value / 4, r4 = decltype(k)::value % 4;
        const uint32_t a = (uint32_t)(m0[r4] >> (32 * (g / 2)));
        const uint32_t b = (uint32_t)(m1[r4] >> (32 * (g / 2)));
        sw = write_lane<4 * g + r4>(sw, pack_half<g % 2>(a, b));
    });
    return sw;
}

__device__ __forceinline__ void load_batch(uint4 (&u)[4], const uint16_t* __restrict__ x, int64_t vec, int64_t n,
                                           int q)
{
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        u[a] = make_uint4(0u, 0u, 0u, 0u);
        if (vec < n) u[a] = *reinterpret_cast<const uint4*>(x + vec * kD + 32 * a + 8 * q);
    }
}

template <int B, bool QJL>
__global__ __launch_bounds__(256) void k_quantize_m128(const uint16_t* __restrict__ x, int64_t n,
                                                       const float* __restrict__ cent,
                                                       const float* __restrict__ bnd,
                                                       const uint32_t* __restrict__ diag,
                                                       const uint16_t* __restrict__ S,
                                                       uint32_t* __restrict__ codes,
                                                       uint32_t* __restrict__ signs,
                                                       uint16_t* __restrict__ norm,
                                                       uint16_t* __restrict__ rnorm)
{
    constexpr int L = 1 << B, K = L / 2 - 1;
    constexpr int CW = B * kD / 32;  // code words per vector
    constexpr int NT = 8, KS = 4;    // projection n-tiles (m = 128) and k-steps
    constexpr bool LUT = B >= 3;
    __shared__ __align__(16) half8_t bfrag[QJL ? KS * NT * 64 : 1];
    __shared__ uint2 lut[LUT ? kLutEntries : 1];
    __shared__ float ctab[L];  // centroids (times kResUnit for keys)
    __shared__ int lut_bad;

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int v = lane & 15, q = lane >> 4;

    float Mth[K > 0 ? K : 1], Cq[K + 1];
#pragma unroll
    for (int j = 1; j <= K; ++j) Mth[j - 1] = bnd[L / 2 - 1 + j];
#pragma unroll
    for (int m = 0; m <= K; ++m) Cq[m] = cent[L / 2 + m] * kResUnit;

    // H_32 slabs and their negations as A operands: lane (row rho = v,
    // k-block q), element e is +-H_32[16 tau + rho][8 q + e]
    half8_t hA[2][2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool neg = __builtin_popcount((16 * tau + v) & (8 * q + e)) & 1;
            hA[tau][0][e] = neg ? (_Float16)-1.0f : (_Float16)1.0f;
            hA[tau][1][e] = neg ? (_Float16)1.0f : (_Float16)-1.0f;
        }

    // diagonal sign flips of the lane's input halves: chunk a', word w holds
    // coordinates 32 a' + 8 q + 2 w (low half) and + 1 (high half)
    uint32_t dm[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const uint32_t word = diag[a] >> (8 * q);
#pragma unroll
        for (int w = 0; w < 4; ++w)
            dm[a][w] = (((word >> (2 * w)) & 1u) << 15) | (((word >> (2 * w + 1)) & 1u) << 31);
    }

    if (threadIdx.x == 0) lut_bad = 0;
    if (threadIdx.x < L) ctab[threadIdx.x] = cent[threadIdx.x] * (QJL ? kResUnit : 1.0f);
    __syncthreads();
    if constexpr (LUT) {
        for (int c = threadIdx.x; c < kLutEntries; c += 256) {
            const float lo = ((float)(c - kLutCells) - 0.5f) / kLutCells;  // exact
            const float win = lo + 2.0f / kLutCells;
            uint32_t base = 0;
            int inwin = 0;
            float next = INFINITY;
            for (int j = 0; j < L - 1; ++j) {
                const float b = bnd[j];
                base += b < lo ? 1u : 0u;
                if (b >= lo && b < next) next = b;
                inwin += (b >= lo && b < win) ? 1 : 0;
            }
            if (inwin > 1) lut_bad = 1;
            lut[c] = make_uint2(__float_as_uint(next), base);
        }
    }
    if constexpr (QJL) {
        // B fragments: lane (k-block kb, column c) of fragment (ks, nu), element e
        // holds S[proj_row(nu, c)][4 kb + ks + 16 e]
        for (int e = threadIdx.x; e < KS * NT * 64; e += 256) {
            const int ks = e / (NT * 64), nu = (e / 64) % NT, ln = e & 63;
            const int kb = ln >> 4, c = ln & 15;
            const uint16_t* row = S + (int64_t)m128_proj_row(nu, c) * kD;
            half8_t f;
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) f[ee] = __builtin_bit_cast(_Float16, row[4 * kb + ks + 16 * ee]);
            bfrag[(ks * NT + nu) * 64 + ln] = f;
        }
    }
    __syncthreads();
    const bool use_lut = LUT && !lut_bad;

    const float sqrt_d = 11.313708498984761f;  // sqrt(128)
    auto none = [](int) {};

    // One 16-vector batch: rotation, norm and codes (stored), and for keys the
    // residual norm (stored) and the scaled residual split into exact fp16
    // hi + lo projection operands (k-step r = group r of the lane).
    auto batch = [&](const uint4(&xin)[4], int64_t vec, bool live, half8_t(&ahi)[KS], half8_t(&alo)[KS]) {
        // ---- rotation: H_32 per chunk on MFMA with the H_4 signs, accumulated
        // into the output chunks; ||x||^2 from the fp16 input
        float4_t acc[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int a = 0; a < 4; ++a) acc[tau][a] = float4_t{0.f, 0.f, 0.f, 0.f};
        float ss = 0.f;
#pragma unroll
        for (int ap = 0; ap < 4; ++ap) {
            const uint32_t w4[4] = {xin[ap].x ^ dm[ap][0], xin[ap].y ^ dm[ap][1], xin[ap].z ^ dm[ap][2],
                                    xin[ap].w ^ dm[ap][3]};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const auto h2 = __builtin_bit_cast(__attribute__((ext_vector_type(2))) _Float16, w4[w]);
                ss = __builtin_amdgcn_fdot2(h2, h2, ss, false);
            }
            const half8_t bx = __builtin_bit_cast(half8_t, w4);
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    acc[tau][a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        hA[tau][__builtin_popcount(a & ap) & 1], bx, acc[tau][a], 0, 0, 0);
        }
        // y[t][r]: coordinate 4 q + r + 16 t, t = 2 a + tau
        float y[8][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int tau = 0; tau < 2; ++tau)
#pragma unroll
                for (int r = 0; r < 4; ++r) y[2 * a + tau][r] = acc[tau][a][r];
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float nrm = sqrtf(ss);
        const float sr = nrm * sqrt_d;  // sqrt(d) ||x||
        const float s = sr > 0.f ? sr : 1.0f;
        const float sc = kResUnit * __builtin_amdgcn_rcpf(s);  // any uniform scale near 1024 / s
        float Ms[K > 0 ? K : 1];
#pragma unroll
        for (int j = 0; j < K; ++j) Ms[j] = Mth[j] * s;

        // ---- codes (and for keys the negated scaled residual)
        uint32_t W[B];
        float g2 = 0.f;
        if (use_lut) codes_lut<B, QJL>(y, lut, ctab, s, (float)kLutCells / s, sc, W, g2, none, none);
        else codes_compare<B, QJL>(y, Ms, Cq, ctab, sc, W, g2, none, none);
        if (live) {
            uint32_t* dst = codes + vec * CW + B * q;
#pragma unroll
            for (int w = 0; w < B; ++w) dst[w] = W[w];
        }
        if constexpr (QJL) {
            g2 += __shfl_xor(g2, 16);
            g2 += __shfl_xor(g2, 32);
            if (live && q == 0) rnorm[vec] = f2h(sqrtf(g2) * (1.0f / kResUnit));
            // hi rounds toward zero; lo is the fp32 remainder (hi taken straight from
            // its fp16 half) rounded once more
#pragma unroll
            for (int r = 0; r < KS; ++r) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float r0 = y[2 * j][r], r1 = y[2 * j + 1][r];
                    hw[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
                    float l0, l1;
                    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l0) : "v"(hw[j]), "v"(r0));
                    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                        : "=v"(l1) : "v"(hw[j]), "v"(r1));
                    lw[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(l0, l1));
                }
                ahi[r] = __builtin_bit_cast(half8_t, hw);
                alo[r] = __builtin_bit_cast(half8_t, lw);
            }
        }
        if (live && q == 0) norm[vec] = f2h(nrm);
    };

    const int64_t step = (int64_t)gridDim.x * 64;  // vectors between a wave's batches
    int64_t base = ((int64_t)blockIdx.x * 4 + wid) * 16;
    uint4 cur[4];
    load_batch(cur, x, base + v, n, q);
    if constexpr (!QJL) {
        half8_t nh[KS], nl[KS];  // unused for values
        for (; base < n; base += step) {
            uint4 nxt[4];
            load_batch(nxt, x, base + step + v, n, q);
            batch(cur, base + v, base + v < n, nh, nl);
#pragma unroll
            for (int a = 0; a < 4; ++a) cur[a] = nxt[a];
        }
    } else {
        // keys: two batches per iteration, then one projection pass in which each
        // S fragment read from LDS feeds four MFMAs (both batches, hi and lo)
        for (; base < n; base += 2 * step) {
            const int64_t baseB = base + step;
            uint4 nxt[4];
            load_batch(nxt, x, baseB + v, n, q);
            half8_t ahiA[KS], aloA[KS], ahiB[KS], aloB[KS];
            batch(cur, base + v, base + v < n, ahiA, aloA);
            load_batch(cur, x, base + 2 * step + v, n, q);
            batch(nxt, baseB + v, baseB + v < n, ahiB, aloB);

            uint32_t SWA[4], SWB[4];
#pragma unroll
            for (int p = 0; p < NT / 2; ++p) {
                float4_t pA0 = {0.f, 0.f, 0.f, 0.f}, pA1 = pA0, pB0 = pA0, pB1 = pA0;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const half8_t b0 = bfrag[(ks * NT + 2 * p) * 64 + lane];
                    const half8_t b1 = bfrag[(ks * NT + 2 * p + 1) * 64 + lane];
                    pA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahiA[ks], b0, pA0, 0, 0, 0);
                    pA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahiA[ks], b1, pA1, 0, 0, 0);
                    pB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahiB[ks], b0, pB0, 0, 0, 0);
                    pB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahiB[ks], b1, pB1, 0, 0, 0);
                    pA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aloA[ks], b0, pA0, 0, 0, 0);
                    pA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aloA[ks], b1, pA1, 0, 0, 0);
                    pB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aloB[ks], b0, pB0, 0, 0, 0);
                    pB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(aloB[ks], b1, pB1, 0, 0, 0);
                }
                SWA[p] = sign_word(pA0, pA1);
                SWB[p] = sign_word(pB0, pB1);
            }
            if (q == 0) {
                if (base + v < n)
                    *reinterpret_cast<uint4*>(signs + (base + v) * 4) = make_uint4(SWA[0], SWA[1], SWA[2], SWA[3]);
                if (baseB + v < n)
                    *reinterpret_cast<uint4*>(signs + (baseB + v) * 4) = make_uint4(SWB[0], SWB[1], SWB[2], SWB[3]);
            }
        }
    }
}

template <int B, bool QJL>
void launch_b(const tq_quantizer* q, const uint16_t* x, int64_t n, const tq_packed* o, hipStream_t s)
{
    auto kern = k_quantize_m128<B, QJL>;
    const int grid = resident_grid(kern, 64, n);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, x, n, q->centroids, q->boundaries, q->diag_signs,
                       q->S, o->codes, o->signs, o->norm, o->rnorm);
}

}  // namespace

void launch_quantize_m128(const tq_quantizer* q, const void* x, int64_t n, const tq_packed* out, hipStream_t s)
{
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    const bool qjl = q->qjl_m != 0;
    switch (q->mse_bits) {
        case 1: qjl ? launch_b<1, true>(q, xh, n, out, s) : launch_b<1, false>(q, xh, n, out, s); break;
        case 2: qjl ? launch_b<2, true>(q, xh, n, out, s) : launch_b<2, false>(q, xh, n, out, s); break;
        case 3: qjl ? launch_b<3, true>(q, xh, n, out, s) : launch_b<3, false>(q, xh, n, out, s); break;
        default: qjl ? launch_b<4, true>(q, xh, n, out, s) : launch_b<4, false>(q, xh, n, out, s); break;
    }
}

}  // namespace tq
