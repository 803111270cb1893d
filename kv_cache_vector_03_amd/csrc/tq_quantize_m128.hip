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
// S. The projection's B operand is the residual with columns = vectors
// (lane % 16) and k-block q: k-step r, element t is coordinate 4 q + r + 16 t,
// which this lane holds. The A operand is S with its rows permuted so that
// lane (v, q) receives the 32 projections of sign word q of vector v, which
// it packs from their sign bits and stores itself.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kD = 128;
// keys below this count take the short-input kernel: the two-group kernel
// needs a few rounds per block (256 vectors each, one block per compute unit)
// before its alternating phases pay off
constexpr int64_t kKeysShort = 131072;
constexpr float kResUnit = 1024.0f;  // residual scale for the projection operands

// S row feeding row c of m-tile nu. The projection lands in lane (v, c / 4),
// register c % 4, as bit 4 nu + c % 4 of sign word c / 4, i.e. stream bit
// j = 32 (c / 4) + 4 nu + c % 4; group-major, that bit is row j / 8 + 16 (j % 8).
__host__ __device__ constexpr int m128_proj_row(int nu, int c)
{
    return (32 * (c / 4) + 4 * nu + c % 4) / 8 + 16 * ((32 * (c / 4) + 4 * nu + c % 4) % 8);
}

// Codes of the 32 coordinates a lane holds by sign-bit arithmetic. The lane
// holds Z = -Y (the rotation produces the negated coordinates, so the sign bit
// of Z is [Y > 0] with Y = 0 below zero, as a rotated exact zero comes out as
// +0). With the symmetric codebook the top code bit is [Y > 0] and the lower
// bits are the count #{M_j s < |Y|} (XOR-folded from the signs of
// M_j s - |Y|), complemented for Y <= 0. Local stream bit 8 B r + B t + p is
// shifted in from the top. For keys, y is replaced by the negated scaled
// residual (c s - Y) * sc and its squared norm accumulates in g2 (Cq: centroid
// magnitudes times kResUnit).
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
            const float Z = y[t][r];                 // -Y
            const uint32_t d2 = __float_as_uint(Z);  // sign bit = [Y > 0]
            const int P = 8 * B * r + B * t;
            float mag = Cq[0];
            if constexpr (K == 0) {
                W[P >> 5] = __builtin_amdgcn_alignbit(W[P >> 5], d2, 31);
            } else if constexpr (K == 1) {
                const bool outer = fabsf(Z) > Ms[0];
                // bit 0 = [|Y| > M s] for Y > 0, its complement otherwise
                const float b0 = outer ? Z : -Z;
                W[(P + 1) >> 5] = __builtin_amdgcn_alignbit(W[(P + 1) >> 5], d2, 31);
                W[P >> 5] = __builtin_amdgcn_alignbit(W[P >> 5], __float_as_uint(b0), 31);
                if constexpr (QJL) mag = outer ? Cq[1] : Cq[0];
            } else {
                uint32_t e[K];
#pragma unroll
                for (int j = 0; j < K; ++j) e[j] = __float_as_uint(Ms[j] - fabsf(Z));  // [|Y| > M_j s]
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
                const float rn = fmaf(Z, sc, c);  // negated scaled residual
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
// As for the sign-bit codes, the lane holds Z = -Y.
constexpr int kLutCells = 256;
constexpr int kLutEntries = 2 * kLutCells + 2;
constexpr uint32_t kMagicBits = 0x4B000000u;  // bit pattern of 2^23
// Widths 5..8: a finer grid over y in [-1/2, 1/2] (cells of 2^-11; the
// boundaries of these codebooks lie well inside, and the build checks that
// none is within two cells of the edge).
constexpr int kLutCellsW = 1024;                    // cells per half-span
constexpr float kLutPerUnitW = 2.0f * kLutCellsW;    // cells per unit of y
constexpr int kLutEntriesW = 2 * kLutCellsW + 2;
template <int B>
constexpr int lut_entries() { return B >= 3 && B <= 4 ? kLutEntries : (B > 4 ? kLutEntriesW : 1); }

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
            const float Z = y[t][r];  // -Y
            uint32_t bits = __float_as_uint(fmaf(Z, -rs_cells, magic));
            bits = min(max(bits, kMagicBits), kMagicBits + (uint32_t)(kLutEntries - 1));
            const uint2 ent = lut[bits - kMagicBits];
            const float e = fmaf(__uint_as_float(ent.x), s, Z);  // < 0 iff Y > next boundary
            const uint32_t code = ent.y - (uint32_t)((int32_t)__float_as_uint(e) >> 31);
            g = __builtin_amdgcn_alignbit(code, g, B);  // code t ends at bits 32 - 8B + B t
            if constexpr (QJL) {
                const float rn = fmaf(Z, sc, ctab[code & ((1u << B) - 1u)]);  // negated residual
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

// Codes of the 32 coordinates a lane holds for widths 5..8: y = -Z / s, its
// code the number of boundaries strictly below y, read from the fine lookup
// grid (LUT: one LDS read and one comparison, as in codes_lut) or found by a
// branch-free binary search over the boundaries in LDS (tb, padded to 2^B
// entries) when the grid does not resolve the codebook.
// Group r's eight codes form a 64-bit field (code t at bit B t) placed at
// bit 8 B r of the lane's B code words. For keys, y is replaced by the
// negated scaled residual and its square accumulates in g2, as in codes_lut.
template <int B, bool QJL, bool LUT>
__device__ __forceinline__ void codes_search(float (&y)[8][4], const float* __restrict__ tb,
                                             const uint2* __restrict__ lut, const float* __restrict__ ctab,
                                             float s, float rs, float sc, uint32_t (&W)[B], float& g2)
{
    constexpr float magic = 8388608.0f + kLutCellsW;  // 2^23 + NC: rounds to an integer index
    const float rs_cells = kLutPerUnitW * rs;
#pragma unroll
    for (int w = 0; w < B; ++w) W[w] = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        uint64_t gg = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float Z = y[t][r];  // -Y
            int k = 0;
            if constexpr (LUT) {
                uint32_t bits = __float_as_uint(fmaf(Z, -rs_cells, magic));
                bits = min(max(bits, kMagicBits), kMagicBits + (uint32_t)(kLutEntriesW - 1));
                const uint2 ent = lut[bits - kMagicBits];
                const float e = fmaf(__uint_as_float(ent.x), s, Z);  // < 0 iff Y > next boundary
                k = (int)(ent.y - (uint32_t)((int32_t)__float_as_uint(e) >> 31));
            } else {
                const float yy = -Z * rs;
#pragma unroll
                for (int step = 1 << (B - 1); step >= 1; step >>= 1) k += tb[k + step - 1] < yy ? step : 0;
            }
            gg |= (uint64_t)k << (B * t);
            if constexpr (QJL) {
                const float rn = fmaf(Z, sc, ctab[k]);  // negated residual
                g2 = fmaf(rn, rn, g2);
                y[t][r] = rn;
            }
        }
        constexpr int FB = 8 * B;  // bits per group
        const int o = FB * r, ow = o >> 5, ob = o & 31;
        W[ow] |= (uint32_t)(gg << ob);
        if (ob + FB > 32) W[ow + 1] |= (uint32_t)(gg >> (32 - ob));
        if (ob + FB > 64) W[ow + 2] |= (uint32_t)(gg >> (64 - ob));
    }
}

// Shift the sign bits of the four projections t[3], .., t[0] into w from
// below. The projections are negated (t = -(S r)), so the sign bit of t is
// the stored bit [S r >= 0] everywhere except at S r = 0 exactly.
__device__ __forceinline__ uint32_t shift_signs(uint32_t w, const float4_t& t)
{
#pragma unroll
    for (int r4 = 3; r4 >= 0; --r4) w = __builtin_amdgcn_alignbit(w, __float_as_uint(t[r4]), 31);
    return w;
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

// Per-lane constants of the rotation: the negated H_32 slabs and the slabs as A
// operands (lane (row rho = v, k-block q), element e of hA[tau][0] is
// -H_32[16 tau + rho][8 q + e], of hA[tau][1] +H_32[..]), so the rotation yields -Y,
// and the random diagonal's sign flips of the lane's input halves (chunk a',
// word w holds coordinates 32 a' + 8 q + 2 w in its low half and + 1 in its high half).
struct RotConsts {
    half8_t hA[2][2];
    uint32_t dm[4][4];
};

__device__ __forceinline__ void rot_consts(RotConsts& rc, const uint32_t* __restrict__ diag, int v, int q)
{
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool neg = __builtin_popcount((16 * tau + v) & (8 * q + e)) & 1;
            rc.hA[tau][0][e] = neg ? (_Float16)1.0f : (_Float16)-1.0f;
            rc.hA[tau][1][e] = neg ? (_Float16)-1.0f : (_Float16)1.0f;
        }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const uint32_t word = diag[a] >> (8 * q);
#pragma unroll
        for (int w = 0; w < 4; ++w)
            rc.dm[a][w] = (((word >> (2 * w)) & 1u) << 15) | (((word >> (2 * w + 1)) & 1u) << 31);
    }
}

// Rotation of one 16-vector batch: H_32 of each input chunk on MFMA with the
// H_4 signs, accumulated into the output chunks (acc[tau][a] register r is
// coordinate 32 a + 16 tau + 4 q + r, negated), and the lane's share of ||x||^2
// from the fp16 input.
__device__ __forceinline__ void rotate_batch(const uint4 (&xin)[4], const RotConsts& rc, float4_t (&acc)[2][4],
                                             float& ss)
{
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int a = 0; a < 4; ++a) acc[tau][a] = float4_t{0.f, 0.f, 0.f, 0.f};
    ss = 0.f;
#pragma unroll
    for (int ap = 0; ap < 4; ++ap) {
        const uint32_t w4[4] = {xin[ap].x ^ rc.dm[ap][0], xin[ap].y ^ rc.dm[ap][1], xin[ap].z ^ rc.dm[ap][2],
                                xin[ap].w ^ rc.dm[ap][3]};
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
                acc[tau][a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rc.hA[tau][__builtin_popcount(a & ap) & 1], bx,
                                                                     acc[tau][a], 0, 0, 0);
    }
}

// Codebook state: boundaries and centroid magnitudes in registers (sign-bit
// arithmetic), the centroid table and the lookup grid in LDS.
template <int B>
struct CodeConsts {
    static constexpr int L = 1 << B, K = B <= 4 ? L / 2 - 1 : 0;
    float Mth[K > 0 ? K : 1];
    float Cq[K + 1];
    const float* ctab;
    const uint2* lut;
    const float* tb;  // widths 5..8: boundaries, padded with +inf to 2^B entries
    bool use_lut;
};

// Fill the block's centroid table (times `unit`) and, for 3 and 4 bits, the
// lookup grid, and set up cc; the grid is used only if it resolves the
// codebook. Ends with a barrier.
template <int B>
__device__ void build_tables(CodeConsts<B>& cc, const float* __restrict__ cent, const float* __restrict__ bnd,
                             float unit, float* ctab, uint2* lut, int* lut_bad, float* tb)
{
    constexpr int L = 1 << B, K = CodeConsts<B>::K;
    constexpr bool LUT = B >= 3;
    constexpr bool WIDE = B > 4;
    constexpr int NCB = WIDE ? kLutCellsW : kLutCells, NE = lut_entries<B>();
    constexpr float PER = WIDE ? kLutPerUnitW : (float)kLutCells;  // cells per unit of y
#pragma unroll
    for (int j = 1; j <= K; ++j) cc.Mth[j - 1] = bnd[L / 2 - 1 + j];
#pragma unroll
    for (int m = 0; m <= K; ++m) cc.Cq[m] = cent[L / 2 + m] * unit;
    if (threadIdx.x == 0) *lut_bad = 0;
    for (int l = threadIdx.x; l < L; l += blockDim.x) ctab[l] = cent[l] * unit;
    if constexpr (B > 4)
        for (int l = threadIdx.x; l < L; l += blockDim.x) tb[l] = l < L - 1 ? bnd[l] : INFINITY;
    __syncthreads();
    if constexpr (LUT) {
        for (int c = threadIdx.x; c < NE; c += blockDim.x) {
            const float lo = ((float)(c - NCB) - 0.5f) / PER;  // exact
            const float win = lo + 2.0f / PER;
            uint32_t base = 0;
            float next = INFINITY;
            if constexpr (WIDE) {
                // boundaries sorted in tb (padded with +inf): base = #{b < lo} by
                // binary search, next = tb[base]; a second boundary in the
                // two-cell window makes the grid unusable
                int k = 0;
#pragma unroll
                for (int step = 1 << (B - 1); step >= 1; step >>= 1) k += tb[k + step - 1] < lo ? step : 0;
                base = (uint32_t)k;
                next = tb[k];
                if (k + 1 < L - 1 && tb[k + 1] < win) *lut_bad = 1;
            } else {
                int inwin = 0;
                for (int j = 0; j < L - 1; ++j) {
                    const float b = bnd[j];
                    base += b < lo ? 1u : 0u;
                    if (b >= lo && b < next) next = b;
                    inwin += (b >= lo && b < win) ? 1 : 0;
                }
                if (inwin > 1) *lut_bad = 1;
            }
            lut[c] = make_uint2(__float_as_uint(next), base);
        }
        if constexpr (WIDE) {
            // the clamped end cells are exact only if every boundary lies inside the span
            const float edge = ((float)NCB - 2.5f) / PER;
            if (threadIdx.x == 0 && !(fabsf(bnd[0]) < edge && fabsf(bnd[L - 2]) < edge)) *lut_bad = 1;
        }
    }
    __syncthreads();
    cc.ctab = ctab;
    cc.lut = lut;
    cc.tb = tb;
    cc.use_lut = LUT && !*lut_bad;
}

// Code one rotated batch (pure register work): norm, code words, and for keys
// the residual norm and the negated scaled residual split into exact fp16
// hi + lo projection operands (k-step r = group r of the lane). Lane (v, q)
// returns code words B q .. B q + B - 1 of vector v; every lane gets the norms.
template <int B, bool QJL, typename Pre = void (*)(int)>
__device__ __forceinline__ void code_batch(const float4_t (&acc)[2][4], float ss, const CodeConsts<B>& cc,
                                           uint32_t (&W)[B], float& nrm, float& gam, half8_t (&ahi)[4],
                                           half8_t (&alo)[4], Pre&& pre = [](int) {})
{
    constexpr int K = CodeConsts<B>::K;
    constexpr float sqrt_d = 11.313708498984761f;  // sqrt(128)
    auto none = [](int) {};
    // y[t][r]: coordinate 4 q + r + 16 t, t = 2 a + tau
    float y[8][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) y[2 * a + tau][r] = acc[tau][a][r];
    ss = rows_sum(ss);
    // hardware square root (within an ulp of fp32); the stored value is fp16
    nrm = __builtin_amdgcn_sqrtf(ss);
    const float sr = nrm * sqrt_d;  // sqrt(d) ||x||
    const float s = sr > 0.f ? sr : 1.0f;
    const float sc = kResUnit * __builtin_amdgcn_rcpf(s);  // any uniform scale near 1024 / s
    float Ms[K > 0 ? K : 1];
#pragma unroll
    for (int j = 0; j < K; ++j) Ms[j] = cc.Mth[j] * s;

    float g2 = 0.f;
    if constexpr (B > 4) {
        if (cc.use_lut) codes_search<B, QJL, true>(y, cc.tb, cc.lut, cc.ctab, s, __builtin_amdgcn_rcpf(s), sc, W, g2);
        else codes_search<B, QJL, false>(y, cc.tb, cc.lut, cc.ctab, s, __builtin_amdgcn_rcpf(s), sc, W, g2);
    }
    else if (cc.use_lut) codes_lut<B, QJL>(y, cc.lut, cc.ctab, s, (float)kLutCells / s, sc, W, g2, pre, none);
    else codes_compare<B, QJL>(y, Ms, cc.Cq, cc.ctab, sc, W, g2, pre, none);
    gam = 0.f;
    if constexpr (QJL) {
        g2 = rows_sum(g2);
        gam = __builtin_amdgcn_sqrtf(g2) * (1.0f / kResUnit);
        // hi rounds toward zero; lo is the remainder r - hi (exact in fp32, hi
        // taken straight from its fp16 half) rounded once to fp16, written
        // straight into its half of the packed word
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float r0 = y[2 * j][r], r1 = y[2 * j + 1][r];
                hw[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
                uint32_t l;  // the mixhi below writes the high half
                asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l) : "v"(hw[j]), "v"(r0));
                asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                    : "+v"(l) : "v"(hw[j]), "v"(r1));
                lw[j] = l;
            }
            ahi[r] = __builtin_bit_cast(half8_t, hw);
            alo[r] = __builtin_bit_cast(half8_t, lw);
        }
    }
}

// Store lane (v, q)'s code words of vector vec and, from lanes q = 0, its norm
// (and residual norm), if vec < n. The packed output is written once and not
// read back by this launch, so it is streamed past the caches.
template <int B, bool QJL>
__device__ __forceinline__ void store_coded(const uint32_t (&W)[B], float nrm, float gam, int64_t vec, int64_t n,
                                            int q, uint32_t* __restrict__ codes, uint16_t* __restrict__ norm,
                                            uint16_t* __restrict__ rnorm)
{
    constexpr int CW = B * kD / 32;  // code words per vector
    if (vec < n) {
        uint32_t* dst = codes + vec * CW + B * q;
        typedef uint32_t u2v __attribute__((ext_vector_type(2)));
        typedef uint32_t u4v __attribute__((ext_vector_type(4)));
        if constexpr (B == 2) {
            __builtin_nontemporal_store(u2v{W[0], W[1]}, reinterpret_cast<u2v*>(dst));
        } else if constexpr (B == 4) {
            __builtin_nontemporal_store(u4v{W[0], W[1], W[2], W[3]}, reinterpret_cast<u4v*>(dst));
        } else {
#pragma unroll
            for (int w = 0; w < B; ++w) __builtin_nontemporal_store(W[w], dst + w);
        }
        if (q == 0) {
            __builtin_nontemporal_store(f2h(nrm), norm + vec);
            if constexpr (QJL) __builtin_nontemporal_store(f2h(gam), rnorm + vec);
        }
    }
}

// Input of one batch for lane (v, q); rows past the end repeat the last row
// (their results are not stored), so the loads need no branch.
__device__ __forceinline__ void load_clamped(uint4 (&u)[4], const uint16_t* __restrict__ x, int64_t vec, int64_t n,
                                             int q)
{
    const uint16_t* row = x + (vec < n ? vec : n - 1) * kD + 8 * q;
#pragma unroll
    for (int a = 0; a < 4; ++a) u[a] = *reinterpret_cast<const uint4*>(row + 32 * a);
}

// Values (MSE codes only). A wave takes one 16-vector batch at a time and
// fetches the next batch while it processes the current one.
template <int B>
__global__ __launch_bounds__(256) void k_quantize_values_m128(const uint16_t* __restrict__ x, int64_t n,
                                                              const float* __restrict__ cent,
                                                              const float* __restrict__ bnd,
                                                              const uint32_t* __restrict__ diag,
                                                              uint32_t* __restrict__ codes,
                                                              uint16_t* __restrict__ norm)
{
    __shared__ uint2 lut[lut_entries<B>()];
    __shared__ float ctab[1 << B];
    __shared__ float tbl[B > 4 ? 1 << B : 1];
    __shared__ int lut_bad;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int v = lane & 15, q = lane >> 4;
    const int64_t step = (int64_t)gridDim.x * 64;  // vectors between a wave's batches
    int64_t base = ((int64_t)blockIdx.x * 4 + wid) * 16;
    // the first batch's loads go out before the tables are built (rows clamped
    // to n - 1, so a wave past the end also reads in bounds)
    uint4 cur[4];
    load_clamped(cur, x, base + v, n, q);
    RotConsts rc;
    rot_consts(rc, diag, v, q);
    CodeConsts<B> cc;
    build_tables<B>(cc, cent, bnd, 1.0f, ctab, lut, &lut_bad, tbl);

    if (base >= n) return;
    half8_t nh[4], nl[4];  // unused for values
    for (; base < n; base += step) {
        uint4 nxt[4];
        load_clamped(nxt, x, base + step + v, n, q);
        float4_t acc[2][4];
        float ss, nrm, gam;
        uint32_t W[B];
        rotate_batch(cur, rc, acc, ss);
        code_batch<B, false>(acc, ss, cc, W, nrm, gam, nh, nl);
        store_coded<B, false>(W, nrm, gam, base + v, n, q, codes, norm, nullptr);
#pragma unroll
        for (int a = 0; a < 4; ++a) cur[a] = nxt[a];
    }
}

// Phase boundary of the keys kernel: a block barrier that the compiler may not
// move any instruction across, so each phase's work stays between its barriers.
__device__ __forceinline__ void phase_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Keys (codes + QJL sketch). A wave works through pairs of 16-vector batches
// in two alternating phases: coding (vector ALU only: norms, codes, residual
// norm and the residual's fp16 hi + lo operands) and matrix (the rotation of
// its next pair and the projection of the coded pair against S, each S
// fragment read from LDS feeding four MFMAs: both batches, hi and lo). A
// 512-thread block places waves w and w + 4 on one SIMD; waves 4..7 run one
// phase behind waves 0..3 and a block barrier closes every phase, so the two
// waves of a SIMD are always in opposite phases and one's vector work issues
// while the other's matrix products run. Round k of block b covers vectors
// 256 (k G + b) .. + 255 (G blocks), wave w the 32 from 32 (8 (k G + b) + w);
// every wave of a block runs the same number of rounds (rows past the end are
// computed from clamped loads and not stored), so the barriers pair up.
template <int B>
__global__ __launch_bounds__(512) void k_quantize_keys_m128(const uint16_t* __restrict__ x, int64_t n,
                                                            const float* __restrict__ cent,
                                                            const float* __restrict__ bnd,
                                                            const uint32_t* __restrict__ diag,
                                                            const uint16_t* __restrict__ S,
                                                            uint32_t* __restrict__ codes,
                                                            uint32_t* __restrict__ signs,
                                                            uint16_t* __restrict__ norm,
                                                            uint16_t* __restrict__ rnorm)
{
    constexpr int NT = 8, KS = 4;  // projection m-tiles (m = 128) and k-steps
    __shared__ __align__(16) half8_t sfrag[KS * NT * 64];  // 32 KiB
    __shared__ uint2 lut[lut_entries<B>()];
    __shared__ float ctab[1 << B];
    __shared__ float tbl[B > 4 ? 1 << B : 1];
    __shared__ int lut_bad;
    // the rotation's constants (RotConsts) per lane, read from LDS where the
    // rotation runs instead of held in registers through the loop
    __shared__ __align__(16) half8_t rot_a[4][64];
    __shared__ __align__(16) uint4 rot_m[4][4];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const bool late = wid >= 4;
    const int v = lane & 15, q = lane >> 4;
    const int64_t G = gridDim.x;
    const int64_t first = (int64_t)blockIdx.x * 256;
    auto pair_base = [&](int64_t k) { return ((k * G + blockIdx.x) * 8 + wid) * 32; };

    // Set-up loads first, all in flight together: the wave's first pair of input
    // batches (rows clamped to n - 1, so a block past the end also reads in
    // bounds), its share of the S fragments, and the diagonal's signs; the tables
    // are built while they arrive. A fragments: lane (row c, k-block kb) of
    // fragment (ks, nu), element e holds S[proj_row(nu, c)][4 kb + ks + 16 e].
    constexpr int kThreads = 512, kFragPer = KS * NT * 64 / kThreads;
    static_assert(KS * NT * 64 % kThreads == 0, "fragment entries per thread");
    uint4 inA[4], inB[4];
    load_clamped(inA, x, pair_base(0) + v, n, q);
    load_clamped(inB, x, pair_base(0) + 16 + v, n, q);
    half8_t sf[kFragPer];
#pragma unroll
    for (int it = 0; it < kFragPer; ++it) {
        const int e = (int)threadIdx.x + it * kThreads;
        const int ks = e / (NT * 64), nu = (e / 64) % NT, ln = e & 63;
        const int kb = ln >> 4, c = ln & 15;
        const uint16_t* row = S + (int64_t)m128_proj_row(nu, c) * kD;
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) sf[it][ee] = __builtin_bit_cast(_Float16, row[4 * kb + ks + 16 * ee]);
    }
    RotConsts rc0;
    if (wid == 0) rot_consts(rc0, diag, v, q);
    CodeConsts<B> cc;
    build_tables<B>(cc, cent, bnd, kResUnit, ctab, lut, &lut_bad, tbl);
#pragma unroll
    for (int it = 0; it < kFragPer; ++it) {
        const int e = (int)threadIdx.x + it * kThreads;
        const int ks = e / (NT * 64), nu = (e / 64) % NT, ln = e & 63;
        sfrag[(ks * NT + nu) * 64 + ln] = sf[it];
    }
    if (wid == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) rot_a[t][lane] = rc0.hA[t >> 1][t & 1];
        if (v == 0)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                rot_m[q][a] = make_uint4(rc0.dm[a][0], rc0.dm[a][1], rc0.dm[a][2], rc0.dm[a][3]);
    }
    __syncthreads();
    auto rotate_pair = [&](const uint4(&ia)[4], const uint4(&ib)[4], float4_t(&aa)[2][4], float4_t(&ab)[2][4],
                           float& sa, float& sb) {
        RotConsts rc;
#pragma unroll
        for (int t = 0; t < 4; ++t) rc.hA[t >> 1][t & 1] = rot_a[t][lane];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint4 m = rot_m[q][a];
            rc.dm[a][0] = m.x;
            rc.dm[a][1] = m.y;
            rc.dm[a][2] = m.z;
            rc.dm[a][3] = m.w;
        }
        rotate_batch(ia, rc, aa, sa);
        rotate_batch(ib, rc, ab, sb);
    };

    if (first >= n) return;  // the whole block: no barrier is left waiting
    const int64_t rounds = (n - first + G * 256 - 1) / (G * 256);

    float4_t accA[2][4], accB[2][4];
    float ssA, ssB;
    rotate_pair(inA, inB, accA, accB, ssA, ssB);
    if (rounds > 1) {
        load_clamped(inA, x, pair_base(1) + v, n, q);
        load_clamped(inB, x, pair_base(1) + 16 + v, n, q);
    }
    if (late) phase_barrier();
    for (int64_t k = 0; k < rounds; ++k) {
        const int64_t base = pair_base(k), baseB = base + 16;
        // coding phase
        half8_t hiA[KS], loA[KS], hiB[KS], loB[KS];
        {
            float nrm, gam;
            uint32_t W[B];
            code_batch<B, true>(accA, ssA, cc, W, nrm, gam, hiA, loA);
            store_coded<B, true>(W, nrm, gam, base + v, n, q, codes, norm, rnorm);
            code_batch<B, true>(accB, ssB, cc, W, nrm, gam, hiB, loB);
            store_coded<B, true>(W, nrm, gam, baseB + v, n, q, codes, norm, rnorm);
        }
        phase_barrier();
        // matrix phase: project this pair, then rotate the next and fetch the
        // one after (the operands of one step are dead before the next's live)
        // m-tiles from the top so the sign bits enter the words from bit 31 down.
        // Step i = 4 (3 - pt) + ks multiplies the fragments of m-tiles 2 pt and
        // 2 pt + 1 at k-step ks; each step's fragments are read from LDS two
        // steps ahead of their products.
        uint32_t swA = 0, swB = 0;
        constexpr int NS = KS * NT / 2;
        half8_t fr[NS][2];
        auto fetch = [&](int i) {
            const int pt = NT / 2 - 1 - i / KS, ks = i % KS;
            fr[i][0] = sfrag[(ks * NT + 2 * pt) * 64 + lane];
            fr[i][1] = sfrag[(ks * NT + 2 * pt + 1) * 64 + lane];
        };
        fetch(0);
        fetch(1);
        float4_t pA0, pA1, pB0, pB1;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (i + 2 < NS) fetch(i + 2);
            __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
            const int ks = i % KS;
            if (ks == 0) pA0 = pA1 = pB0 = pB1 = float4_t{0.f, 0.f, 0.f, 0.f};
            const half8_t s0 = fr[i][0], s1 = fr[i][1];
            pA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, hiA[ks], pA0, 0, 0, 0);
            pA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, hiA[ks], pA1, 0, 0, 0);
            pB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, hiB[ks], pB0, 0, 0, 0);
            pB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, hiB[ks], pB1, 0, 0, 0);
            pA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, loA[ks], pA0, 0, 0, 0);
            pA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, loA[ks], pA1, 0, 0, 0);
            pB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, loB[ks], pB0, 0, 0, 0);
            pB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, loB[ks], pB1, 0, 0, 0);
            if (ks == KS - 1) {
                swA = shift_signs(shift_signs(swA, pA1), pA0);
                swB = shift_signs(shift_signs(swB, pB1), pB0);
                asm volatile("" : "+v"(swA), "+v"(swB));  // take the sign bits now, freeing the products
            }
        }
        if (base + v < n) __builtin_nontemporal_store(swA, signs + (base + v) * 4 + q);
        if (baseB + v < n) __builtin_nontemporal_store(swB, signs + (baseB + v) * 4 + q);
        if (k + 1 < rounds) {
            rotate_pair(inA, inB, accA, accB, ssA, ssB);
            if (k + 2 < rounds) {
                load_clamped(inA, x, pair_base(k + 2) + v, n, q);
                load_clamped(inB, x, pair_base(k + 2) + 16 + v, n, q);
            }
        }
        phase_barrier();
    }
    if (!late) phase_barrier();
}

// Keys for inputs too short to give every block of the kernel above several
// rounds: 256-thread blocks, each wave coding two 16-vector batches, then
// projecting both residuals against S in one pass in which each S fragment
// read from LDS feeds four MFMAs (both batches, hi and lo). The next pair of
// batches is fetched while the current pair is processed.
template <int B>
__global__ __launch_bounds__(256) void k_quantize_keys_m128_short(const uint16_t* __restrict__ x, int64_t n,
                                                            const float* __restrict__ cent,
                                                            const float* __restrict__ bnd,
                                                            const uint32_t* __restrict__ diag,
                                                            const uint16_t* __restrict__ S,
                                                            uint32_t* __restrict__ codes,
                                                            uint32_t* __restrict__ signs,
                                                            uint16_t* __restrict__ norm,
                                                            uint16_t* __restrict__ rnorm)
{
    constexpr int NT = 8, KS = 4;  // projection m-tiles (m = 128) and k-steps
    __shared__ __align__(16) half8_t sfrag[KS * NT * 64];  // 32 KiB
    __shared__ uint2 lut[lut_entries<B>()];
    __shared__ float ctab[1 << B];
    __shared__ float tbl[B > 4 ? 1 << B : 1];
    __shared__ int lut_bad;

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int v = lane & 15, q = lane >> 4;
    const int64_t step = (int64_t)gridDim.x * 64;  // vectors between a wave's batches
    int64_t base = ((int64_t)blockIdx.x * 4 + wid) * 16;

    // Set-up loads first, all in flight together: the wave's first two input
    // batches (rows clamped to n - 1, so a wave past the end also reads in
    // bounds) and the thread's share of the S fragments; the tables are built
    // while they arrive. A fragments: lane (row c, k-block kb) of fragment
    // (ks, nu), element e holds S[proj_row(nu, c)][4 kb + ks + 16 e].
    constexpr int kThreads = 256, kFragPer = KS * NT * 64 / kThreads;
    static_assert(KS * NT * 64 % kThreads == 0, "fragment entries per thread");
    uint4 inA[4], inB[4];
    load_clamped(inA, x, base + v, n, q);
    load_clamped(inB, x, base + step + v, n, q);
    half8_t sf[kFragPer];
#pragma unroll
    for (int it = 0; it < kFragPer; ++it) {
        const int e = (int)threadIdx.x + it * kThreads;
        const int ks = e / (NT * 64), nu = (e / 64) % NT, ln = e & 63;
        const int kb = ln >> 4, c = ln & 15;
        const uint16_t* row = S + (int64_t)m128_proj_row(nu, c) * kD;
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) sf[it][ee] = __builtin_bit_cast(_Float16, row[4 * kb + ks + 16 * ee]);
    }
    RotConsts rc;
    rot_consts(rc, diag, v, q);
    CodeConsts<B> cc;
    build_tables<B>(cc, cent, bnd, kResUnit, ctab, lut, &lut_bad, tbl);
#pragma unroll
    for (int it = 0; it < kFragPer; ++it) {
        const int e = (int)threadIdx.x + it * kThreads;
        const int ks = e / (NT * 64), nu = (e / 64) % NT, ln = e & 63;
        sfrag[(ks * NT + nu) * 64 + ln] = sf[it];
    }
    __syncthreads();

    if (base >= n) return;
    // one batch: rotation, codes and norms (stored), residual operands
    auto batch = [&](const uint4(&in)[4], int64_t b0, half8_t(&hi)[KS], half8_t(&lo)[KS]) {
        float4_t acc[2][4];
        float ss, nrm, gam;
        uint32_t W[B];
        rotate_batch(in, rc, acc, ss);
        code_batch<B, true>(acc, ss, cc, W, nrm, gam, hi, lo);
        store_coded<B, true>(W, nrm, gam, b0 + v, n, q, codes, norm, rnorm);
    };
    for (; base < n; base += 2 * step) {
        const int64_t baseB = base + step;
        half8_t hiA[KS], loA[KS], hiB[KS], loB[KS];
        batch(inA, base, hiA, loA);
        load_clamped(inA, x, base + 2 * step + v, n, q);
        batch(inB, baseB, hiB, loB);
        load_clamped(inB, x, base + 3 * step + v, n, q);

        // m-tiles from the top so the sign bits enter the words from bit 31 down
        uint32_t swA = 0, swB = 0;
#pragma unroll
        for (int pt = NT / 2 - 1; pt >= 0; --pt) {
            float4_t pA0 = {0.f, 0.f, 0.f, 0.f}, pA1 = pA0, pB0 = pA0, pB1 = pA0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const half8_t s0 = sfrag[(ks * NT + 2 * pt) * 64 + lane];
                const half8_t s1 = sfrag[(ks * NT + 2 * pt + 1) * 64 + lane];
                pA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, hiA[ks], pA0, 0, 0, 0);
                pA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, hiA[ks], pA1, 0, 0, 0);
                pB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, hiB[ks], pB0, 0, 0, 0);
                pB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, hiB[ks], pB1, 0, 0, 0);
                pA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, loA[ks], pA0, 0, 0, 0);
                pA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, loA[ks], pA1, 0, 0, 0);
                pB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s0, loB[ks], pB0, 0, 0, 0);
                pB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(s1, loB[ks], pB1, 0, 0, 0);
            }
            swA = shift_signs(shift_signs(swA, pA1), pA0);
            swB = shift_signs(shift_signs(swB, pB1), pB0);
        }
        if (base + v < n) __builtin_nontemporal_store(swA, signs + (base + v) * 4 + q);
        if (baseB + v < n) __builtin_nontemporal_store(swB, signs + (baseB + v) * 4 + q);
    }
}

// Values (MSE codes only) for d = 256 on MFMA, fp16 or fp32 input.
// H_256 = H_8 (x) H_32 over the coordinate bits (i = 32 a + rho): a wave takes
// 16 vectors at a time, lane (v, q) holding coordinates 32 a' + 8 q .. + 7 of
// vector v for each input chunk a' = 0..7 (the B operand of a 16x16x32 MFMA).
// The A operand of chunk a' and slab tau is the negated H_32 slab (rows
// 16 tau + rho) with the random diagonal's signs of chunk a' folded into its
// columns, read from LDS, so acc[tau][a'] register r holds
// -(H_32 D x)[16 tau + 4 q + r] of chunk a'. H_8 across a' then runs as
// butterflies in registers: output chunk a gives coordinate
// 32 a + 16 tau + 4 q + r, i.e. group n = 16 tau + 4 q + r and member a of the
// group-major layout (groups of stride 32), so lane (v, q) holds groups
// 4 q .. 4 q + 3 (tau = 0) and 16 + 4 q .. (tau = 1) complete and codes them as
// the d = 128 kernels do (Z = -Y, s = sqrt(d) ||x||). fp32 input is scaled by
// a power of two that brings the norm into [1/2, 1) and split into fp16 hi and
// lo operands (two passes; the remainder left over is below 2^-22 of the
// norm); fp16 input is exact as it is.
template <int B, bool F16>
__global__ __launch_bounds__(256) void k_quantize_values_d256(const void* __restrict__ x, int64_t n,
                                                              const float* __restrict__ cent,
                                                              const float* __restrict__ bnd,
                                                              const uint32_t* __restrict__ diag,
                                                              uint32_t* __restrict__ codes,
                                                              uint16_t* __restrict__ norm)
{
    constexpr int D = 256, NA = 8, CW = B * D / 32;  // input chunks, code words per vector
    __shared__ uint2 lut[lut_entries<B>()];
    __shared__ float ctab[1 << B];
    __shared__ float tbl[1];
    __shared__ int lut_bad;
    __shared__ __align__(16) half8_t slab[2][NA][64];  // A operands [tau][a'][lane]
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int v = lane & 15, q = lane >> 4;
    constexpr float sqrt_d = 16.0f;
    const int64_t step = (int64_t)gridDim.x * 64;  // vectors between a wave's batches
    int64_t base = ((int64_t)blockIdx.x * 4 + wid) * 16;
    // one batch's input for lane (v, q): chunk a' holds coordinates 32 a' + 8 q .. + 7;
    // rows past the end repeat the last row (not stored)
    typedef float f8_t __attribute__((ext_vector_type(8)));
    uint4 in16[F16 ? NA : 1];
    f8_t in32[F16 ? 1 : NA];
    auto load = [&](int64_t b0) {
        const int64_t vec = b0 + v < n ? b0 + v : n - 1;
#pragma unroll
        for (int ap = 0; ap < NA; ++ap) {
            if constexpr (F16) in16[ap] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + vec * D + 32 * ap + 8 * q);
            else in32[ap] = *reinterpret_cast<const f8_t*>(static_cast<const float*>(x) + vec * D + 32 * ap + 8 * q);
        }
    };
    // fp16 rows are issued before the tables are built (rows clamped, so in
    // bounds); fp32 rows (twice the registers) after them, to keep two waves per SIMD
    if constexpr (F16) load(base);
    CodeConsts<B> cc;
    build_tables<B>(cc, cent, bnd, 1.0f, ctab, lut, &lut_bad, tbl);
    // lane (row rho, k-block kb) of slab (tau, a'), element e: column c = 8 kb + e,
    // -H_32[16 tau + rho][c] times the diagonal sign of coordinate 32 a' + c
    for (int i = threadIdx.x; i < 2 * NA * 64; i += blockDim.x) {
        const int tau = i / (NA * 64), ap = (i / 64) % NA, ln = i & 63;
        const int rho = ln & 15, kb = ln >> 4;
        const uint32_t dw = diag[ap];
        half8_t h;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * kb + e;
            const bool neg = ((__builtin_popcount((16 * tau + rho) & c) & 1) != 0) != (((dw >> c) & 1u) != 0);
            h[e] = neg ? (_Float16)1.0f : (_Float16)-1.0f;
        }
        slab[tau][ap][ln] = h;
    }
    __syncthreads();

    if (base >= n) return;
    if constexpr (!F16) load(base);
    for (; base < n; base += step) {
        // norm (the lane's 64 coordinates, then the four lanes of the vector)
        float ss = 0.f;
#pragma unroll
        for (int ap = 0; ap < NA; ++ap) {
            if constexpr (F16) {
                const uint32_t w4[4] = {in16[ap].x, in16[ap].y, in16[ap].z, in16[ap].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const auto h2 = __builtin_bit_cast(__attribute__((ext_vector_type(2))) _Float16, w4[w]);
                    ss = __builtin_amdgcn_fdot2(h2, h2, ss, false);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(in32[ap][e], in32[ap][e], ss);
            }
        }
        ss = rows_sum(ss);
        const float nrm = __builtin_amdgcn_sqrtf(ss);
        // fp32: scale 2^-ex with nrm = m 2^ex, m in [1/2, 1) (1 for a zero vector)
        int ex = 0;
        if constexpr (!F16) (void)frexpf(nrm, &ex);
        const float sc = F16 ? 1.0f : ldexpf(1.0f, -ex);
        // H_32 of each chunk on MFMA
        float4_t acc[2][NA];
#pragma unroll
        for (int ap = 0; ap < NA; ++ap) {
            half8_t bh, bl;
            if constexpr (F16) {
                bh = __builtin_bit_cast(half8_t, in16[ap]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float xs = in32[ap][e] * sc;  // exact: a power of two
                    const _Float16 h = (_Float16)xs;
                    bh[e] = h;
                    bl[e] = (_Float16)(xs - (float)h);  // the remainder is exact in fp32
                }
            }
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const half8_t a = slab[tau][ap][lane];
                acc[tau][ap] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                if constexpr (!F16) acc[tau][ap] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, acc[tau][ap], 0, 0, 0);
            }
        }
        load(base + step);  // the next batch, into the registers just read
        // H_8 across the chunks: butterflies (u, w) -> (u + w, u - w) on chunk bit h
#pragma unroll
        for (int h = 1; h < NA; h <<= 1)
#pragma unroll
            for (int ap = 0; ap < NA; ++ap)
                if (!(ap & h))
#pragma unroll
                    for (int tau = 0; tau < 2; ++tau) {
                        const float4_t u = acc[tau][ap], w = acc[tau][ap + h];
                        acc[tau][ap] = u + w;
                        acc[tau][ap + h] = u - w;
                    }
        // codes of the two group sets (tau); Z and s carry the same scale
        const float sr = nrm * sc * sqrt_d;
        const float s_ = sr > 0.f ? sr : 1.0f;
        float Ms[CodeConsts<B>::K > 0 ? CodeConsts<B>::K : 1];
#pragma unroll
        for (int j = 0; j < CodeConsts<B>::K; ++j) Ms[j] = cc.Mth[j] * s_;
        const int64_t vec = base + v;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            float y[8][4];
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) y[a][r] = acc[tau][a][r];
            uint32_t W[B];
            float g2 = 0.f;
            auto none = [](int) {};
            if (cc.use_lut) codes_lut<B, false>(y, cc.lut, cc.ctab, s_, (float)kLutCells / s_, 0.f, W, g2, none, none);
            else codes_compare<B, false>(y, Ms, cc.Cq, cc.ctab, 0.f, W, g2, none, none);
            if (vec < n) {
                uint32_t* dst = codes + vec * CW + B * (4 * tau + q);
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                typedef uint32_t u4v __attribute__((ext_vector_type(4)));
                if constexpr (B == 2) {
                    __builtin_nontemporal_store(u2v{W[0], W[1]}, reinterpret_cast<u2v*>(dst));
                } else if constexpr (B == 4) {
                    __builtin_nontemporal_store(u4v{W[0], W[1], W[2], W[3]}, reinterpret_cast<u4v*>(dst));
                } else {
#pragma unroll
                    for (int w = 0; w < B; ++w) __builtin_nontemporal_store(W[w], dst + w);
                }
            }
        }
        if (vec < n && q == 0) __builtin_nontemporal_store(f2h(nrm), norm + vec);
    }
}

// S row feeding row c of m-tile nu in the d = 256 keys kernel (m = 256). The
// projection lands in lane (v, c / 4), register c % 4; that lane owns sign
// words 2 (c / 4) and 2 (c / 4) + 1 of vector v, i.e. stream bits
// J = 64 (c / 4) + 4 nu + c % 4, and stream bit J holds the sign of row
// J / 8 + 32 (J % 8) (groups of stride 32).
__host__ __device__ constexpr int d256_proj_row(int nu, int c)
{
    return (64 * (c / 4) + 4 * nu + c % 4) / 8 + 32 * ((64 * (c / 4) + 4 * nu + c % 4) % 8);
}

// Keys (codes + QJL sketch, m = 256) for d = 256, fp16 or fp32 input. The
// rotation and coding are the values kernel's above (k_quantize_values_d256);
// the negated scaled residual replaces each coordinate as the codes are
// taken, and its fp16 hi and lo parts are the projection's B operand: k-step
// ks = 4 tau + r, element a is coordinate 32 a + 16 tau + 4 q + r, which lane
// (v, q) holds. The A operand is S with rows and columns permuted to match
// (fragments in LDS, 128 KiB, one block per compute unit); four m-tiles run
// side by side so each accumulator's next MFMA is four instructions away.
template <int B, bool F16>
__global__ __launch_bounds__(512) void k_quantize_keys_d256(const void* __restrict__ x, int64_t n,
                                                            const float* __restrict__ cent,
                                                            const float* __restrict__ bnd,
                                                            const uint32_t* __restrict__ diag,
                                                            const uint16_t* __restrict__ S,
                                                            uint32_t* __restrict__ codes,
                                                            uint32_t* __restrict__ signs,
                                                            uint16_t* __restrict__ norm,
                                                            uint16_t* __restrict__ rnorm)
{
    constexpr int D = 256, NA = 8, CW = B * D / 32, NT = 16, KS = 8;
    extern __shared__ __align__(16) half8_t dyn[];
    half8_t* const sfrag = dyn;  // [KS][NT][64]: 128 KiB
    __shared__ uint2 lut[lut_entries<B>()];
    __shared__ float ctab[1 << B];
    __shared__ float tbl[1];
    __shared__ int lut_bad;
    __shared__ __align__(16) half8_t slab[2][NA][64];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int v = lane & 15, q = lane >> 4;
    constexpr float sqrt_d = 16.0f;
    const int64_t step = (int64_t)gridDim.x * 128;  // vectors between a wave's batches
    int64_t base = ((int64_t)blockIdx.x * 8 + wid) * 16;
    typedef float f8_t __attribute__((ext_vector_type(8)));
    uint4 in16[F16 ? NA : 1];
    f8_t in32[F16 ? 1 : NA];
    auto load = [&](int64_t b0) {
        const int64_t vec = b0 + v < n ? b0 + v : n - 1;
#pragma unroll
        for (int ap = 0; ap < NA; ++ap) {
            if constexpr (F16) in16[ap] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + vec * D + 32 * ap + 8 * q);
            else in32[ap] = *reinterpret_cast<const f8_t*>(static_cast<const float*>(x) + vec * D + 32 * ap + 8 * q);
        }
    };
    // Set-up loads first, all in flight together: the wave's first batch (rows
    // clamped to n - 1, so a wave past the end also reads in bounds) and the
    // thread's share of the S fragments (a fixed trip count); the tables are
    // built while they arrive. A fragments: lane (row c, k-block kb) of fragment
    // (ks = 4 tau + r, nu), element e holds S[d256_proj_row(nu, c)][32 e + 16 tau + 4 kb + r].
    constexpr int kThreads = 512, kFragPer = KS * NT * 64 / kThreads;
    static_assert(KS * NT * 64 % kThreads == 0, "fragment entries per thread");
    load(base);
    half8_t sf[kFragPer];
#pragma unroll
    for (int it = 0; it < kFragPer; ++it) {
        const int i = (int)threadIdx.x + it * kThreads;
        const int ks = i / (NT * 64), nu = (i / 64) % NT, ln = i & 63;
        const int c = ln & 15, kb = ln >> 4, tau = ks >> 2, r = ks & 3;
        const uint16_t* row = S + (int64_t)d256_proj_row(nu, c) * D;
#pragma unroll
        for (int e = 0; e < 8; ++e) sf[it][e] = __builtin_bit_cast(_Float16, row[32 * e + 16 * tau + 4 * kb + r]);
    }
    CodeConsts<B> cc;
    build_tables<B>(cc, cent, bnd, kResUnit, ctab, lut, &lut_bad, tbl);
    for (int i = threadIdx.x; i < 2 * NA * 64; i += blockDim.x) {
        const int tau = i / (NA * 64), ap = (i / 64) % NA, ln = i & 63;
        const int rho = ln & 15, kb = ln >> 4;
        const uint32_t dw = diag[ap];
        half8_t h;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * kb + e;
            const bool neg = ((__builtin_popcount((16 * tau + rho) & c) & 1) != 0) != (((dw >> c) & 1u) != 0);
            h[e] = neg ? (_Float16)1.0f : (_Float16)-1.0f;
        }
        slab[tau][ap][ln] = h;
    }
#pragma unroll
    for (int it = 0; it < kFragPer; ++it) sfrag[(int)threadIdx.x + it * kThreads] = sf[it];
    __syncthreads();

    if (base >= n) return;
    for (; base < n; base += step) {
        float ss = 0.f;
#pragma unroll
        for (int ap = 0; ap < NA; ++ap) {
            if constexpr (F16) {
                const uint32_t w4[4] = {in16[ap].x, in16[ap].y, in16[ap].z, in16[ap].w};
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const auto h2 = __builtin_bit_cast(__attribute__((ext_vector_type(2))) _Float16, w4[w]);
                    ss = __builtin_amdgcn_fdot2(h2, h2, ss, false);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(in32[ap][e], in32[ap][e], ss);
            }
        }
        ss = rows_sum(ss);
        const float nrm = __builtin_amdgcn_sqrtf(ss);
        int ex = 0;
        if constexpr (!F16) (void)frexpf(nrm, &ex);
        const float scl = F16 ? 1.0f : ldexpf(1.0f, -ex);
        float4_t acc[2][NA];
#pragma unroll
        for (int ap = 0; ap < NA; ++ap) {
            half8_t bh, bl;
            if constexpr (F16) {
                bh = __builtin_bit_cast(half8_t, in16[ap]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float xs = in32[ap][e] * scl;
                    const _Float16 h = (_Float16)xs;
                    bh[e] = h;
                    bl[e] = (_Float16)(xs - (float)h);
                }
            }
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const half8_t a = slab[tau][ap][lane];
                acc[tau][ap] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                if constexpr (!F16) acc[tau][ap] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, acc[tau][ap], 0, 0, 0);
            }
        }
#pragma unroll
        for (int h = 1; h < NA; h <<= 1)
#pragma unroll
            for (int ap = 0; ap < NA; ++ap)
                if (!(ap & h))
#pragma unroll
                    for (int tau = 0; tau < 2; ++tau) {
                        const float4_t u = acc[tau][ap], w = acc[tau][ap + h];
                        acc[tau][ap] = u + w;
                        acc[tau][ap + h] = u - w;
                    }
        const float sr = nrm * scl * sqrt_d;
        const float s_ = sr > 0.f ? sr : 1.0f;
        const float sc = kResUnit * __builtin_amdgcn_rcpf(s_);
        float Ms[CodeConsts<B>::K > 0 ? CodeConsts<B>::K : 1];
#pragma unroll
        for (int j = 0; j < CodeConsts<B>::K; ++j) Ms[j] = cc.Mth[j] * s_;
        const int64_t vec = base + v;
        float g2 = 0.f;
        half8_t hi[KS], lo[KS];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            float y[8][4];
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) y[a][r] = acc[tau][a][r];
            uint32_t W[B];
            auto none = [](int) {};
            if (cc.use_lut) codes_lut<B, true>(y, cc.lut, cc.ctab, s_, (float)kLutCells / s_, sc, W, g2, none, none);
            else codes_compare<B, true>(y, Ms, cc.Cq, cc.ctab, sc, W, g2, none, none);
            if (vec < n) {
                uint32_t* dst = codes + vec * CW + B * (4 * tau + q);
                typedef uint32_t u2v __attribute__((ext_vector_type(2)));
                typedef uint32_t u4v __attribute__((ext_vector_type(4)));
                if constexpr (B == 2) {
                    __builtin_nontemporal_store(u2v{W[0], W[1]}, reinterpret_cast<u2v*>(dst));
                } else if constexpr (B == 4) {
                    __builtin_nontemporal_store(u4v{W[0], W[1], W[2], W[3]}, reinterpret_cast<u4v*>(dst));
                } else {
#pragma unroll
                    for (int w = 0; w < B; ++w) __builtin_nontemporal_store(W[w], dst + w);
                }
            }
            // the residual's fp16 parts: k-step 4 tau + r, element a; hi rounds toward
            // zero, lo is the remainder rounded once (as in the d = 128 keys kernel)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float r0 = y[2 * j][r], r1 = y[2 * j + 1][r];
                    hw[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
                    uint32_t l;  // the mixhi below writes the high half
                    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l) : "v"(hw[j]), "v"(r0));
                    asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                        : "+v"(l) : "v"(hw[j]), "v"(r1));
                    lw[j] = l;
                }
                hi[4 * tau + r] = __builtin_bit_cast(half8_t, hw);
                lo[4 * tau + r] = __builtin_bit_cast(half8_t, lw);
            }
        }
        g2 = rows_sum(g2);
        const float gam = __builtin_amdgcn_sqrtf(g2) * (1.0f / kResUnit);
        if (vec < n && q == 0) {
            __builtin_nontemporal_store(f2h(nrm), norm + vec);
            __builtin_nontemporal_store(f2h(gam), rnorm + vec);
        }
        load(base + step);  // the next batch, in flight during the projection
        // projection: m-tiles from the top (sign bits enter each word from bit 31
        // down), four at a time
        uint32_t sw[2] = {0u, 0u};
#pragma unroll
        for (int g4 = NT / 4 - 1; g4 >= 0; --g4) {
            float4_t p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) p[j] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                half8_t f[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) f[j] = sfrag[(ks * NT + 4 * g4 + j) * 64 + lane];
#pragma unroll
                for (int j = 3; j >= 0; --j) p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[j], hi[ks], p[j], 0, 0, 0);
#pragma unroll
                for (int j = 3; j >= 0; --j) p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[j], lo[ks], p[j], 0, 0, 0);
            }
            uint32_t& w = sw[g4 >> 1];
#pragma unroll
            for (int j = 3; j >= 0; --j) w = shift_signs(w, p[j]);
        }
        if (vec < n) {
            typedef uint32_t u2v __attribute__((ext_vector_type(2)));
            __builtin_nontemporal_store(u2v{sw[0], sw[1]}, reinterpret_cast<u2v*>(signs + vec * 8 + 2 * q));
        }
    }
}

template <int B>
void launch_b(const tq_quantizer* q, const uint16_t* x, int64_t n, const tq_packed* o, hipStream_t s)
{
    if (q->qjl_m != 0 && n < kKeysShort) {
        auto kern = k_quantize_keys_m128_short<B>;
        const int grid = resident_grid(kern, 64, n);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, x, n, q->centroids, q->boundaries, q->diag_signs,
                           q->S, o->codes, o->signs, o->norm, o->rnorm);
    } else if (q->qjl_m != 0) {
        auto kern = k_quantize_keys_m128<B>;
        const int grid = resident_grid(kern, 256, n, 512);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(512), 0, s, x, n, q->centroids, q->boundaries, q->diag_signs,
                           q->S, o->codes, o->signs, o->norm, o->rnorm);
    } else {
        auto kern = k_quantize_values_m128<B>;
        const int grid = resident_grid(kern, 64, n);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, x, n, q->centroids, q->boundaries, q->diag_signs,
                           o->codes, o->norm);
    }
}

template <int B, bool F16>
void launch_keys_d256(const tq_quantizer* q, const void* x, int64_t n, const tq_packed* out, hipStream_t s)
{
    constexpr size_t kFrag = 8 * 16 * 64 * sizeof(half8_t);  // the S fragments, 128 KiB of dynamic LDS
    auto kern = k_quantize_keys_d256<B, F16>;
    // once per instance (thread-safe static initialisation): allow the dynamic
    // LDS above the default limit
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kFrag);
    (void)attr;
    const int grid = resident_grid(kern, 128, n, 512);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(512), kFrag, s, x, n, q->centroids, q->boundaries, q->diag_signs, q->S,
                       out->codes, out->signs, out->norm, out->rnorm);
}

}  // namespace

void launch_quantize_values_d256(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* out,
                                 hipStream_t s)
{
    auto go = [&](auto kern) {
        const int grid = resident_grid(kern, 64, n);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, x, n, q->centroids, q->boundaries, q->diag_signs,
                           out->codes, out->norm);
    };
    const bool f16 = dtype == TQ_F16;
    switch (q->mse_bits) {
        case 1: f16 ? go(k_quantize_values_d256<1, true>) : go(k_quantize_values_d256<1, false>); break;
        case 2: f16 ? go(k_quantize_values_d256<2, true>) : go(k_quantize_values_d256<2, false>); break;
        case 3: f16 ? go(k_quantize_values_d256<3, true>) : go(k_quantize_values_d256<3, false>); break;
        default: f16 ? go(k_quantize_values_d256<4, true>) : go(k_quantize_values_d256<4, false>); break;
    }
}

void launch_quantize_keys_d256(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* out,
                               hipStream_t s)
{
    const bool f16 = dtype == TQ_F16;
    switch (q->mse_bits) {
        case 1: f16 ? launch_keys_d256<1, true>(q, x, n, out, s) : launch_keys_d256<1, false>(q, x, n, out, s); break;
        case 2: f16 ? launch_keys_d256<2, true>(q, x, n, out, s) : launch_keys_d256<2, false>(q, x, n, out, s); break;
        case 3: f16 ? launch_keys_d256<3, true>(q, x, n, out, s) : launch_keys_d256<3, false>(q, x, n, out, s); break;
        default: f16 ? launch_keys_d256<4, true>(q, x, n, out, s) : launch_keys_d256<4, false>(q, x, n, out, s); break;
    }
}

void launch_quantize_m128(const tq_quantizer* q, const void* x, int64_t n, const tq_packed* out, hipStream_t s)
{
    const uint16_t* xh = static_cast<const uint16_t*>(x);
    switch (q->mse_bits) {
        case 1: launch_b<1>(q, xh, n, out, s); break;
        case 2: launch_b<2>(q, xh, n, out, s); break;
        case 3: launch_b<3>(q, xh, n, out, s); break;
        case 4: launch_b<4>(q, xh, n, out, s); break;
        case 5: launch_b<5>(q, xh, n, out, s); break;
        case 6: launch_b<6>(q, xh, n, out, s); break;
        case 7: launch_b<7>(q, xh, n, out, s); break;
        default: launch_b<8>(q, xh, n, out, s); break;
    }
}

}  // namespace tq
