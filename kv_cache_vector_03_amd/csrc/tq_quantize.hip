// Quantize, query preparation and dequantize kernels.
//
// The quantizer is the two-stage method of "[Benchmark] TurboQuant 實測：KV
// Cache 3-bit 壓縮，真的零損失？", section "TurboQuant 是什麼：30 秒懶人包":
// random rotation, stored norm, per-coordinate Lloyd-Max codes, and for keys
// a 1-bit Johnson-Lindenstrauss sketch of the residual plus its norm.
//
// d = 64, 128: "quad" kernel. Four lanes own one vector (lanes v, v+16, v+32,
// v+48 of a wave; 16 vectors per wave pass), which is exactly the row layout
// of the 16x16x32 MFMA A operand. Each lane loads a contiguous quarter of its
// vector (staged through LDS so the global loads are fully coalesced), runs
// the Walsh-Hadamard butterflies of the quarter's index bits in registers,
// and finishes the two remaining butterflies with permlane16/32 swaps that
// also transpose which coordinates a lane owns: afterwards a lane holds whole
// code groups (coordinates c + (d/8) t, t = 0..7), so it can pack its part of
// the group-major code stream alone. Codes come from sign bits: with the
// symmetric codebook, the top code bit is [y > 0] and the lower bits are the
// magnitude count #{M_j < |y|} (XOR-folded from the signs of M_j - |y|),
// complemented for y <= 0; thresholds are scaled by sqrt(d) ||x|| instead of
// normalising every coordinate. For keys the residual is split into fp16
// hi + lo parts (both exact operands) and projected on MFMA against the fp16
// matrix S (the A operand, rows permuted) so that each lane receives the sign
// bits of one word (d = 128) or half-word (d = 64) of its own vector's stream.
//
// d = 256: the MFMA rotation kernels in tq_quantize_m128.hip (values, and
// keys with the m = 256 projection).
//
// Dequantize: d = 128 takes 16 vectors per wave pass with the sketch term
// S^T s on MFMA; d = 64 and 256 take one wave per vector.
#include "tq_device.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kWavesPerBlock = 4;

// ---------------------------------------------------------------- quad kernel

template <int D>
struct QuadShape {
    static constexpr int Q4 = D / 4;                 // values per lane
    static constexpr int LOG = D == 64 ? 6 : 7;
    static constexpr int Y1 = LOG - 5, Y2 = LOG - 4; // coordinate bits that become lane bits
    static constexpr int MY1 = 1 << Y1, MY2 = 1 << Y2;
    static constexpr int G = D / 8, GL = D / 32;     // groups, groups per lane
    static constexpr int KS = D / 32;                // MFMA k-steps
    static constexpr int NT = D / 16;                // MFMA n-tiles (m = d rows of S)

    // coordinate held in register r by lane quarter q after the transform
    __host__ __device__ static constexpr int coord(int q, int r)
    {
        return (r & ~(MY1 | MY2)) | ((q & 1) << Y1) | ((q >> 1) << Y2) | (((r >> Y1) & 1) << (LOG - 2)) |
               (((r >> Y2) & 1) << (LOG - 1));
    }
    // register holding code t of local group g (the same in every lane)
    __host__ __device__ static constexpr int reg(int g, int t)
    {
        return g | (((t >> 1) & 1) << Y1) | (((t >> 2) & 1) << Y2) | ((t & 1) << (LOG - 3));
    }
    // S row feeding row n = 4 q + r4 of m-tile nu. The projection lands in lane
    // (v, q), register r4, of vector v; the rows are chosen so that lane q's
    // 4 x NT projections are exactly sign word q (d = 128) or the 16-bit half q
    // of the sign stream (d = 64), at bit sign_pos(nu, r4).
    __host__ __device__ static constexpr int proj_row(int nu, int n)
    {
        return D == 128 ? n + 16 * nu : 2 * (n >> 2) + (n & 1) + 8 * (2 * nu + ((n & 3) >> 1));
    }
    __host__ __device__ static constexpr int sign_pos(int nu, int r4)
    {
        return D == 128 ? 8 * r4 + nu : 8 * (r4 & 1) + 2 * nu + (r4 >> 1);
    }
};

template <int D, int B, bool QJL, bool F16>
__global__ __launch_bounds__(256) void k_quantize_quad(const void* __restrict__ x, int64_t n,
                                                       const float* __restrict__ cent,
                                                       const float* __restrict__ bnd,
                                                       const uint32_t* __restrict__ diag,
                                                       const uint16_t* __restrict__ S,
                                                       uint32_t* __restrict__ codes,
                                                       uint32_t* __restrict__ signs,
                                                       uint16_t* __restrict__ norm,
                                                       uint16_t* __restrict__ rnorm)
{
    using Sh = QuadShape<D>;
    constexpr int Q4 = Sh::Q4, GL = Sh::GL, KS = Sh::KS, NT = Sh::NT;
    constexpr int L = 1 << B, K = L / 2 - 1;
    constexpr int ES = F16 ? 2 : 4;
    constexpr int NV = 16;                           // vectors per wave pass
    constexpr int ROW = D * ES + 16;                 // padded LDS row (conflict-free reads)
    constexpr int CH = NV * D * ES / (16 * 64);      // 16-byte chunks per lane per pass
    constexpr int LBITS = 8 * B * GL;                // code-stream bits owned by a lane
    constexpr int LW = (LBITS + 31) / 32;
    constexpr int CW = B * D / 32;                   // code words per vector
    constexpr int SWN = D / 32;                      // sign words per vector

    __shared__ __align__(16) unsigned char stage[kWavesPerBlock][NV * ROW];
    __shared__ __align__(16) half8_t bfrag[QJL ? KS * NT * 64 : 1];

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int v = lane & 15, q = lane >> 4;

    const unsigned char* xb = static_cast<const unsigned char*>(x);
    unsigned char* st = stage[wid];

    // coalesced loads of a pass's NV vectors per wave (16 bytes per lane per
    // chunk); the next pass's chunks are in flight while a pass is processed.
    // The first pass's loads and (for keys) the S gathers go out before the
    // tables are built, so their latencies overlap.
    const int64_t pstep = (int64_t)gridDim.x * (kWavesPerBlock * NV);
    uint4 pre[CH];
    auto fetch = [&](int64_t b0) {
        const int64_t vb0 = b0 + (int64_t)wid * NV;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int off = (c * 64 + lane) * 16;
            const int vec = off / (D * ES);
            pre[c] = vb0 + vec < n ? *reinterpret_cast<const uint4*>(xb + (vb0 * D) * ES + off)
                                   : make_uint4(0, 0, 0, 0);
        }
    };
    fetch((int64_t)blockIdx.x * (kWavesPerBlock * NV));
    // B fragments: lane (qq, nn) of fragment (t, nu) holds S[proj_row(nu, nn)][coord(qq, 8t + e)];
    // a fixed trip count, so all of a thread's gathers are in flight together
    constexpr int kFragPer = QJL ? KS * NT * 64 / 256 : 1;
    static_assert(!QJL || KS * NT * 64 % 256 == 0, "fragment entries per thread");
    half8_t sf[kFragPer];
    if constexpr (QJL) {
#pragma unroll
        for (int it = 0; it < kFragPer; ++it) {
            const int e = (int)threadIdx.x + it * 256;
            const int t = e / (NT * 64), nu = (e / 64) % NT, ln = e & 63;
            const int qq = ln >> 4, nn = ln & 15;
            const uint16_t* row = S + (int64_t)Sh::proj_row(nu, nn) * D;
#pragma unroll
            for (int ee = 0; ee < 8; ++ee) sf[it][ee] = __builtin_bit_cast(_Float16, row[Sh::coord(qq, 8 * t + ee)]);
        }
    }

    float Mth[K > 0 ? K : 1], Cm[K + 1];
#pragma unroll
    for (int j = 1; j <= K; ++j) Mth[j - 1] = bnd[L / 2 - 1 + j];
#pragma unroll
    for (int m = 0; m <= K; ++m) Cm[m] = cent[L / 2 + m];
    // 3 and 4 bits without the sketch: a lookup grid over y in [-1, 1] (cells
    // of 1/256; entry: boundaries below the cell start, first boundary at or
    // above it), used if no window of two cells holds two boundaries (the cell
    // index of the scaled coordinate may be off by one at a cell edge); else,
    // and for keys (where the second code path costs occupancy), sign-bit
    // arithmetic
    constexpr bool GRID = B >= 3 && !QJL;
    constexpr int NC = 256, NE = GRID ? 2 * NC + 2 : 1;
    __shared__ uint2 glut[NE];
    __shared__ float gcent[L];
    __shared__ int glut_bad;
    if (threadIdx.x == 0) glut_bad = 0;
    if (threadIdx.x < L) gcent[threadIdx.x] = cent[threadIdx.x];
    __syncthreads();
    if constexpr (GRID) {
        for (int e = threadIdx.x; e < NE; e += 256) {
            const float lo = ((float)(e - NC) - 0.5f) / NC;  // exact
            const float win = lo + 2.0f / NC;
            uint32_t base = 0;
            int inwin = 0;
            float next = INFINITY;
            for (int l = 0; l < L - 1; ++l) {
                const float bl = bnd[l];
                base += bl < lo ? 1u : 0u;
                if (bl >= lo && bl < next) next = bl;
                inwin += (bl >= lo && bl < win) ? 1 : 0;
            }
            if (inwin > 1) glut_bad = 1;
            glut[e] = make_uint2(__float_as_uint(next), base);
        }
    }
    __syncthreads();
    const bool use_grid = GRID && !glut_bad;

    // sign flips of this lane's initial coordinates q*Q4 + k
    uint32_t fl[F16 ? Q4 / 2 : Q4];
    {
        uint32_t dbits[(Q4 + 31) / 32];
#pragma unroll
        for (int w = 0; w < (Q4 + 31) / 32; ++w) {
            const int c0 = q * Q4 + 32 * w;
            const uint32_t word = diag[c0 >> 5];
            dbits[w] = Q4 >= 32 ? word : (word >> (c0 & 31));
        }
#pragma unroll
        for (int k = 0; k < Q4; ++k) {
            const uint32_t b = (dbits[k >> 5] >> (k & 31)) & 1u;
            if constexpr (F16) {
                if (k & 1) fl[k >> 1] |= b << 31;
                else fl[k >> 1] = b << 15;
            } else {
                fl[k] = b << 31;
            }
        }
    }

    if constexpr (QJL) {
#pragma unroll
        for (int it = 0; it < kFragPer; ++it) {
            const int e = (int)threadIdx.x + it * 256;
            const int t = e / (NT * 64), nu = (e / 64) % NT, ln = e & 63;
            bfrag[(t * NT + nu) * 64 + ln] = sf[it];
        }
    }

    for (int64_t base = (int64_t)blockIdx.x * (kWavesPerBlock * NV); base < n; base += pstep) {
        const int64_t vb = base + (int64_t)wid * NV;
        // this pass's chunks into the wave's staging rows
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int off = (c * 64 + lane) * 16;
            const int vec = off / (D * ES), in = off % (D * ES);
            *reinterpret_cast<uint4*>(st + vec * ROW + in) = pre[c];
        }
        fetch(base + pstep);
        __syncthreads();

        // this lane's quarter, with the diagonal flips and the first butterfly
        float y[Q4];
        float ss = 0.f;
        if constexpr (F16) {
#pragma unroll
            for (int c = 0; c < Q4 / 8; ++c) {
                const uint4 u = *reinterpret_cast<const uint4*>(st + v * ROW + q * Q4 * 2 + 16 * c);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t pr = w4[i] ^ fl[4 * c + i];
                    const float a = h2f((uint16_t)(pr & 0xFFFF)), b = h2f((uint16_t)(pr >> 16));
                    ss += a * a + b * b;
                    y[8 * c + 2 * i] = a + b;
                    y[8 * c + 2 * i + 1] = a - b;
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < Q4 / 4; ++c) {
                const uint4 u = *reinterpret_cast<const uint4*>(st + v * ROW + q * Q4 * 4 + 16 * c);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float a = __uint_as_float(w4[i] ^ fl[4 * c + i]);
                    const float b = __uint_as_float(w4[i + 1] ^ fl[4 * c + i + 1]);
                    ss += a * a + b * b;
                    y[4 * c + i] = a + b;
                    y[4 * c + i + 1] = a - b;
                }
            }
        }
        // remaining in-register butterflies (register bits 1 .. log2(Q4)-1)
#pragma unroll
        for (int h = 2; h < Q4; h <<= 1)
#pragma unroll
            for (int r = 0; r < Q4; ++r)
                if (!(r & h)) {
                    const float a = y[r], b = y[r + h];
                    y[r] = a + b;
                    y[r + h] = a - b;
                }
        // butterfly on index bit log2(d)-2 across lanes q^1; the swap leaves each
        // lane holding one value of coordinate bit Y1 (register bit Y1 now means bit log2(d)-2)
#pragma unroll
        for (int r = 0; r < Q4; ++r)
            if (!(r & Sh::MY1)) {
                const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(y[r]),
                                                                __float_as_uint(y[r | Sh::MY1]), false, false);
                const float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
                y[r] = a + b;
                y[r | Sh::MY1] = a - b;
            }
        // butterfly on index bit log2(d)-1 across lanes q^2 (lane bit becomes Y2)
#pragma unroll
        for (int r = 0; r < Q4; ++r)
            if (!(r & Sh::MY2)) {
                const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(y[r]),
                                                                __float_as_uint(y[r | Sh::MY2]), false, false);
                const float a = __uint_as_float(p[0]), b = __uint_as_float(p[1]);
                y[r] = a + b;
                y[r | Sh::MY2] = a - b;
            }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float nrm = sqrtf(ss);
        const float s = nrm > 0.f ? sqrtf((float)D) * nrm : 1.0f;
        float Ms[K > 0 ? K : 1], Cs[K + 1];
#pragma unroll
        for (int j = 0; j < K; ++j) Ms[j] = Mth[j] * s;
#pragma unroll
        for (int m = 0; m <= K; ++m) Cs[m] = Cm[m] * s;

        // codes: stream bits in descending order, shifted into LW words
        uint32_t W[LW];
#pragma unroll
        for (int w = 0; w < LW; ++w) W[w] = 0;
        float g2 = 0.f;
        if (use_grid) {
            const float rs_cells = (float)NC * __builtin_amdgcn_rcpf(s);
#pragma unroll
            for (int gp = GL - 1; gp >= 0; --gp)
#pragma unroll
                for (int t = 7; t >= 0; --t) {
                    const int r = Sh::reg(gp, t);
                    const float Y = y[r];
                    uint32_t bits = __float_as_uint(fmaf(Y, rs_cells, 8388608.0f + NC));
                    bits = min(max(bits, 0x4B000000u), 0x4B000000u + (uint32_t)(NE - 1));
                    const uint2 ent = glut[bits - 0x4B000000u];
                    const float e = fmaf(-__uint_as_float(ent.x), s, Y);  // > 0 iff Y > next boundary
                    const uint32_t k = ent.y + (e > 0.f ? 1u : 0u);
#pragma unroll
                    for (int p = B - 1; p >= 0; --p) {
                        const int P = 8 * B * gp + B * t + p;
                        W[P >> 5] = __builtin_amdgcn_alignbit(W[P >> 5], k << (31 - p), 31);
                    }
                    if constexpr (QJL) {
                        const float rr = fmaf(-gcent[k], s, Y);
                        g2 += rr * rr;
                        y[r] = rr;
                    }
                }
        } else
#pragma unroll
        for (int gp = GL - 1; gp >= 0; --gp)
#pragma unroll
            for (int t = 7; t >= 0; --t) {
                const int r = Sh::reg(gp, t);
                const float Y = y[r];
                const uint32_t d2 = __float_as_uint(0.0f - Y);     // sign bit = [Y > 0]
                uint32_t e[K > 0 ? K : 1];
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
                    const int P = 8 * B * gp + B * t + p;
                    W[P >> 5] = __builtin_amdgcn_alignbit(W[P >> 5], val, 31);
                }
                if constexpr (QJL) {
                    float mag = Cs[0];
#pragma unroll
                    for (int j = 0; j < K; ++j) mag = fabsf(Y) > Ms[j] ? Cs[j + 1] : mag;
                    // c = +mag for Y > 0, -mag otherwise (y = 0 maps to the level just below 0)
                    const float c = __uint_as_float((__float_as_uint(mag) & 0x7FFFFFFFu) | (~d2 & 0x80000000u));
                    const float rr = Y - c;
                    g2 += rr * rr;
                    y[r] = rr;
                }
            }

        const int64_t vec = vb + v;
        const bool live = vec < n;
        if (live) {
            if constexpr (LBITS % 32 == 0) {
                uint32_t* dst = codes + vec * CW + q * LW;
#pragma unroll
                for (int w = 0; w < LW; ++w) dst[w] = W[w];
            } else {
                uint16_t* dst = reinterpret_cast<uint16_t*>(codes + vec * CW) + q * (LBITS / 16);
#pragma unroll
                for (int h = 0; h < LBITS / 16; ++h) dst[h] = (uint16_t)(W[h >> 1] >> (16 * (h & 1)));
            }
        }

        if constexpr (QJL) {
            g2 += __shfl_xor(g2, 16);
            g2 += __shfl_xor(g2, 32);
            // residual in units of 1/(1024 s) (fp16 range), split into exact fp16 hi + lo
            const float sc = 1024.0f / s;
            half8_t ahi[KS], alo[KS];
#pragma unroll
            for (int t = 0; t < KS; ++t)
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    const float rs = y[8 * t + e2] * sc;
                    const _Float16 hi = (_Float16)rs;
                    ahi[t][e2] = hi;
                    alo[t][e2] = (_Float16)(rs - (float)hi);
                }
            // S as the A operand (rows = projections), the residual as the B operand
            // (columns = vectors): lane (v, q) receives its own sign bits
            uint32_t sw = 0;
#pragma unroll
            for (int nu = 0; nu < NT; ++nu) {
                float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    const half8_t bf = bfrag[(t * NT + nu) * 64 + lane];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, ahi[t], acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf, alo[t], acc, 0, 0, 0);
                }
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) sw |= (acc[r4] >= 0.f ? 1u : 0u) << Sh::sign_pos(nu, r4);
            }
            if (live) {
                if constexpr (D == 128) signs[vec * SWN + q] = sw;
                else reinterpret_cast<uint16_t*>(signs + vec * SWN)[q] = (uint16_t)sw;
                if (q == 0) rnorm[vec] = f2h(sqrtf(g2) / s);
            }
        }
        if (live && q == 0) norm[vec] = f2h(nrm);
        __syncthreads();
    }
}

// q' = H (D .* q) / sqrt(d) and p = S q' (one wave per query). Queries are
// few, so this runs in double and stores fp32 results rounded once, which
// keeps the rotation and projection error far below the score tolerance.
template <int D, bool QJL, bool F16>
__global__ __launch_bounds__(256) void k_qprep(const void* __restrict__ q, int64_t nq,
                                               const uint32_t* __restrict__ diag,
                                               const uint16_t* __restrict__ S,
                                               float* __restrict__ qr, float* __restrict__ p)
{
    constexpr int R = D / 64;
    __shared__ double sq[kWavesPerBlock][D];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);
    for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < nq;
         base += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t a = base + wid;
        const bool active = a < nq;
        double y[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float xv = active ? load_elem<F16>(q, a * D + 64 * r + lane) : 0.f;
            y[r] = (double)flip(xv, dm[r]);
        }
        fwht_wave<R>(y, lane);
        const double sc = 1.0 / sqrt((double)D);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            y[r] *= sc;
            if (active) qr[a * D + 64 * r + lane] = (float)y[r];
            sq[wid][64 * r + lane] = y[r];
        }
        if constexpr (QJL) {
            __syncthreads();
#pragma unroll
            for (int k = 0; k < R; ++k) {
                const int j = 64 * k + lane;
                const uint16_t* Sj = S + (int64_t)j * D;
                double u = 0.0;
                for (int i = 0; i < D; ++i) u += (double)h2f(Sj[i]) * sq[wid][i];
                if (active) p[a * D + j] = (float)u;
            }
            __syncthreads();
        }
    }
}

// x_hat = n D H (c[idx] + [qjl] g sqrt(pi/2)/m S^T s) / sqrt(d)  (one wave per vector)
template <int D, int B, bool QJL, bool F16OUT>
__global__ __launch_bounds__(256) void k_dequantize(const uint32_t* __restrict__ codes,
                                                    const uint32_t* __restrict__ signs,
                                                    const uint16_t* __restrict__ norm,
                                                    const uint16_t* __restrict__ rnorm, int64_t n,
                                                    const float* __restrict__ cent,
                                                    const uint32_t* __restrict__ diag,
                                                    const uint16_t* __restrict__ S,
                                                    void* __restrict__ out)
{
    constexpr int R = D / 64, L = 1 << B, CW = B * D / 32;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    float c[L];
#pragma unroll
    for (int l = 0; l < L; ++l) c[l] = cent[l];
    uint32_t dm[R];
    load_diag<R>(diag, lane, dm);
    for (int64_t base = (int64_t)blockIdx.x * kWavesPerBlock; base < n;
         base += (int64_t)gridDim.x * kWavesPerBlock) {
        const int64_t v = base + wid;
        if (v >= n) continue;  // no block-level synchronisation below
        const uint32_t* cv = codes + v * CW;
        float a[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = 64 * r + lane;
            int k = 0;
#pragma unroll
            for (int p = 0; p < B; ++p) {
                const int P = code_bit<D, B>(i, p);
                k |= (int)((cv[P >> 5] >> (P & 31)) & 1u) << p;
            }
            a[r] = pick<L>(c, k);
        }
        if constexpr (QJL) {
            const float g = h2f(rnorm[v]) * (kSqrtHalfPi / (float)D);
            const uint32_t* sv = signs + v * (D / 32);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = 64 * r + lane;
                float acc = 0.f;
                for (int j = 0; j < D; ++j) {
                    const int P = sign_bit<D>(j);
                    const float sg = ((sv[P >> 5] >> (P & 31)) & 1u) ? 1.f : -1.f;
                    acc += h2f(S[(int64_t)j * D + i]) * sg;
                }
                a[r] += g * acc;
            }
        }
        fwht_wave<R>(a, lane);
        const float sc = h2f(norm[v]) / sqrtf((float)D);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float o = flip(a[r], dm[r]) * sc;
            const int64_t e = v * D + 64 * r + lane;
            if constexpr (F16OUT) static_cast<uint16_t*>(out)[e] = f2h(o);
            else static_cast<float*>(out)[e] = o;
        }
    }
}

// d = 128 dequantize; for keys the sketch term runs on MFMA. A wave takes 16
// vectors per pass; the term u_i = sum_j S[j][i] s_j (s_j = +-1) is a 16-vector x 128 x
// 128 product. The A operand is vector (lane % 16)'s sign byte c = 4 ks + q
// (rows c + 16 e of the group-major sign stream, e = 0..7), expanded to +-1
// through an LDS table; the B operand holds the same rows of S for coordinate
// 16 nt + lane % 16 (fragments built once per block in LDS). Output register
// r of n-tile nt in lane (i, q) = (lane % 16, lane / 16) is coordinate
// 16 nt + i of vector 4 q + r. In the group-major code layout the codes of
// coordinates i + 16 t are group i's field, so one B-byte load per vector
// gives the lane all its codes; the inverse rotation runs over nt in registers
// (coordinate bits 4..6) and over i by DPP (bits 0..3).
template <int B, bool QJL, bool F16OUT>
__global__ __launch_bounds__(256, 4) void k_dequantize128(const uint32_t* __restrict__ codes,
                                                            const uint32_t* __restrict__ signs,
                                                            const uint16_t* __restrict__ norm,
                                                            const uint16_t* __restrict__ rnorm, int64_t n,
                                                            const float* __restrict__ cent,
                                                            const uint32_t* __restrict__ diag,
                                                            const uint16_t* __restrict__ S,
                                                            void* __restrict__ out)
{
    constexpr int D = 128, L = 1 << B, NT = 8, KS = 4, NV = 16;
    __shared__ half8_t sfr[QJL ? KS * NT * 64 : 1];
    __shared__ uint4 slut[QJL ? 256 : 1];
    __shared__ float ctab[L];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int i = lane & 15, q = lane >> 4;
    for (int e = tid; e < (QJL ? KS * NT * 64 : 0); e += 256) {
        const int ks = e / (NT * 64), nt = (e / 64) % NT, ln = e & 63;
        const int col = 16 * nt + (ln & 15), c = 4 * ks + (ln >> 4);
        half8_t f;
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) f[ee] = __builtin_bit_cast(_Float16, S[(c + 16 * ee) * D + col]);
        sfr[e] = f;
    }
    if constexpr (QJL) {
        // sign byte tid -> eight fp16 values, element t = +1 where bit t is set, else -1
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (((tid >> (2 * j)) & 1) ? 0x3C00u : 0xBC00u) |
                   ((((tid >> (2 * j + 1)) & 1) ? 0x3C00u : 0xBC00u) << 16);
        slut[tid] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (tid < L) ctab[tid] = cent[tid];
    // diagonal flips of this lane's coordinates 16 nt + i (bit nt), and the
    // sign masks of the DPP butterflies (lane bit b of i)
    uint32_t dmask = 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int cc = 16 * nt + i;
        dmask |= ((diag[cc >> 5] >> (cc & 31)) & 1u) << nt;
    }
    uint32_t sm[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) sm[b] = ((uint32_t)(i >> b) & 1u) << 31;
    const float kap = kSqrtHalfPi / (float)D;
    const float isd = 1.0f / sqrtf((float)D);
    __syncthreads();

    // one pass's packed inputs for this lane: sign words of vector vb + i, and
    // group i's code field and the norms of vectors vb + 4 q + r (rows past the
    // end read the last vector and are not stored); the next pass's are loaded
    // while a pass is processed
    struct In {
        uint32_t sw[4], f[4];
        uint16_t nv[4], rn[4];
    };
    auto fetch = [&](int64_t vb, In& t) {
        if constexpr (QJL) {
            const int64_t va = vb + i < n ? vb + i : n - 1;
            const uint4 w = *reinterpret_cast<const uint4*>(signs + va * (D / 32));
            t.sw[0] = w.x;
            t.sw[1] = w.y;
            t.sw[2] = w.z;
            t.sw[3] = w.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t v = vb + 4 * q + r;
            const int64_t vr = v < n ? v : n - 1;
            const unsigned char* cb = reinterpret_cast<const unsigned char*>(codes + vr * (B * D / 32)) + B * i;
            if constexpr (B == 4) t.f[r] = *reinterpret_cast<const uint32_t*>(cb);
            else if constexpr (B == 2) t.f[r] = *reinterpret_cast<const uint16_t*>(cb);
            else if constexpr (B == 3) t.f[r] = (uint32_t)cb[0] | ((uint32_t)cb[1] << 8) | ((uint32_t)cb[2] << 16);
            else t.f[r] = cb[0];
            t.nv[r] = norm[vr];
            t.rn[r] = QJL ? rnorm[vr] : (uint16_t)0;
        }
    };
    const int64_t pstep = (int64_t)gridDim.x * (kWavesPerBlock * NV);
    In cur;
    if ((int64_t)blockIdx.x * (kWavesPerBlock * NV) + (int64_t)wid * NV < n)
        fetch((int64_t)blockIdx.x * (kWavesPerBlock * NV) + (int64_t)wid * NV, cur);
    for (int64_t base = (int64_t)blockIdx.x * (kWavesPerBlock * NV); base < n; base += pstep) {
        const int64_t vb = base + (int64_t)wid * NV;
        if (vb >= n) continue;  // whole waves; no block synchronisation below
        In nxt = cur;
        if (vb + pstep < n) fetch(vb + pstep, nxt);
        const uint32_t swa[4] = {cur.sw[0], cur.sw[1], cur.sw[2], cur.sw[3]};
        float4_t acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < (QJL ? KS : 0); ++ks) {
            const half8_t a = __builtin_bit_cast(half8_t, slut[(swa[ks] >> (8 * q)) & 0xFFu]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, sfr[(ks * NT + nt) * 64 + lane], acc[nt], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t v = vb + 4 * q + r;
            const bool ok = v < n;
            const uint32_t f = cur.f[r];  // group i's codes, code t at bit B t
            const float g = QJL ? h2f(cur.rn[r]) * kap : 0.f;
            float a[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                a[nt] = ctab[(f >> (B * nt)) & (L - 1)];
                if constexpr (QJL) a[nt] += g * acc[nt][r];
            }
#pragma unroll
            for (int h = 1; h < NT; h <<= 1)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    if (!(nt & h)) {
                        const float x0 = a[nt], x1 = a[nt + h];
                        a[nt] = x0 + x1;
                        a[nt + h] = x0 - x1;
                    }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                a[nt] = lane_bfly<1>(a[nt], sm[0]);
                a[nt] = lane_bfly<2>(a[nt], sm[1]);
                a[nt] = lane_bfly<4>(a[nt], sm[2]);
                a[nt] = lane_bfly<8>(a[nt], sm[3]);
            }
            const float sc = h2f(cur.nv[r]) * isd;
            if (ok) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float o = flip(a[nt], ((dmask >> nt) & 1u) << 31) * sc;
                    const int64_t e = v * D + 16 * nt + i;
                    if constexpr (F16OUT) static_cast<uint16_t*>(out)[e] = f2h(o);
                    else static_cast<float*>(out)[e] = o;
                }
            }
        }
        cur = nxt;
    }
}

int grid_for(int64_t units, int per_block, int cap = 65536)
{
    int64_t b = (units + per_block - 1) / per_block;
    return (int)(b < cap ? b : cap);
}

int device_status(const char* who)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, "%s: %s", who, hipGetErrorString(e));
    return TQ_OK;
}

// ---------------------------------------------------------------- dispatch

template <int D, int B, bool QJL>
void quantize_d_b(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* o,
                  hipStream_t s)
{
    dim3 block(256);
    if constexpr (D <= 128) {
        if (D == 128 && dtype == TQ_F16) {
            launch_quantize_m128(q, x, n, o, s);
        } else if (dtype == TQ_F16) {
            auto kern = k_quantize_quad<D, B, QJL, true>;
            hipLaunchKernelGGL(kern, dim3(resident_grid(kern, kWavesPerBlock * 16, n)), block, 0, s, x, n,
                               q->centroids, q->boundaries, q->diag_signs, q->S, o->codes, o->signs, o->norm,
                               o->rnorm);
        } else {
            auto kern = k_quantize_quad<D, B, QJL, false>;
            hipLaunchKernelGGL(kern, dim3(resident_grid(kern, kWavesPerBlock * 16, n)), block, 0, s, x, n,
                               q->centroids, q->boundaries, q->diag_signs, q->S, o->codes, o->signs, o->norm,
                               o->rnorm);
        }
    } else {
        static_assert(D == 256, "d = 256 kernel");
        if constexpr (QJL) launch_quantize_keys_d256(q, x, dtype, n, o, s);
        else launch_quantize_values_d256(q, x, dtype, n, o, s);
    }
}

template <int D>
void quantize_d(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* o,
                hipStream_t s)
{
    const bool qjl = q->qjl_m != 0;
    switch (q->mse_bits) {
        case 1: qjl ? quantize_d_b<D, 1, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 1, false>(q, x, dtype, n, o, s); break;
        case 2: qjl ? quantize_d_b<D, 2, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 2, false>(q, x, dtype, n, o, s); break;
        case 3: qjl ? quantize_d_b<D, 3, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 3, false>(q, x, dtype, n, o, s); break;
        default: qjl ? quantize_d_b<D, 4, true>(q, x, dtype, n, o, s) : quantize_d_b<D, 4, false>(q, x, dtype, n, o, s); break;
    }
}

template <int D>
void qprep_d(const tq_quantizer* q, const void* queries, int dtype, int64_t nq, float* qr, float* p,
             hipStream_t s)
{
    dim3 grid(grid_for(nq, kWavesPerBlock)), block(256);
    const bool qjl = q->qjl_m != 0;
    if (dtype == TQ_F16) {
        if (qjl) hipLaunchKernelGGL((k_qprep<D, true, true>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
        else hipLaunchKernelGGL((k_qprep<D, false, true>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
    } else {
        if (qjl) hipLaunchKernelGGL((k_qprep<D, true, false>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
        else hipLaunchKernelGGL((k_qprep<D, false, false>), grid, block, 0, s, queries, nq, q->diag_signs, q->S, qr, p);
    }
}

template <int D, int B, bool QJL>
void dequant_d_b(const tq_quantizer* q, const tq_packed* in, int64_t n, void* out, int dtype, hipStream_t s)
{
    dim3 grid(grid_for(n, kWavesPerBlock)), block(256);
    if constexpr (D == 128) {
        if (dtype == TQ_F16) {
            auto kern = k_dequantize128<B, QJL, true>;
            hipLaunchKernelGGL(kern, dim3(resident_grid(kern, kWavesPerBlock * 16, n)), block, 0, s, in->codes,
                               in->signs, in->norm, in->rnorm, n, q->centroids, q->diag_signs, q->S, out);
        } else {
            auto kern = k_dequantize128<B, QJL, false>;
            hipLaunchKernelGGL(kern, dim3(resident_grid(kern, kWavesPerBlock * 16, n)), block, 0, s, in->codes,
                               in->signs, in->norm, in->rnorm, n, q->centroids, q->diag_signs, q->S, out);
        }
        return;
    }
    if (dtype == TQ_F16)
        hipLaunchKernelGGL((k_dequantize<D, B, QJL, true>), grid, block, 0, s, in->codes, in->signs,
                           in->norm, in->rnorm, n, q->centroids, q->diag_signs, q->S, out);
    else
        hipLaunchKernelGGL((k_dequantize<D, B, QJL, false>), grid, block, 0, s, in->codes, in->signs,
                           in->norm, in->rnorm, n, q->centroids, q->diag_signs, q->S, out);
}

template <int D>
void dequant_d(const tq_quantizer* q, const tq_packed* in, int64_t n, int qjl, void* out, int dtype,
               hipStream_t s)
{
    switch (q->mse_bits) {
        case 1: qjl ? dequant_d_b<D, 1, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 1, false>(q, in, n, out, dtype, s); break;
        case 2: qjl ? dequant_d_b<D, 2, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 2, false>(q, in, n, out, dtype, s); break;
        case 3: qjl ? dequant_d_b<D, 3, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 3, false>(q, in, n, out, dtype, s); break;
        default: qjl ? dequant_d_b<D, 4, true>(q, in, n, out, dtype, s) : dequant_d_b<D, 4, false>(q, in, n, out, dtype, s); break;
    }
}

}  // namespace

int launch_quantize(const tq_quantizer* q, const void* x, int dtype, int64_t n, const tq_packed* out,
                    hipStream_t s)
{
    if (q->mse_bits > 4) {
        // widths 5..8: the MFMA quantizer for d = 128 fp16 input, else the wide-code kernel
        if (q->d != 128 || dtype != TQ_F16) return launch_quantize_wide(q, x, dtype, n, out, s);
        launch_quantize_m128(q, x, n, out, s);
        return device_status("tq_quantize");
    }
    switch (q->d) {
        case 64: quantize_d<64>(q, x, dtype, n, out, s); break;
        case 128: quantize_d<128>(q, x, dtype, n, out, s); break;
        default: quantize_d<256>(q, x, dtype, n, out, s); break;
    }
    return device_status("tq_quantize");
}

int launch_qprep(const tq_quantizer* q, const void* queries, int dtype, int64_t nq, float* qr, float* p,
                 hipStream_t s)
{
    switch (q->d) {
        case 64: qprep_d<64>(q, queries, dtype, nq, qr, p, s); break;
        case 128: qprep_d<128>(q, queries, dtype, nq, qr, p, s); break;
        default: qprep_d<256>(q, queries, dtype, nq, qr, p, s); break;
    }
    return device_status("query preparation");
}

int launch_dequantize(const tq_quantizer* q, const tq_packed* in, int64_t n, int include_qjl, void* out,
                      int dtype, hipStream_t s)
{
    if (q->mse_bits > 4) return launch_dequantize_wide(q, in, n, include_qjl, out, dtype, s);
    switch (q->d) {
        case 64: dequant_d<64>(q, in, n, include_qjl, out, dtype, s); break;
        case 128: dequant_d<128>(q, in, n, include_qjl, out, dtype, s); break;
        default: dequant_d<256>(q, in, n, include_qjl, out, dtype, s); break;
    }
    return device_status("tq_dequantize");
}

}  // namespace tq
