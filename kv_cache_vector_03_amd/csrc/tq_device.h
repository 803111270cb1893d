// Device helpers shared by the kernels: fp16 access, wave reductions and the
// wave-layout Walsh-Hadamard transform.
#ifndef TQ_DEVICE_H
#define TQ_DEVICE_H

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tq {

constexpr int kWave = 64;

template <int V>
struct ic {
    static constexpr int value = V;
};

// compile-time loop: f(ic<I>{}) for I in [B, E)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

// Block barrier for LDS traffic only: waits for this wave's LDS operations and
// meets the other waves, leaving global loads in flight (a __syncthreads fence
// would also wait for those).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

template <bool F16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i)
{
    if constexpr (F16) return h2f(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// Natural-order (Sylvester) Walsh-Hadamard transform, unnormalised, of a
// d = 64 R vector held across one wave: lane l, slot r holds coordinate
// 64 r + l. Butterflies on the slot bits run in registers; the six lane bits
// use cross-lane exchanges. Every butterfly maps (a, b) -> (a + b, a - b)
// with a the element whose index bit is 0, so the result is H x exactly as
// H_ij = (-1)^popcount(i & j) defines it. T is float or double.
template <int R, typename T>
__device__ __forceinline__ void fwht_wave(T (&v)[R], int lane)
{
#pragma unroll
    for (int h = 1; h < R; h <<= 1)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (!(r & h)) {
                T a = v[r], b = v[r + h];
                v[r] = a + b;
                v[r + h] = a - b;
            }
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            T p = __shfl_xor(v[r], m);
            v[r] = (lane & m) ? (p - v[r]) : (v[r] + p);
        }
}

// sign flips of the random diagonal for the coordinates a lane holds
template <int R>
__device__ __forceinline__ void load_diag(const uint32_t* diag, int lane, uint32_t (&mask)[R])
{
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int c = 64 * r + lane;
        mask[r] = ((diag[c >> 5] >> (c & 31)) & 1u) << 31;
    }
}

__device__ __forceinline__ float flip(float x, uint32_t m) { return __uint_as_float(__float_as_uint(x) ^ m); }

// (own value, value of lane l ^ M) for M = 16, 32: a permlane swap of a
// register with itself returns (row pair's even row, odd row) in every lane
template <int M>
__device__ __forceinline__ void row_pair(float v, float& even, float& odd)
{
    const uint32_t u = __float_as_uint(v);
    if constexpr (M == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        even = __uint_as_float(p[0]);
        odd = __uint_as_float(p[1]);
    } else {
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        even = __uint_as_float(p[0]);
        odd = __uint_as_float(p[1]);
    }
}

// max of two floats that are never NaN, without the compiler's NaN quieting
// of each operand (two extra instructions per fmaxf on cross-lane values)
__device__ __forceinline__ float max2nn(float a, float b)
{
    float d;
    asm("v_max_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four rows of 16 lanes), on
// permlane swaps instead of LDS round trips; never-NaN values
__device__ __forceinline__ float rows_max(float v)
{
    float e, o;
    row_pair<16>(v, e, o);
    v = max2nn(e, o);
    row_pair<32>(v, e, o);
    return max2nn(e, o);
}

// sum over lanes l, l ^ 16, l ^ 32, l ^ 48, on permlane swaps; every lane adds
// the same two values in the same order, so all four get the same sum
__device__ __forceinline__ float rows_sum(float v)
{
    float e, o;
    row_pair<16>(v, e, o);
    v = e + o;
    row_pair<32>(v, e, o);
    return e + o;
}

// Value held by lane l ^ M (M = 1, 2, 4, 8) by DPP moves within 16-lane rows:
// quad permutations for 1 and 2, quad reversal (l ^ 3) then half-row mirror
// (l ^ 7) for 4, a rotation by 8 within the row for 8.
template <int M>
__device__ __forceinline__ float dpp_xor(float v)
{
    const int i = __float_as_int(v);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false));
    else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false));
    else if constexpr (M == 4)
        return __int_as_float(
            __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(i, 0x1B, 0xF, 0xF, false), 0x141, 0xF, 0xF, false));
    else return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, false));
}

// Butterfly on lane bit M: a + b where the lane's bit is clear, a - b where it
// is set, a being the value of the lane with the bit clear -- the same
// operands and roundings as fwht_wave. sm = sign bit where the lane bit is set.
template <int M>
__device__ __forceinline__ float lane_bfly(float v, uint32_t sm)
{
    if constexpr (M <= 8) {
        return dpp_xor<M>(v) + flip(v, sm);  // p + v, or p - v with p the bit-clear lane's value
    } else {
        float e, o;
        row_pair<M>(v, e, o);
        return e + flip(o, sm);
    }
}

// Sum over the wave in the order of wave_sum (lane bits 5, 4, .., 0), so the
// result is the same to the bit.
__device__ __forceinline__ float wave_sum_dpp(float v)
{
    float e, o;
    row_pair<32>(v, e, o);
    v = e + o;
    row_pair<16>(v, e, o);
    v = e + o;
    v += dpp_xor<8>(v);
    v += dpp_xor<4>(v);
    v += dpp_xor<2>(v);
    v += dpp_xor<1>(v);
    return v;
}

// Wave max in the lane-bit order 5, 4, .., 0 on permlane swaps and DPP.
__device__ __forceinline__ float wave_max_dpp(float v)
{
    float e, o;
    row_pair<32>(v, e, o);
    v = fmaxf(e, o);
    row_pair<16>(v, e, o);
    v = fmaxf(e, o);
    v = fmaxf(v, dpp_xor<8>(v));
    v = fmaxf(v, dpp_xor<4>(v));
    v = fmaxf(v, dpp_xor<2>(v));
    return fmaxf(v, dpp_xor<1>(v));
}

// fwht_wave with the lane stages on DPP and permlane swaps instead of LDS
// exchanges: the same butterflies, operands and roundings, in the same order
// (register stages, then lane bits 0 .. 5).
template <int R>
__device__ __forceinline__ void fwht_wave_dpp(float (&v)[R], int lane)
{
#pragma unroll
    for (int h = 1; h < R; h <<= 1)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (!(r & h)) {
                const float a = v[r], b = v[r + h];
                v[r] = a + b;
                v[r + h] = a - b;
            }
    static_for<0, 6>([&](auto bb) {
        constexpr int M = 1 << decltype(bb)::value;
        const uint32_t sm = (lane & M) ? 0x80000000u : 0u;
#pragma unroll
        for (int r = 0; r < R; ++r) v[r] = lane_bfly<M>(v[r], sm);
    });
}


// c[k] for a small register table without dynamic register indexing
template <int L>
__device__ __forceinline__ float pick(const float (&c)[L], int k)
{
    float v = c[0];
#pragma unroll
    for (int l = 1; l < L; ++l) v = (k == l) ? c[l] : v;
    return v;
}

// Group-major packed layout: the D coordinates form D/8 groups, group c
// holding coordinates c + (D/8) t for t = 0..7. Code bit p of coordinate i
// sits at bit code_bit(i, p) of the vector's little-endian code stream; the
// sign of projection row j at bit sign_bit(j) of the sign stream.
template <int D, int B>
__host__ __device__ constexpr int code_bit(int i, int p)
{
    return 8 * B * (i % (D / 8)) + B * (i / (D / 8)) + p;
}

template <int M>
__host__ __device__ constexpr int sign_bit(int j)
{
    return 8 * (j % (M / 8)) + j / (M / 8);
}

// Replace lane LN of a VGPR with a wave-uniform value (v_writelane_b32 with an
// immediate lane select; it ignores EXEC and leaves the other lanes untouched).
template <int LN>
__device__ __forceinline__ uint32_t write_lane(uint32_t dst, uint32_t val)
{
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(dst) : "s"(val), "n"(LN));
    return dst;
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// sqrt(pi/2)
constexpr float kSqrtHalfPi = 1.2533141373155003f;

int device_cus();

// Grid for a grid-stride kernel of `threads`-thread blocks: enough blocks to
// cover n units (units_per_block each), but no more than fit on the device at
// once, so every block is resident and the work divides evenly.
int resident_blocks(const void* kern, int threads = 256);

template <typename Kern>
int resident_grid(Kern kern, int64_t units_per_block, int64_t n, int threads = 256)
{
    const int cap = resident_blocks(reinterpret_cast<const void*>(kern), threads);
    int64_t want = (n + units_per_block - 1) / units_per_block;
    if (want < 1) want = 1;
    return (int)(want < cap ? want : cap);
}

}  // namespace tq

#endif
