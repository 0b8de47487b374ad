// Device helpers shared by the gfx950 kernels of the tree-verification library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eagle {

constexpr int kWave = 64;

// Order-preserving map of an fp32 value to uint32 (larger float -> larger key).
// -0.0 is folded onto +0.0 so that equal floats give equal keys.
__device__ __forceinline__ uint32_t float_order_key(float x) {
    if (x == 0.0f) x = 0.0f;
    uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit key whose maximum is the larger logit, and among equal logits the lower
// token id.
__device__ __forceinline__ uint64_t logit_key(float z, uint32_t token) {
    return ((uint64_t)float_order_key(z) << 32) | (uint64_t)(0xFFFFFFFFu - token);
}
__device__ __forceinline__ uint32_t logit_key_token(uint64_t key) {
    return 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu);
}
// Inverse of float_order_key (-0.0 comes back as +0.0, which subtracts alike).
__device__ __forceinline__ float key_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}
// The logit a logit_key was made from.
__device__ __forceinline__ float logit_key_value(uint64_t key) { return key_float((uint32_t)(key >> 32)); }

// Wave reductions on the VALU: four DPP steps inside each 16-lane row (quad
// permutations for distances 1 and 2, the half-row and row mirrors to join 4- and
// 8-lane groups), then the row swaps permlane16 (l <-> l^16) and permlane32
// (l <-> l^32).  Each step combines a lane with a partner holding the other
// group's result, so every lane ends with the full reduction; a pair computes
// op(a, b) and op(b, a), which agree for max and for +.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
// Both values of a row swap: one is the lane's own, the other its partner's.
__device__ __forceinline__ void swap16_u64(uint64_t v, uint64_t& a, uint64_t& b) {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    a = ((uint64_t)hi[0] << 32) | lo[0];
    b = ((uint64_t)hi[1] << 32) | lo[1];
}
__device__ __forceinline__ void swap32_u64(uint64_t v, uint64_t& a, uint64_t& b) {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    a = ((uint64_t)hi[0] << 32) | lo[0];
    b = ((uint64_t)hi[1] << 32) | lo[1];
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    uint64_t p, a, b;
    p = dpp_u64<kDppXor1>(v); v = p > v ? p : v;
    p = dpp_u64<kDppXor2>(v); v = p > v ? p : v;
    p = dpp_u64<kDppHalfMirror>(v); v = p > v ? p : v;
    p = dpp_u64<kDppMirror>(v); v = p > v ? p : v;
    swap16_u64(v, a, b); v = a > b ? a : b;
    swap32_u64(v, a, b); v = a > b ? a : b;
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max(r[0], r[1]);
}

// Wave maximum of 64-bit keys by 32-bit steps: the maximum high word, then, if one
// lane alone holds it, that lane's key; otherwise the maximum low word among the
// lanes holding it.  Equal to wave_max_u64 for any keys.
__device__ __forceinline__ uint64_t wave_max_key_u64(uint64_t v) {
    const uint32_t hi = (uint32_t)(v >> 32);
    const uint32_t mhi = wave_max_u32(hi);
    const uint64_t holders = __ballot(hi == mhi);
    if (__builtin_popcountll(holders) == 1) {
        const int l = __builtin_ctzll(holders);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
        return ((uint64_t)mhi << 32) | lo;
    }
    const uint32_t mlo = wave_max_u32(hi == mhi ? (uint32_t)v : 0u);
    return ((uint64_t)mhi << 32) | mlo;
}

// e^x for x <= 0 in fp64, within about 1 ulp of the correctly rounded value (0 for
// x < -745).  Cody and Waite's reduction x = n ln2 + r, ln2 split in two parts (the
// first with 21 trailing zero bits, so n * hi is exact), |r| <= ln2 / 2; then the
// degree-13 Taylor polynomial of e^r (truncation error below 2e-17) by Horner, and
// the scale by 2^n.
__device__ __forceinline__ double exp_nonpos_f64(double x) {
    if (x < -745.0) return 0.0;
    const double n = __builtin_rint(x * 1.4426950408889634);
    const double r = __builtin_fma(-n, 1.90821492927058770002e-10, __builtin_fma(-n, 6.93147180369123816490e-01, x));
    double p = 1.0 / 6227020800.0;         // 1/13!
    p = __builtin_fma(p, r, 1.0 / 479001600.0);  // 1/12!
    p = __builtin_fma(p, r, 1.0 / 39916800.0);
    p = __builtin_fma(p, r, 1.0 / 3628800.0);
    p = __builtin_fma(p, r, 1.0 / 362880.0);
    p = __builtin_fma(p, r, 1.0 / 40320.0);
    p = __builtin_fma(p, r, 1.0 / 5040.0);
    p = __builtin_fma(p, r, 1.0 / 720.0);
    p = __builtin_fma(p, r, 1.0 / 120.0);
    p = __builtin_fma(p, r, 1.0 / 24.0);
    p = __builtin_fma(p, r, 1.0 / 6.0);
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = __builtin_fma(p, r, 1.0);
    return __builtin_ldexp(p, (int)n);
}

__device__ __forceinline__ double u64_f64(uint64_t u) { return __longlong_as_double((long long)u); }
__device__ __forceinline__ uint64_t f64_u64(double d) { return (uint64_t)__double_as_longlong(d); }

__device__ __forceinline__ double wave_sum_f64(double v) {
    uint64_t a, b;
    v += u64_f64(dpp_u64<kDppXor1>(f64_u64(v)));
    v += u64_f64(dpp_u64<kDppXor2>(f64_u64(v)));
    v += u64_f64(dpp_u64<kDppHalfMirror>(f64_u64(v)));
    v += u64_f64(dpp_u64<kDppMirror>(f64_u64(v)));
    swap16_u64(f64_u64(v), a, b); v = u64_f64(a) + u64_f64(b);
    swap32_u64(f64_u64(v), a, b); v = u64_f64(a) + u64_f64(b);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v))));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
    v += __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v)));
    v += __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v)));
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Block-wide sum of one double per thread; every thread receives the total.
// `scratch` needs blockDim.x / 64 doubles of LDS.  Contains __syncthreads.
__device__ __forceinline__ double block_sum_f64(double v, double* scratch) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    v = wave_sum_f64(v);
    if (lane == 0) scratch[wid] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < nw; ++w) t += scratch[w];
    __syncthreads();
    return t;
}

// In-place bitonic sort of P (power of two) uint64 keys in LDS into DESCENDING
// order, by all threads of the block.  Ends with __syncthreads.
__device__ __forceinline__ void lds_bitonic_sort_desc(uint64_t* keys, int P) {
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (P >> 1); i += blockDim.x) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool desc = (lo & size) == 0;
                const uint64_t a = keys[lo], b = keys[hi];
                if ((a < b) == desc) { keys[lo] = b; keys[hi] = a; }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): the 4x32 S-box with its two
// published multipliers, the key bumped by the two Weyl constants between the
// ten rounds.
// ---------------------------------------------------------------------------
struct Philox4x32 {
    uint32_t c0, c1, c2, c3;
};

__device__ __forceinline__ Philox4x32 philox4x32_10(Philox4x32 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint64_t a = (uint64_t)0xD2511F53u * c.c0;
        const uint64_t b = (uint64_t)0xCD9E8D57u * c.c2;
        Philox4x32 n;
        n.c0 = (uint32_t)(b >> 32) ^ c.c1 ^ k0;
        n.c1 = (uint32_t)b;
        n.c2 = (uint32_t)(a >> 32) ^ c.c3 ^ k1;
        n.c3 = (uint32_t)a;
        c = n;
    }
    return c;
}

// Uniform in [0, 1) for one acceptance decision: key = the seed's two words,
// counter = (slot, tree row, sequence, low word of the step); 24 top bits of
// the first output word.
__device__ __forceinline__ double decision_uniform(uint64_t seed, uint64_t step, uint32_t seq,
                                                   uint32_t row, uint32_t slot) {
    Philox4x32 c{slot, row, seq, (uint32_t)step};
    Philox4x32 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    return (double)(o.c0 >> 8) * (1.0 / 16777216.0);
}

constexpr uint32_t kBonusSlot = 0xFFFFFFFFu;

// ---------------------------------------------------------------------------
// Rotary position encoding (half-split pairs).  The fp64 form: the pair (x, y)
// rotated by an angle with cosine cs and sine sn, each product rounded (no fused
// multiply-add), then rounded to fp32; bf16 storage rounds that to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_rotate_f64(double x, double y, double cs, double sn, float& xr, float& yr) {
#pragma clang fp contract(off)
    xr = (float)(x * cs - y * sn);
    yr = (float)(y * cs + x * sn);
}
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN stays a (quiet) NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
// The fp32 form used inside the attention kernel: cos and sin of pos * f, with
// f_turns = f / (2 pi) the frequency in turns per position; the angle is taken
// modulo one turn in fp64, and the hardware cosine and sine (which take turns)
// of the remaining fraction give fp32 values.
__device__ __forceinline__ void rope_cs_turns(int pos, double f_turns, float& c, float& s) {
    const double t = (double)pos * f_turns;
    const float fr = (float)(t - rint(t));  // in [-1/2, 1/2] turn
    c = __builtin_amdgcn_cosf(fr);
    s = __builtin_amdgcn_sinf(fr);
}

// Workgroup barrier that orders LDS traffic only: outstanding global loads and
// stores stay in flight (__syncthreads would also wait for every store to complete).
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace eagle
