// common.hpp -- device and host helpers shared by the gfx950 kernels of
// libdflash.so.  Nothing here is shared with the CPU reference.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <initializer_list>

#include "dflash.h"

namespace dfl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ----------------------------------------------------------------- numbers
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// two floats -> packed bf16 pair (lo = a), round to nearest even (hardware cvt)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;

// Cache-policy operand of global loads (gfx950 encoding: 1 = sc0, 2 = nt,
// 16 = sc1).  Streams read once per step (context K/V rings, logits, GEMM
// weights) are loaded non-temporal: measured on MI355X, HBM-to-LDS streaming
// of the 256 x 2 x 1 MB ring pattern runs at 6.9 TB/s with nt against
// 6.1 TB/s with the default policy, and nt weight tiles leave the fusion
// GEMM's re-read activation slice in L2.
constexpr int kLoadStream = 2;
constexpr int kLoadDefault = 0;

// ------------------------------------------------------------ wave helpers
// Cross-lane exchange without LDS round trips.  Within a row of 16 lanes, DPP
// moves (gfx9 controls: quad_perm [1,0,3,2] = lane ^ 1, quad_perm [2,3,0,1] =
// lane ^ 2, row_half_mirror = 7 - lane within 8, row_mirror = 15 - lane
// within 16) give each lane a partner whose partial result covers the other
// half of a growing group; v_permlane16_swap / v_permlane32_swap (gfx950)
// with both operands = v give each lane {v, v of lane l ^ 16 (resp. l ^ 32)}
// in some order.  Every combine used with them is symmetric, so all lanes
// end with bit-identical results.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const int lo = dpp_i<CTRL>((int)(unsigned)u), hi = dpp_i<CTRL>((int)(unsigned)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
// {v, partner's v} for partner = lane ^ 16 (W = 16) or lane ^ 32 (W = 32)
template <int W>
__device__ __forceinline__ void swap_pair(unsigned v, unsigned& r0, unsigned& r1) {
    if (W == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        r0 = r[0]; r1 = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        r0 = r[0]; r1 = r[1];
    }
}
template <int W>
__device__ __forceinline__ float swap_max(float v) {
    unsigned r0, r1;
    swap_pair<W>(__float_as_uint(v), r0, r1);
    return fmaxf(__uint_as_float(r0), __uint_as_float(r1));
}
template <int W>
__device__ __forceinline__ float swap_sum(float v) {
    unsigned r0, r1;
    swap_pair<W>(__float_as_uint(v), r0, r1);
    return __uint_as_float(r0) + __uint_as_float(r1);
}
template <int W>
__device__ __forceinline__ double swap_sum(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    unsigned l0, l1, h0, h1;
    swap_pair<W>((unsigned)u, l0, l1);
    swap_pair<W>((unsigned)(u >> 32), h0, h1);
    const double a = __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0));
    const double b = __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1));
    return a + b;
}
__device__ __forceinline__ float xor16_max(float v) { return swap_max<16>(v); }
__device__ __forceinline__ float xor32_max(float v) { return swap_max<32>(v); }
__device__ __forceinline__ float xor16_sum(float v) { return swap_sum<16>(v); }
__device__ __forceinline__ float xor32_sum(float v) { return swap_sum<32>(v); }

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return swap_max<32>(swap_max<16>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return swap_sum<32>(swap_sum<16>(v));
}
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_d<kDppXor1>(v);
    v += dpp_d<kDppXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppMirror>(v);
    return swap_sum<32>(swap_sum<16>(v));
}
// value of lane `src` (wave-uniform) broadcast to every lane
__device__ __forceinline__ int lane_value(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ double lane_value(double v, int src) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)u, src);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(u >> 32), src);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// inclusive prefix sum over the wave's lanes (lane order): DPP row_shr 1, 2, 4, 8
// within rows of 16, then row_bcast15 (rows 1, 3 add lane 15 of the row before)
// and row_bcast31 (rows 2, 3 add lane 31); lanes without a source add 0.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_scan_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWMASK, 0xF, false);
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_scan_d(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const int lo = dpp_scan_i<CTRL, ROWMASK>((int)(unsigned)u);
    const int hi = dpp_scan_i<CTRL, ROWMASK>((int)(unsigned)(u >> 32));
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ __forceinline__ double wave_inclusive_scan(double v) {
    v += dpp_scan_d<0x111, 0xF>(v);
    v += dpp_scan_d<0x112, 0xF>(v);
    v += dpp_scan_d<0x114, 0xF>(v);
    v += dpp_scan_d<0x118, 0xF>(v);
    v += dpp_scan_d<0x142, 0xA>(v);
    v += dpp_scan_d<0x143, 0xC>(v);
    return v;
}

// (value desc, index asc) ordering: true if (va, ia) ranks ahead of (vb, ib)
__device__ __forceinline__ bool ranks_ahead(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && (unsigned)ia < (unsigned)ib);
}

// wave-wide best (value desc, index asc); idx -1 = empty (ranks last via unsigned compare)
__device__ __forceinline__ void best_of(float& v, int& i, float ov, int oi) {
    if (ranks_ahead(ov, oi, v, i)) { v = ov; i = oi; }
}
template <int CTRL>
__device__ __forceinline__ void best_dpp(float& v, int& i) {
    best_of(v, i, dpp_f<CTRL>(v), dpp_i<CTRL>(i));
}
template <int W>
__device__ __forceinline__ void best_swap(float& v, int& i) {
    unsigned v0, v1, i0, i1;
    swap_pair<W>(__float_as_uint(v), v0, v1);
    swap_pair<W>((unsigned)i, i0, i1);
    v = __uint_as_float(v0);
    i = (int)i0;
    best_of(v, i, __uint_as_float(v1), (int)i1);
}
__device__ __forceinline__ void wave_best(float& v, int& i) {
    best_dpp<kDppXor1>(v, i);
    best_dpp<kDppXor2>(v, i);
    best_dpp<kDppHalfMirror>(v, i);
    best_dpp<kDppMirror>(v, i);
    best_swap<16>(v, i);
    best_swap<32>(v, i);
}

// ------------------------------------------------------------------ Philox
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// two-multiplier S-box over a 4x64-bit counter with a Weyl key schedule.
__device__ __forceinline__ void philox4x64_10(uint64_t& x0, uint64_t& x1, uint64_t& x2,
                                              uint64_t& x3, uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t hi0 = __umul64hi(M0, x0), lo0 = M0 * x0;
        const uint64_t hi1 = __umul64hi(M1, x2), lo1 = M1 * x2;
        const uint64_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
        x0 = n0; x1 = lo1; x2 = n2; x3 = lo0;
        k0 += W0; k1 += W1;
    }
}

// uniform in [0,1): key (seed, 0), counter (step, b, row, purpose), top 53 bits
__device__ __forceinline__ double philox_uniform(uint64_t seed, uint64_t step, uint64_t b,
                                                 uint64_t row, uint64_t purpose) {
    uint64_t x0 = step, x1 = b, x2 = row, x3 = purpose;
    philox4x64_10(x0, x1, x2, x3, seed, 0);
    return (double)(x0 >> 11) * 0x1.0p-53;
}

enum Purpose : uint64_t { kDraftDraw = 0, kAcceptTest = 1, kFinalDraw = 2 };

// ----------------------------------------------------------------- host side
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bump allocator over the caller's workspace (offsets only, no allocation).
struct Carve {
    size_t off = 0;
    template <class T>
    size_t take(size_t count) {
        const size_t at = align_up(off, 256);
        off = at + count * sizeof(T);
        return at;
    }
    size_t total() const { return align_up(off, 256); }
};

// Product of non-negative factors if it stays at or below `cap`, else -1; no
// intermediate product can overflow.  Shape checks use it so that every count
// the host derives from the caller's sizes fits the type it is computed in.
inline int64_t capped_product(int64_t cap, std::initializer_list<int64_t> factors) {
    int64_t p = 1;
    for (const int64_t x : factors) {
        if (x < 0 || (x != 0 && p > cap / x)) return -1;
        p *= x;
    }
    return p;
}

// Rows of one call for the kernels that give each row its own workgroup of up
// to 1,024 threads (twice that many rows in spec_verify's statistics launch):
// a launch counts its work-items in 32 bits.
constexpr int64_t kMaxRowsPerCall = 1 << 20;

// ------------------------------------------------------ device-data checks
// Compiled with DFLASH_DEVICE_CHECKS=1 (libdflash_checked.so), kernels record
// the device-data preconditions they find violated (DFLASH_VIOLATION_* bits)
// in a word per source file and GPU; dflash_violations ORs the files' words.
// A release build compiles the checks away.  The record is a vector-memory
// atomic OR, never a scalar store.
#ifndef DFLASH_DEVICE_CHECKS
#define DFLASH_DEVICE_CHECKS 0
#endif
// Host readers of each file's word (defined only with device checks).
int violations_attn(uint32_t* word, bool clear, hipStream_t st);
int violations_fuse(uint32_t* word, bool clear, hipStream_t st);
int violations_rows(uint32_t* word, bool clear, hipStream_t st);
int violations_select(uint32_t* word, bool clear, hipStream_t st);
#if DFLASH_DEVICE_CHECKS
#define DFL_VIOLATION_WORD(reader)                                                              \
    static __device__ unsigned int g_violations;                                                 \
    int reader(uint32_t* word, bool clear, hipStream_t st) {                                      \
        uint32_t v = 0;                                                                           \
        if (hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_violations), sizeof v, 0,                   \
                                     hipMemcpyDeviceToHost, st) != hipSuccess ||                  \
            hipStreamSynchronize(st) != hipSuccess)                                               \
            return DFLASH_ERR_HIP;                                                                \
        if (clear) {                                                                              \
            const uint32_t zero = 0;                                                              \
            if (hipMemcpyToSymbolAsync(HIP_SYMBOL(g_violations), &zero, sizeof zero, 0,           \
                                       hipMemcpyHostToDevice, st) != hipSuccess ||                \
                hipStreamSynchronize(st) != hipSuccess)                                           \
                return DFLASH_ERR_HIP;                                                            \
        }                                                                                         \
        *word |= v;                                                                               \
        return DFLASH_OK;                                                                         \
    }
#define DFL_VIOLATION(bit) atomicOr(&g_violations, (unsigned int)(bit))
#else
#define DFL_VIOLATION_WORD(reader)
#define DFL_VIOLATION(bit) ((void)0)
#endif

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

}  // namespace dfl
