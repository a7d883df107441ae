// top_p.hip -- top-p (nucleus) masking of logits rows, for gfx950.
//
// "Beam 1.0 DFlash2" model card, "Evaluation": sampled runs use temperature
// 0.7 and top-p 0.99.  The nucleus of softmax(z/T) is the shortest prefix of
// the row in the order (logit descending, index ascending) whose probability
// reaches top_p.  Entries outside it are set to -inf, so that softmax(z/T) of
// the masked row is the renormalised truncation: the unchanged draws and
// verification then sample and verify against the truncated distributions
// ("DFlash vs DFlash 2", "The problem: one expensive token at a time": the
// committed tokens follow the target's distribution, here the truncated one).
//
// One 512-thread workgroup per row (two per CU); the row is streamed a few times:
//   A  row maximum m;
//   B  a histogram of the entries' masses over 4,096 bins of
//      x = (m - z) log2(e)/T (64 bins per unit of log2 weight; the last bin
//      takes everything below 2^-64 of the maximum).  Bins are monotone in z,
//      so the bin where the cumulative mass (from the top) reaches top_p of the
//      total holds the nucleus boundary.  Masses are fixed point (2^-40 of the
//      maximum's weight) added with integer atomics: exact and order free;
//   C  the entries of that bin are gathered into LDS (if there are more than
//      2,048, histograms over successive 12-bit digits of the 64-bit rank key
//      (ordered logit, inverted index), one pass each, narrow the set and it is
//      gathered again) and the boundary entry is found by counting, for every
//      gathered entry, the mass of the gathered entries ranked at or ahead of it;
//   D  every entry ranked after the boundary is written as -inf.
#include <cmath>

#include "common.hpp"

namespace dfl {
namespace {

constexpr int kPThreads = 512;
constexpr int kPBins = 4096;
constexpr float kPBinsPerUnit = 64.f;   // bins per unit of log2 weight below the maximum
constexpr int kPCap = 2048;             // entries gathered for the final count
constexpr int kPInFlight = 8;           // 16-byte loads per thread in flight in a pass over the row
constexpr float kFix = 1099511627776.f; // 2^40: fixed-point scale of a weight
constexpr int kMaxTopPVocab = 1 << 24;   // rows shorter than this cannot overflow the 64-bit sums

struct TopPArgs {
    const float* z;
    float* out;
    int32_t* kept;
    int V;
    float c2;     // log2(e) / T
    double top_p;
};

// logit -> unsigned key with the same order; (key << 32) | ~index: the rank key,
// larger = ranked ahead (logit descending, index ascending), unique per entry
__device__ __forceinline__ uint32_t ord_key(float z) {
    const uint32_t b = __float_as_uint(z);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t rank_key(float z, int v) {
    return ((uint64_t)ord_key(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
}
__device__ __forceinline__ uint64_t weight_fx(float z, float m, float c2) {
    const float w = fast_exp2((z - m) * c2);  // in [0, 1]
    return (uint64_t)(w * kFix);
}
__device__ __forceinline__ int bin_of(float z, float m, float c2) {
    const float x = (m - z) * c2 * kPBinsPerUnit;
    return x < (float)(kPBins - 1) ? (int)x : kPBins - 1;  // -inf and the far tail: last bin
}

template <class T, class Op>
__device__ __forceinline__ T block_reduce(T v, T* red, Op op) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = op(v, __shfl_xor(v, o));
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    T r = red[0];
    for (int w = 1; w < kPThreads / 64; ++w) r = op(r, red[w]);
    return r;
}

__global__ void __launch_bounds__(kPThreads) top_p_kernel(TopPArgs a) {
    __shared__ unsigned long long h_mass[kPBins];
    __shared__ unsigned long long g_key[kPCap];
    __shared__ unsigned long long g_w[kPCap];  // also the digit counts while narrowing
    __shared__ float red_f[kPThreads / 64];
    __shared__ unsigned long long red_u[kPThreads / 64];
    __shared__ unsigned long long s_before, s_prefix;
    __shared__ int s_bin, s_n;
    static_assert(sizeof(g_w) >= kPBins * sizeof(unsigned int), "digit counts fit");
    unsigned int* const h_cnt = reinterpret_cast<unsigned int*>(g_w);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t R = blockIdx.x;
    const float* z = a.z + R * a.V;
    float* out = a.out + R * a.V;
    const int V = a.V;
    const float c2 = a.c2;
    const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(out) & 15) == 0;
    // fn(logit, index) for every entry of the row (16-byte loads when aligned)
    auto each = [&](auto&& fn) {
        if (vec) {
            // kPInFlight 16-byte loads in flight per thread before any is used
            // (one workgroup streams a whole row: its passes are bound by the
            // loads it keeps in flight)
            const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
            const int V4 = V >> 2;
            int i = tid;
            for (; i + (kPInFlight - 1) * kPThreads < V4; i += kPInFlight * kPThreads) {
                f32x4 q[kPInFlight];
#pragma unroll
                for (int u = 0; u < kPInFlight; ++u) q[u] = z4[i + u * kPThreads];
#pragma unroll
                for (int u = 0; u < kPInFlight; ++u) {
                    const int b = 4 * (i + u * kPThreads);
                    fn(q[u][0], b); fn(q[u][1], b + 1); fn(q[u][2], b + 2); fn(q[u][3], b + 3);
                }
            }
            for (; i < V4; i += kPThreads) {
                const f32x4 q = z4[i];
                fn(q[0], 4 * i); fn(q[1], 4 * i + 1); fn(q[2], 4 * i + 2); fn(q[3], 4 * i + 3);
            }
        } else {
            for (int v = tid; v < V; v += kPThreads) fn(z[v], v);
        }
    };
    auto block_sum_u = [&](unsigned long long v) {
        return block_reduce(v, red_u, [](unsigned long long x, unsigned long long y) { return x + y; });
    };
    // exclusive prefix over threads of `mine` (ascending thread order)
    auto thread_prefix = [&](unsigned long long mine) {
        unsigned long long incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const unsigned long long t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        __syncthreads();
        if (lane == 63) red_u[wave] = incl;
        __syncthreads();
        unsigned long long before = incl - mine;
        for (int w = 0; w < wave; ++w) before += red_u[w];
        return before;
    };

    // A: the row maximum
    float m = -INFINITY;
    each([&](float x, int) { m = fmaxf(m, x); });
    m = block_reduce(m, red_f, [](float x, float y) { return fmaxf(x, y); });

    unsigned long long cut = 0;  // rank key of the last kept entry (0: keep everything)
    if (a.top_p < 1.0 && m != -INFINITY) {
        // B: bin masses
        for (int b = tid; b < kPBins; b += kPThreads) h_mass[b] = 0;
        __syncthreads();
        each([&](float x, int) {
            atomicAdd(&h_mass[bin_of(x, m, c2)], (unsigned long long)weight_fx(x, m, c2));
        });
        __syncthreads();
        // the bin where the cumulative mass from the top reaches top_p of the total
        constexpr int kPer = kPBins / kPThreads;
        unsigned long long mine = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) mine += h_mass[tid * kPer + i];
        const unsigned long long total = block_sum_u(mine);
        const unsigned long long target = (unsigned long long)ceil(a.top_p * (double)total);
        if (tid == 0) { s_bin = kPBins - 1; s_before = 0; s_prefix = 0; }
        const unsigned long long before = thread_prefix(mine);
        if (before < target && before + mine >= target) {
            unsigned long long c = before;
            for (int i = 0; i < kPer; ++i) {
                const int b = tid * kPer + i;
                if (c + h_mass[b] >= target) { s_bin = b; s_before = c; break; }
                c += h_mass[b];
            }
        }
        __syncthreads();
        const int bstar = s_bin;
        // the candidate set: bin bstar and, after `level` narrowing steps, the
        // rank keys whose top 12*level bits equal `prefix`
        auto in_set = [&](uint64_t key, int b, int level, unsigned long long prefix) {
            if (b != bstar) return false;
            if (level == 0) return true;
            const int sh = 64 - 12 * level;
            return sh <= 0 ? key == prefix : (key >> sh) == (prefix >> sh);
        };
        int level = 0;
        unsigned long long prefix = 0;
        // C: gather the set (every pass counts it; entries beyond kPCap are dropped)
        auto gather = [&]() {
            __syncthreads();
            if (tid == 0) s_n = 0;
            __syncthreads();
            each([&](float x, int v) {
                const uint64_t key = rank_key(x, v);
                if (in_set(key, bin_of(x, m, c2), level, prefix)) {
                    const int at = atomicAdd(&s_n, 1);
                    if (at < kPCap) {
                        g_key[at] = key;
                        g_w[at] = weight_fx(x, m, c2);
                    }
                }
            });
            __syncthreads();
            return s_n;
        };
        int count = gather();
        // more than kPCap: narrow the set, 12 bits of the rank key at a time, then gather again
        while (count > kPCap && level < 6) {  // 6 digits cover the 64-bit key
            const int sh = 64 - 12 * (level + 1);  // digit = bits [sh, sh + 12)
            __syncthreads();
            for (int b = tid; b < kPBins; b += kPThreads) { h_mass[b] = 0; h_cnt[b] = 0; }
            __syncthreads();
            each([&](float x, int v) {
                const uint64_t key = rank_key(x, v);
                if (!in_set(key, bin_of(x, m, c2), level, prefix)) return;
                const int d = sh >= 0 ? (int)((key >> sh) & 0xFFF) : (int)((key << -sh) & 0xFFF);
                atomicAdd(&h_mass[kPBins - 1 - d], (unsigned long long)weight_fx(x, m, c2));
                atomicAdd(&h_cnt[kPBins - 1 - d], 1u);
            });
            __syncthreads();
            const unsigned long long sb = s_before;  // read by every thread before the winner rewrites it
            // digits in descending order = bins in ascending order
            unsigned long long mine2 = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) mine2 += h_mass[tid * kPer + i];
            const unsigned long long bef2 = sb + thread_prefix(mine2);
            if (bef2 < target && bef2 + mine2 >= target) {
                unsigned long long c = bef2;
                for (int i = 0; i < kPer; ++i) {
                    const int b = tid * kPer + i;
                    if (c + h_mass[b] >= target) {
                        const uint64_t d = (uint64_t)(kPBins - 1 - b);
                        s_prefix = sh >= 0 ? (prefix | (d << sh)) : (prefix | (d >> -sh));
                        s_before = c;
                        break;
                    }
                    c += h_mass[b];
                }
            }
            __syncthreads();
            prefix = s_prefix;
            ++level;
            count = gather();
        }
        // the entry where the mass reaches the target: for every gathered entry,
        // the mass of the gathered entries ranked at or ahead of it
        const int n = min(count, kPCap);
        const unsigned long long need = target - s_before;  // > 0
        unsigned long long best = 0;
        for (int i = tid; i < n; i += kPThreads) {
            const uint64_t ki = g_key[i];
            unsigned long long ge = 0;
#pragma unroll 8
            for (int j = 0; j < n; ++j) ge += g_key[j] >= ki ? g_w[j] : 0ull;
            if (ge >= need && ki > best) best = ki;
        }
        cut = block_reduce(best, red_u, [](unsigned long long x, unsigned long long y) { return x > y ? x : y; });
    }
    // D: mask everything ranked after the cut
    unsigned int kept = 0;
    const bool inplace = out == z;
    if (vec) {
        const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
        f32x4* o4 = reinterpret_cast<f32x4*>(out);
        const int V4 = V >> 2;
        auto mask4 = [&](f32x4 q, int i) {
            bool any_masked = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool keep = cut == 0 || rank_key(q[e], 4 * i + e) >= cut;
                kept += keep ? 1u : 0u;
                any_masked |= !keep;
                q[e] = keep ? q[e] : -INFINITY;
            }
            if (!inplace || any_masked) o4[i] = q;
        };
        int i = tid;
        for (; i + (kPInFlight - 1) * kPThreads < V4; i += kPInFlight * kPThreads) {
            f32x4 q[kPInFlight];
#pragma unroll
            for (int u = 0; u < kPInFlight; ++u) q[u] = z4[i + u * kPThreads];
#pragma unroll
            for (int u = 0; u < kPInFlight; ++u) mask4(q[u], i + u * kPThreads);
        }
        for (; i < V4; i += kPThreads) mask4(z4[i], i);
    } else {
        for (int v = tid; v < V; v += kPThreads) {
            const float x = z[v];
            const bool keep = cut == 0 || rank_key(x, v) >= cut;
            kept += keep ? 1u : 0u;
            if (!keep) out[v] = -INFINITY;
            else if (!inplace) out[v] = x;
        }
    }
    if (a.kept) {
        kept = block_reduce(kept, (unsigned int*)red_f, [](unsigned int x, unsigned int y) { return x + y; });
        if (tid == 0) a.kept[R] = (int32_t)kept;
    }
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" int dflash_top_p_mask(const float* logits, float* out, int32_t* kept, int rows, int vocab,
                                 float temperature, float top_p, void* stream) {
    if (rows < 0 || vocab < 1) return DFLASH_ERR_SHAPE;
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return DFLASH_ERR_SHAPE;
    if (!(top_p > 0.f) || !(top_p <= 1.f)) return DFLASH_ERR_SHAPE;
    if (rows == 0) return DFLASH_OK;
    if (!logits || !out) return DFLASH_ERR_NULL;
    // every weight is at most 2^40 in fixed point, so a row's 64-bit total
    // cannot overflow below 2^24 entries
    if (vocab >= kMaxTopPVocab || rows > kMaxRowsPerCall) return DFLASH_ERR_UNSUPPORTED;
    TopPArgs a{logits, out, kept, vocab, (float)(1.4426950408889634 / (double)temperature), (double)top_p};
    hipLaunchKernelGGL(top_p_kernel, dim3(rows), dim3(kPThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return launch_status();
}
