// top_p.hip -- top-p (nucleus) truncation of logits rows, for gfx950.
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
// dflash_top_p_mask writes the masked rows; dflash_top_p_cut writes only the
// nucleus' last entry (logit, index) per row, which dflash_topk and
// spec_verify apply in their own row scans.
//
// One 1,024-thread workgroup per row; ordinary (cached) loads, eight 16-byte
// loads in flight per thread.  Weights are measured in log2 units below a
// reference `ref` >= every entry: y = (z - ref) log2(e)/T <= 0.
//   AB  ref = the maximum of a first sample of the row (every thread's first
//       loads) plus kHeadroom log2 units, and in one pass over the row: the
//       row maximum m and a mass histogram over 4,096 bins of -y (64 bins per
//       log2 unit; the last bin takes the far tail).  Bins are monotone in z,
//       so the bin where the cumulative mass (from the top) reaches top_p of
//       the total holds the nucleus boundary.  An entry weighs within a factor
//       2^(1/64) of its bin's top, so each adds 2^(y - top) in 31-bit fixed
//       point to its bin with a 64-bit integer atomic: exact and independent
//       of the order.  If an entry lies above ref after all (the sample
//       missed a far larger maximum), the histogram is rebuilt with ref = m.
//   C   the entries of the boundary bin are gathered into LDS (if there are
//       more than 2,048 of them, histograms over successive 12-bit digits of
//       the 64-bit rank key (ordered logit, inverted index), one pass each,
//       narrow the set and it is gathered again), counting the entries ranked
//       ahead of the set on the way; in LDS, a histogram over 4,096 sub-bins
//       of the boundary bin narrows the gathered set to the few entries
//       around the boundary, and each of those counts the mass of the ones
//       ranked at or ahead of it: the boundary is the first to reach top_p.
//   D   (masking only) every entry ranked after the boundary is written as
//       -inf.
// The nucleus size is the number of entries ranked ahead of the gathered set
// plus the gathered entries at or ahead of the boundary.
#include <cmath>

#include "common.hpp"

namespace dfl {
namespace {

constexpr int kPThreads = 1024;
constexpr int kPBins = 4096;            // bins of -y: 64 per log2 unit below ref
constexpr float kPBinsPerUnit = 64.f;
constexpr float kPSubPerUnit = 64.f * 4096.f;  // sub-bins of one bin: 4,096
constexpr int kPCap = 2048;             // entries gathered for the final count
constexpr int kPInFlight = 8;           // 16-byte loads per thread in flight in a pass over the row
constexpr float kLocalFix = 2147483648.f;  // 2^31: fixed point of a weight relative to its bin's top
constexpr float kHeadroom = 8.f;        // log2 units above the sample maximum
constexpr int kMaxTopPVocab = 1 << 24;  // keeps a bin's 64-bit sum (< 2^24 x 2^32) exact

struct TopPArgs {
    const float* z;
    float* out;                    // masked rows, or NULL
    dflash_nucleus_cut* cut_out;   // the cut, or NULL
    int32_t* kept;
    int V;
    float c2;     // log2(e) / T
    double top_p;
};

// logit -> unsigned key with the same order (-0.0 taken as +0.0, as the
// comparison of logits takes them); (key << 32) | ~index: the rank key,
// larger = ranked ahead (logit descending, index ascending), unique per entry
__device__ __forceinline__ uint32_t ord_key(float z) {
    uint32_t b = __float_as_uint(z);
    b = b == 0x80000000u ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint64_t rank_key(float z, int v) {
    return ((uint64_t)ord_key(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)v);
}

// Bins of the log2 weight below the reference.  Every entry goes through the
// same roundings (y, then its bin, then its weight within the bin), so the
// passes agree on bins and weights, and both are monotone in z.
struct Bins {
    float ref, c2, nrc;  // nrc = -(ref c2)
    __device__ __forceinline__ void set_ref(float r) {
        ref = r;
        nrc = -(r * c2);
    }
    __device__ __forceinline__ float y(float z) const { return fmaf(z, c2, nrc); }
    // floor(-64 y) in [0, 4095]: above ref 0, the far tail and -inf 4095
    __device__ __forceinline__ int bin(float y) const {
        return (int)__builtin_amdgcn_fmed3f(-y * kPBinsPerUnit, 0.f, (float)(kPBins - 1));
    }
    // log2 weight relative to the top of bin b: in (-1/64, 0] except in the tail bin
    __device__ __forceinline__ float local(float y, int b) const { return fmaf((float)b, 1.f / kPBinsPerUnit, y); }
    __device__ __forceinline__ uint32_t weight(float y, int b) const {
        return (uint32_t)(fast_exp2(local(y, b)) * kLocalFix);
    }
    // sub-bin of an entry of bin b: floor(-4096 * 64 local) in [0, 4095]
    __device__ __forceinline__ int sub(float y, int b) const {
        const float x = -local(y, b) * kPSubPerUnit;
        if (!(x > 0.f)) return 0;
        return x < (float)(kPBins - 1) ? (int)x : kPBins - 1;
    }
};

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

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
    __shared__ unsigned long long h_mass[kPBins];  // bin sums; later the final candidates
    __shared__ unsigned long long g_key[kPCap];
    __shared__ unsigned long long g_w[kPCap];      // also the digit counts while narrowing
    __shared__ float red_f[kPThreads / 64];
    __shared__ unsigned long long red_u[kPThreads / 64];
    __shared__ double red_d[kPThreads / 64];
    __shared__ double s_before_d;
    __shared__ unsigned long long s_before, s_prefix, s_qb;
    __shared__ int s_bin, s_n, s_sub;
    __shared__ double s_tab[64];  // 2^(-k/64)
    static_assert(sizeof(g_w) >= kPBins * sizeof(unsigned int), "digit counts fit");
    static_assert(sizeof(h_mass) >= kPCap * 2 * sizeof(unsigned long long), "final candidates fit");
    unsigned int* const h_cnt = reinterpret_cast<unsigned int*>(g_w);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t R = blockIdx.x;
    const float* z = a.z + R * a.V;
    float* out = a.out ? a.out + R * a.V : nullptr;  // NULL when only the cut is wanted
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
            // (the last batch too: its loads past the row re-read quad 0 and
            // go unused, so they never wait one after another)
            const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
            const int V4 = V >> 2;
            for (int i = tid; i < V4; i += kPInFlight * kPThreads) {
                f32x4 q[kPInFlight];
#pragma unroll
                for (int u = 0; u < kPInFlight; ++u) {
                    const int j = i + u * kPThreads;
                    q[u] = z4[j < V4 ? j : 0];
                }
#pragma unroll
                for (int u = 0; u < kPInFlight; ++u) {
                    const int j = i + u * kPThreads;
                    if (j < V4) {
                        const int b = 4 * j;
                        fn(q[u][0], b); fn(q[u][1], b + 1); fn(q[u][2], b + 2); fn(q[u][3], b + 3);
                    }
                }
            }
        } else {
            for (int v = tid; v < V; v += kPThreads) fn(z[v], v);
        }
    };
    auto fmax_op = [](float x, float y) { return fmaxf(x, y); };
    // exclusive prefix over threads of `mine` (ascending thread order)
    auto thread_prefix = [&](auto mine, auto* red) {
        auto incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const auto t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        __syncthreads();
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        auto before = incl - mine;
        for (int w = 0; w < wave; ++w) before += red[w];
        return before;
    };
    constexpr int kPer = kPBins / kPThreads;  // bins per thread in the scans over bins

    unsigned long long cut = 0;  // rank key of the last kept entry (0: keep everything)
    unsigned int nucleus = (unsigned int)V;
    float m = -INFINITY;
    Bins bins{-INFINITY, c2, INFINITY};
    if (a.top_p < 1.0) {
        // AB (see the header): the sample's maximum, then the row's maximum and
        // the histogram in one pass
        float r = -INFINITY;
        if (vec) {
            const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
            f32x4 q[kPInFlight];
#pragma unroll
            for (int u = 0; u < kPInFlight; ++u) {
                const int i = tid + u * kPThreads;
                q[u] = z4[i < (V >> 2) ? i : 0];
            }
#pragma unroll
            for (int u = 0; u < kPInFlight; ++u)
                r = fmaxf(r, fmaxf(fmaxf(q[u][0], q[u][1]), fmaxf(q[u][2], q[u][3])));
        } else {
            for (int u = 0; u < kPInFlight; ++u) r = fmaxf(r, z[min(tid + u * kPThreads, V - 1)]);
        }
        for (int b = tid; b < kPBins; b += kPThreads) h_mass[b] = 0;
        if (tid < 64) s_tab[tid] = exp2(-(double)tid / 64.0);
        r = block_reduce(r, red_f, fmax_op);
        bool rebuild = true;
        if (r != -INFINITY) {
            bins.set_ref(r + kHeadroom / c2);
            each([&](float x, int) {
                m = fmaxf(m, x);
                const float y = bins.y(x);
                const int b = bins.bin(y);
                atomicAdd(&h_mass[b], (unsigned long long)bins.weight(y, b));
            });
            m = block_reduce(m, red_f, fmax_op);
            rebuild = m > bins.ref;  // an entry above ref: its weight would exceed the bin's top
        } else {
            each([&](float x, int) { m = fmaxf(m, x); });
            m = block_reduce(m, red_f, fmax_op);
        }
        if (rebuild && m != -INFINITY) {
            __syncthreads();
            for (int b = tid; b < kPBins; b += kPThreads) h_mass[b] = 0;
            __syncthreads();
            bins.set_ref(m);
            each([&](float x, int) {
                const float y = bins.y(x);
                const int b = bins.bin(y);
                atomicAdd(&h_mass[b], (unsigned long long)bins.weight(y, b));
            });
        }
        __syncthreads();
    }
    if (a.top_p < 1.0 && m != -INFINITY) {
        // bin masses relative to ref: sum x 2^-31 x 2^(-b/64)
        double mass[kPer];
        double mine = 0.0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int b = tid * kPer + i;
            mass[i] = ldexp((double)h_mass[b] * s_tab[b & 63], -31 - (b >> 6));
            mine += mass[i];
        }
        const double total = block_reduce(mine, red_d, [](double x, double y) { return x + y; });
        const double target = a.top_p * total;
        if (tid == 0) { s_bin = kPBins - 1; s_before_d = 0.0; s_prefix = 0; s_before = 0; }
        const double before = thread_prefix(mine, red_d);
        if (before < target && before + mine >= target) {
            double c = before;
            for (int i = 0; i < kPer; ++i) {
                if (c + mass[i] >= target) { s_bin = tid * kPer + i; s_before_d = c; break; }
                c += mass[i];
            }
        }
        __syncthreads();
        const int bstar = s_bin;
        const unsigned long long qb = h_mass[bstar];  // the boundary bin's fixed-point sum
        // mass still needed inside the boundary bin, in its fixed point (at
        // least one unit; at most the bin's sum, so rounding cannot push the
        // boundary past the bin)
        unsigned long long need;
        {
            const double nq = ceil(ldexp((target - s_before_d) * exp2((double)(bstar & 63) / 64.0),
                                         31 + (bstar >> 6)));
            need = nq < 1.0 ? 1ull : (unsigned long long)nq;
            if (qb > 0 && need > qb) need = qb;
        }
        // the candidate set: bin bstar and, after `level` narrowing steps, the
        // rank keys whose top 12*level bits equal `prefix`
        auto in_set = [&](uint64_t key, int level, unsigned long long prefix) {
            if (level == 0) return true;
            const int sh = 64 - 12 * level;
            return sh <= 0 ? key == prefix : (key >> sh) == (prefix >> sh);
        };
        // ranked ahead of every entry of the set (bins count down from the top)
        auto ahead_of_set = [&](uint64_t key, int level, unsigned long long prefix) {
            if (level == 0) return false;
            const int sh = 64 - 12 * level;
            return sh <= 0 ? key > prefix : (key >> sh) > (prefix >> sh);
        };
        int level = 0;
        unsigned long long prefix = 0;
        unsigned int ahead = 0;  // this thread's entries ranked ahead of the set
        // C: gather the set (every pass counts it; entries beyond kPCap are dropped)
        auto gather = [&]() {
            __syncthreads();
            if (tid == 0) s_n = 0;
            __syncthreads();
            ahead = 0;
            each([&](float x, int v) {
                const float y = bins.y(x);
                const int b = bins.bin(y);
                ahead += b < bstar ? 1u : 0u;
                const bool hit = b == bstar;
                // about one entry in a thousand: a wave-uniform test keeps the
                // common path free of per-entry branches
                if (ballot(hit)) {
                    if (hit) {
                        const uint64_t key = rank_key(x, v);
                        if (in_set(key, level, prefix)) {
                            const int at = atomicAdd(&s_n, 1);
                            if (at < kPCap) {
                                g_key[at] = key;
                                g_w[at] = bins.weight(y, b);
                            }
                        } else {
                            ahead += ahead_of_set(key, level, prefix) ? 1u : 0u;
                        }
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
                const float y = bins.y(x);
                const int b = bins.bin(y);
                if (b != bstar) return;
                const uint64_t key = rank_key(x, v);
                if (!in_set(key, level, prefix)) return;
                const int d = sh >= 0 ? (int)((key >> sh) & 0xFFF) : (int)((key << -sh) & 0xFFF);
                atomicAdd(&h_mass[kPBins - 1 - d], (unsigned long long)bins.weight(y, b));
                atomicAdd(&h_cnt[kPBins - 1 - d], 1u);
            });
            __syncthreads();
            const unsigned long long sb = s_before;  // read by every thread before the winner rewrites it
            // digits in descending order = bins in ascending order
            unsigned long long mine2 = 0;
#pragma unroll
            for (int i = 0; i < kPer; ++i) mine2 += h_mass[tid * kPer + i];
            const unsigned long long bef2 = sb + thread_prefix(mine2, red_u);
            if (bef2 < need && bef2 + mine2 >= need) {
                unsigned long long c = bef2;
                for (int i = 0; i < kPer; ++i) {
                    const int b = tid * kPer + i;
                    if (c + h_mass[b] >= need) {
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
        const int n = min(count, kPCap);
        // sub-bins of the gathered set (all in bin bstar): the one where the
        // mass reaches `need` holds the boundary; entries of earlier sub-bins
        // rank ahead of it
        for (int b = tid; b < kPBins; b += kPThreads) h_mass[b] = 0;
        if (tid == 0) { s_sub = kPBins - 1; s_qb = 0; }
        __syncthreads();
        auto sub_of = [&](uint64_t key) { return bins.sub(bins.y(key_logit((uint32_t)(key >> 32))), bstar); };
        for (int i = tid; i < n; i += kPThreads) atomicAdd(&h_mass[sub_of(g_key[i])], g_w[i]);
        __syncthreads();
        const unsigned long long sb = s_before;
        unsigned long long mine3 = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) mine3 += h_mass[tid * kPer + i];
        const unsigned long long bef3 = sb + thread_prefix(mine3, red_u);
        if (bef3 < need && bef3 + mine3 >= need) {
            unsigned long long c = bef3;
            for (int i = 0; i < kPer; ++i) {
                const int b = tid * kPer + i;
                if (c + h_mass[b] >= need) { s_sub = b; s_qb = c; break; }
                c += h_mass[b];
            }
        }
        __syncthreads();
        const int ssub = s_sub;
        const unsigned long long sub_before = s_qb;
        if (tid == 0) s_n = 0;
        __syncthreads();
        // the sub-bin's entries, compacted into h_mass as (key, weight) pairs
        for (int i = tid; i < n; i += kPThreads) {
            const uint64_t key = g_key[i];
            if (sub_of(key) == ssub) {
                const int at = atomicAdd(&s_n, 1);
                h_mass[2 * at] = key;
                h_mass[2 * at + 1] = g_w[i];
            }
        }
        __syncthreads();
        const int nc = s_n;
        // each: the mass of the sub-bin's entries ranked at or ahead of it
        unsigned long long best = 0;
        for (int i = tid; i < nc; i += kPThreads) {
            const uint64_t ki = h_mass[2 * i];
            unsigned long long ge = sub_before;
            for (int j = 0; j < nc; ++j) ge += h_mass[2 * j] >= ki ? h_mass[2 * j + 1] : 0ull;
            if (ge >= need && ki > best) best = ki;
        }
        cut = block_reduce(best, red_u, [](unsigned long long x, unsigned long long y) { return x > y ? x : y; });
        // nucleus size: the entries ahead of the set, then the set's entries at or ahead of the cut
        unsigned int in_nucleus = ahead;
        for (int i = tid; i < n; i += kPThreads) in_nucleus += g_key[i] >= cut ? 1u : 0u;
        nucleus = block_reduce(in_nucleus, (unsigned int*)red_f,
                               [](unsigned int x, unsigned int y) { return x + y; });
        if (cut == 0) nucleus = (unsigned int)V;
    }
    if (a.cut_out && tid == 0) {
        a.cut_out[R] = cut == 0 ? dflash_nucleus_cut{-INFINITY, INT32_MAX}
                                : dflash_nucleus_cut{key_logit((uint32_t)(cut >> 32)),
                                                     (int32_t)(0xFFFFFFFFu - (uint32_t)cut)};
    }
    if (!a.out) {
        if (a.kept && tid == 0) a.kept[R] = (int32_t)nucleus;
        return;
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
        for (int i = tid; i < V4; i += kPInFlight * kPThreads) {
            f32x4 q[kPInFlight];
#pragma unroll
            for (int u = 0; u < kPInFlight; ++u) {
                const int j = i + u * kPThreads;
                q[u] = z4[j < V4 ? j : 0];
            }
#pragma unroll
            for (int u = 0; u < kPInFlight; ++u) {
                const int j = i + u * kPThreads;
                if (j < V4) mask4(q[u], j);
            }
        }
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

// `out` (masking) or `cut` is the required output; the other one is NULL.
int top_p_launch(const float* logits, float* out, dflash_nucleus_cut* cut, int32_t* kept, int rows,
                 int vocab, float temperature, float top_p, bool masking, void* stream) {
    if (rows < 0 || vocab < 1) return DFLASH_ERR_SHAPE;
    if (!(temperature > 0.f) || !std::isfinite(temperature)) return DFLASH_ERR_SHAPE;
    if (!(top_p > 0.f) || !(top_p <= 1.f)) return DFLASH_ERR_SHAPE;
    if (rows == 0) return DFLASH_OK;
    if (!logits || (masking ? !out : !cut)) return DFLASH_ERR_NULL;
    if (vocab >= kMaxTopPVocab || rows > kMaxRowsPerCall) return DFLASH_ERR_UNSUPPORTED;
    TopPArgs a{logits, out, cut, kept, vocab, (float)(1.4426950408889634 / (double)temperature),
               (double)top_p};
    hipLaunchKernelGGL(top_p_kernel, dim3(rows), dim3(kPThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return launch_status();
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" int dflash_top_p_mask(const float* logits, float* out, int32_t* kept, int rows, int vocab,
                                 float temperature, float top_p, void* stream) {
    return top_p_launch(logits, out, nullptr, kept, rows, vocab, temperature, top_p, true, stream);
}

extern "C" int dflash_top_p_cut(const float* logits, dflash_nucleus_cut* cut, int32_t* kept, int rows,
                                int vocab, float temperature, float top_p, void* stream) {
    return top_p_launch(logits, nullptr, cut, kept, rows, vocab, temperature, top_p, false, stream);
}
