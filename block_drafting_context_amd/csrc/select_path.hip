// select_path.hip -- the DFlash 2 candidate selector, for gfx950.
//
// "DFlash vs DFlash 2", "The candidate selector": every block position keeps the
// top-k draft candidates; a transition from candidate a at the preceding
// position to candidate b at position t scores
//     S_t(a, b) = U_t(b) + sum_i A(a)_i H(h_t)_i B(b)_i,
// all transition scores are computed in parallel, and only the walk through
// them is sequential.  The walk is greedy: position 0 follows the anchor token,
// every later position follows the token just chosen; ties go to the candidate
// listed first.
//
// One workgroup per sequence.  Positions are taken in chunks whose score table
// (k x k doubles per position) fits in LDS: the 1,024 threads compute the table
// entries of a chunk (one (position, a, b) triple at a time per thread, the sum
// over i in increasing order in fp64 -- each term is a product of three bf16
// values, exact in fp64, so the sum is rounded exactly as a sequential fp64
// sum), then wave 0 walks the chunk with one lane per candidate.
#include "common.hpp"

namespace dfl {
DFL_VIOLATION_WORD(violations_select)
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelTableDoubles = 12288;  // 96 KB of LDS for the score table
constexpr int kSelMaxGamma = 4096;         // block positions: t * k stays far inside int

struct SelArgs {
    const int32_t* cand;    // [B, G, k]
    const float* score;     // [B, G, k]  U_t(b)
    const uint16_t* emb_a;  // [V, r] bf16
    const uint16_t* emb_b;  // [V, r] bf16
    const uint16_t* gate;   // [B, G, r] bf16
    const int32_t* anchor;  // [B]
    int32_t* path;          // [B, G]
    float* path_score;      // [B, G] or null
    int B, G, k, V, r, chunk;
};

__device__ __forceinline__ double bf16_to_f64(uint16_t h) {
    return (double)__uint_as_float((uint32_t)h << 16);
}
__device__ __forceinline__ int clamp_id(int v, int V) { return v < 0 ? 0 : (v >= V ? V - 1 : v); }

// wave-wide best (value desc, index asc) over doubles
__device__ __forceinline__ void best_of_d(double& v, int& i, double ov, int oi) {
    if (ov > v || (ov == v && (unsigned)oi < (unsigned)i)) { v = ov; i = oi; }
}
template <int CTRL>
__device__ __forceinline__ void best_dpp_d(double& v, int& i) {
    best_of_d(v, i, dpp_d<CTRL>(v), dpp_i<CTRL>(i));
}
template <int W>
__device__ __forceinline__ void best_swap_d(double& v, int& i) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    unsigned l0, l1, h0, h1, i0, i1;
    swap_pair<W>((unsigned)u, l0, l1);
    swap_pair<W>((unsigned)(u >> 32), h0, h1);
    swap_pair<W>((unsigned)i, i0, i1);
    v = __longlong_as_double((long long)(((unsigned long long)h0 << 32) | l0));
    i = (int)i0;
    best_of_d(v, i, __longlong_as_double((long long)(((unsigned long long)h1 << 32) | l1)), (int)i1);
}
__device__ __forceinline__ void wave_best_d(double& v, int& i) {
    best_dpp_d<kDppXor1>(v, i);
    best_dpp_d<kDppXor2>(v, i);
    best_dpp_d<kDppHalfMirror>(v, i);
    best_dpp_d<kDppMirror>(v, i);
    best_swap_d<16>(v, i);
    best_swap_d<32>(v, i);
}

__global__ void __launch_bounds__(kSelThreads) select_path_kernel(SelArgs a) {
    __shared__ double table[kSelTableDoubles];  // [chunk position][a][b]
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int G = a.G, k = a.k, r = a.r;
    const int32_t* cand = a.cand + (size_t)b * G * k;
    const float* U = a.score + (size_t)b * G * k;
    const int anchor = clamp_id(a.anchor[b], a.V);
    if (DFLASH_DEVICE_CHECKS) {
        bool bad = tid == 0 && (a.anchor[b] < 0 || a.anchor[b] >= a.V);
        for (int e = tid; e < G * k; e += kSelThreads) bad |= cand[e] < 0 || cand[e] >= a.V;
        if (bad) DFL_VIOLATION(DFLASH_VIOLATION_TOKEN);
    }
    int prev_i = 0;  // wave 0: slot of the last chosen candidate among its position's list
    for (int t0 = 0; t0 < G; t0 += a.chunk) {
        const int nt = min(a.chunk, G - t0);
        // table[tl][ai][bi] = S_t(a_i, b_i), a_i = candidate ai of position t - 1
        // (position 0: the anchor, ai = 0 only)
        const int total = nt * k * k;
        for (int e = tid; e < total; e += kSelThreads) {
            const int tl = e / (k * k), ai = (e / k) % k, bi = e % k;
            const int t = t0 + tl;
            if (t == 0 && ai > 0) continue;
            const int tok_a = t == 0 ? anchor : clamp_id(cand[(t - 1) * k + ai], a.V);
            const int tok_b = clamp_id(cand[t * k + bi], a.V);
            const u32x4* ea = reinterpret_cast<const u32x4*>(a.emb_a + (size_t)tok_a * r);
            const u32x4* eb = reinterpret_cast<const u32x4*>(a.emb_b + (size_t)tok_b * r);
            const u32x4* gt = reinterpret_cast<const u32x4*>(a.gate + ((size_t)b * G + t) * r);
            double s = (double)U[t * k + bi];
            // blocks of 32 elements: the 12 loads of a block are issued before its math
            for (int i0 = 0; i0 < r / 8; i0 += 4) {
                u32x4 va[4], vg[4], vb[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // a block past the row's end reads its last block and adds nothing
                    // (addresses clamped, so the 12 loads are never behind a branch)
                    const bool in = i0 + q < r / 8;
                    const int qc = in ? i0 + q : r / 8 - 1;
                    const u32x4 xa = ea[qc], xg = gt[qc], xb = eb[qc];
                    va[q] = in ? xa : u32x4{0u, 0u, 0u, 0u};
                    vg[q] = in ? xg : u32x4{0u, 0u, 0u, 0u};
                    vb[q] = in ? xb : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const double x = bf16_to_f64((uint16_t)(va[q][c] >> (16 * h)));
                            const double y = bf16_to_f64((uint16_t)(vg[q][c] >> (16 * h)));
                            const double z = bf16_to_f64((uint16_t)(vb[q][c] >> (16 * h)));
                            s += x * y * z;  // exact product: the rounding is the sum's alone
                        }
            }
            table[e] = s;
        }
        __syncthreads();
        if (tid < 64) {
            for (int tl = 0; tl < nt; ++tl) {
                const int t = t0 + tl;
                const int ai = t == 0 ? 0 : prev_i;
                double v = lane < k ? table[(tl * k + ai) * k + lane] : -INFINITY;
                int idx = lane < k ? lane : -1;
                wave_best_d(v, idx);
                prev_i = idx;
                if (lane == 0) {
                    a.path[(size_t)b * G + t] = clamp_id(cand[t * k + idx], a.V);
                    if (a.path_score) a.path_score[(size_t)b * G + t] = (float)v;
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" int dflash_select_path(const int32_t* cand_idx, const float* cand_score,
                                  const uint16_t* emb_a, const uint16_t* emb_b, const uint16_t* gate,
                                  const int32_t* anchor, int32_t* path, float* path_score, int batch,
                                  int gamma, int k, int vocab, int r, void* stream) {
    if (batch < 0 || gamma < 1 || k < 1 || vocab < 1 || r < 1) return DFLASH_ERR_SHAPE;
    if (batch == 0) return DFLASH_OK;
    if (!cand_idx || !cand_score || !emb_a || !emb_b || !gate || !anchor || !path)
        return DFLASH_ERR_NULL;
    if (k > 64 || r % 8 != 0 || r > 4096 || gamma > kSelMaxGamma || batch > kMaxRowsPerCall)
        return DFLASH_ERR_UNSUPPORTED;
    const uintptr_t align = reinterpret_cast<uintptr_t>(emb_a) | reinterpret_cast<uintptr_t>(emb_b) |
                            reinterpret_cast<uintptr_t>(gate);
    if (align & 15) return DFLASH_ERR_UNSUPPORTED;
    SelArgs a{cand_idx, cand_score, emb_a, emb_b, gate, anchor, path, path_score,
              batch, gamma, k, vocab, r, kSelTableDoubles / (k * k)};
    hipLaunchKernelGGL(select_path_kernel, dim3(batch), dim3(kSelThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return launch_status();
}
