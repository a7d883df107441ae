// vocab_rows.hip -- per-position top-k, drafted-token draws and lossless
// verification over 151,936-entry logits rows, for gfx950.
//
// "DFlash vs DFlash 2", "The candidate selector": top-k candidates per block
// position.  "The problem: one expensive token at a time": the drafter
// proposes y ~ q; the target keeps the longest valid prefix (greedy: drafts
// equal to its argmax; sampled: accept with probability min(1, p/q)),
// corrects the first rejection from [p - q]_+ and adds a bonus token when
// every draft survives.
//
// Every pass over a row is one streaming read, split into 2,048-element
// segments.  A wave owns a run of consecutive segments of one row and, per
// segment, holds all 32 of each lane's elements in registers (8 float4
// loads issued together), so it can take an exact wave-uniform segment
// maximum m_s before exponentiating.  Per segment it can produce
//   * m_s, and s_s = sum 2^((z - m_s) * log2(e)/T)   (fp32 pairwise sums,
//     fp64 across), or
//   * the wave's argmax.
// Top-k needs only the segment maxima from the streaming pass: tau = the k-th
// largest m_s of the row (counting repeats) is a lower bound of the row's k-th
// largest entry, since those k maxima are k distinct entries, so every top-k
// entry lies in a segment with m_s >= tau.  The finalize re-reads just those
// segments (about k of them) with tau as the first filter: entries that can
// still rank are compacted into an LDS buffer, whose list is rebuilt by k
// rounds of a wave-wide (value desc, index asc) reduction when it fills.
// An inverse-CDF draw needs only the segment sums plus one re-read of the
// single 2,048-element segment holding the crossing, recomputing the element
// weights with exactly the arithmetic that produced the sums.
#include <cmath>

#include "common.hpp"
#include "verify_run.hpp"

namespace dfl {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSeg = 2048;             // elements per segment (8 x 64 lanes x 4)
constexpr int kIters = kSeg / 256;     // float4 loads per lane per segment
constexpr int kCap = 256;              // top-k candidate buffer fill that triggers a rebuild
constexpr int kBuf = kCap + 256;       // buffer size: one load group (4 x 64) of slack
constexpr int kScanWaves = 4;          // waves per workgroup
constexpr int kFinWaves = 4;           // waves per top-k finalize workgroup (one row)
constexpr int kTargetWaves = 3072;     // waves per row-scan launch (~12 per CU)
constexpr int kRsrcWord3 = 0x00020000; // buffer resource word 3 for raw byte buffers on gfx9 parts
constexpr int kMaxVocab = 1 << 29;     // a row's bytes, and a segment past it, fit 32-bit offsets

enum : int { kArgmax = 1, kSumExp = 2, kSegMax = 4 };

struct ScanArgs {
    const float* z;  // [rows, V]
    int rows, V, nseg, spw, wpr;
    float c2;        // log2(e) / T
    float* seg_m;    // [rows][nseg]
    double* seg_s;   // [rows][nseg]
    float* cand_v;   // [rows][wpr]: each wave's argmax
    int* cand_i;
};

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------- wave top-k state
// Per-wave state of the candidate search.  The LDS arrays are indexed
// directly from the kernel's __shared__ declarations (never through generic
// pointers), and the scalars live in registers, so every access is a ds_*
// instruction with a compile-time address space.
constexpr int kNPL = (64 + kBuf + 63) / 64;  // candidates per lane in a rebuild

struct TopKRegs {
    int cnt;     // buffer fill (wave-uniform)
    int lcount;  // list length (wave-uniform)
    float tv;    // filter: a quad is appended when its maximum is >= tv
};

// Rebuild the sorted list of `wave` from list + buffer: k rounds of a
// wave-wide (value desc, index asc) reduction.
// Entries below `floor` are known not to rank, so the filter never drops under it.
__device__ __forceinline__ void topk_compact(TopKRegs& s, float (*lv)[64], int (*li)[64],
                                             float (*bv)[kBuf], int (*bi)[kBuf], int wave, int k,
                                             int lane, float floor) {
    wave_lds_sync();
    const int N = s.lcount + s.cnt;
    float cv[kNPL];
    int ci[kNPL];
#pragma unroll
    for (int e = 0; e < kNPL; ++e) {
        const int at = e * 64 + lane;
        if (at < s.lcount) { cv[e] = lv[wave][at]; ci[e] = li[wave][at]; }
        else if (at < N) { cv[e] = bv[wave][at - s.lcount]; ci[e] = bi[wave][at - s.lcount]; }
        else { cv[e] = -INFINITY; ci[e] = -1; }
    }
    wave_lds_sync();
    const int newcount = N < k ? N : k;
    float lastv = -INFINITY;
    for (int r = 0; r < newcount; ++r) {
        float b_v = cv[0];
        int b_i = ci[0];
#pragma unroll
        for (int e = 1; e < kNPL; ++e)
            if (ranks_ahead(cv[e], ci[e], b_v, b_i)) { b_v = cv[e]; b_i = ci[e]; }
        wave_best(b_v, b_i);
#pragma unroll
        for (int e = 0; e < kNPL; ++e)
            if (ci[e] == b_i && ci[e] != -1) { cv[e] = -INFINITY; ci[e] = -1; }
        if (lane == 0) { lv[wave][r] = b_v; li[wave][r] = b_i; }
        lastv = b_v;
    }
    wave_lds_sync();
    s.lcount = newcount;
    s.cnt = 0;
    s.tv = newcount == k ? fmaxf(lastv, floor) : floor;
}

template <int MODE>
__global__ void __launch_bounds__(256) row_scan_kernel(ScanArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kScanWaves + wave;
    const int row = gw / a.wpr, wr = gw % a.wpr;
    if (row >= a.rows) return;
    const int seg0 = wr * a.spw;
    const int seg1 = min(seg0 + a.spw, a.nseg);
    const float* zr = a.z + (size_t)row * a.V;

    float best_v = -INFINITY;
    int best_i = -1;

    // The 32 elements of this lane in segment `seg`: base + it*256 + c.  The
    // row is read through a raw buffer of V*4 bytes, so every load is issued
    // unconditionally: a quad past the row's end (V % 4 == 0, so quads are
    // whole) or of a segment past this wave's run reads as zeros without
    // touching memory, and the compiler counts the loads in flight exactly
    // (with the loads in branches it waited for all of them, the next
    // segment's prefetch included, before processing the current one).
    const __amdgpu_buffer_rsrc_t zr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(zr), (short)0, a.V * 4, kRsrcWord3);
    auto load = [&](f32x4 (&vv)[kIters], int seg) {
        const uint32_t base = (uint32_t)(seg * kSeg + 4 * lane) * 4u;  // < 2^32: V <= 2^29
#pragma unroll
        for (int it = 0; it < kIters; ++it)
            // logits rows are streamed once: non-temporal loads
            vv[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  zr_rsrc, (int)(base + it * 1024u), 0, kLoadStream));
    };
    auto process = [&](f32x4 (&v)[kIters], int seg) {
        const int base = seg * kSeg + 4 * lane;
        if (seg * kSeg + kSeg > a.V) {
            // quads past the row's end read as zeros: they take no part
#pragma unroll
            for (int it = 0; it < kIters; ++it)
                if (base + it * 256 >= a.V) v[it] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
        if (MODE & kArgmax) {
#pragma unroll
            for (int it = 0; it < kIters; ++it)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (v[it][c] > best_v) { best_v = v[it][c]; best_i = base + it * 256 + c; }
        }
        float lane_m = -INFINITY;
        if (MODE & (kSumExp | kSegMax)) {
#pragma unroll
            for (int it = 0; it < kIters; ++it)
                lane_m = fmaxf(lane_m, fmaxf(fmaxf(v[it][0], v[it][1]), fmaxf(v[it][2], v[it][3])));
        }
        if (MODE & kSegMax) {
            const float m = wave_max(lane_m);
            if (lane == 0) a.seg_m[(size_t)row * a.nseg + seg] = m;
        }
        if (MODE & kSumExp) {
            const float m = wave_max(lane_m);
            double sacc = 0.0;
            if (m != -INFINITY) {
#pragma unroll
                for (int h = 0; h < kIters / 2; ++h) {
                    float w[8];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            w[q * 4 + c] = fast_exp2((v[2 * h + q][c] - m) * a.c2);
                    const float t = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
                    sacc += (double)t;
                }
            }
            sacc = wave_sum(sacc);
            if (lane == 0) {
                a.seg_m[(size_t)row * a.nseg + seg] = m;
                a.seg_s[(size_t)row * a.nseg + seg] = sacc;
            }
        }
    };

    // two segments per trip, each one's loads issued before the other is
    // processed; a segment past the run is loaded from past the row's end
    const int dead = a.nseg;
    f32x4 va[kIters], vb[kIters];
    load(va, seg0 < seg1 ? seg0 : dead);
    for (int seg = seg0; seg < seg1; seg += 2) {
        const bool has_b = seg + 1 < seg1;
        load(vb, has_b ? seg + 1 : dead);
        process(va, seg);
        load(va, seg + 2 < seg1 ? seg + 2 : dead);
        if (has_b) process(vb, seg + 1);
    }

    if (MODE & kArgmax) {
        wave_best(best_v, best_i);
        if (lane == 0) {
            a.cand_v[(size_t)row * a.wpr + wr] = best_v;
            a.cand_i[(size_t)row * a.wpr + wr] = best_i;
        }
    }
}

// ----------------------------------------------------------- draws
// Merge a row's segment statistics: M = max m_s, S = sum s_s 2^((m_s - M) c2)
// (each lane sums its segments lane, lane + 64, ... in that order).  The
// first 64 * kStatRegs segments are loaded at once into registers (addresses
// clamped into the row, so no load sits behind a branch), the rest in a loop.
constexpr int kStatRegs = 4;
__device__ __forceinline__ void merge_row_stats(const float* sm, const double* ss, int nseg, float c2, int lane,
                                float& M, double& S) {
    float mv[kStatRegs];
    double sv[kStatRegs];
#pragma unroll
    for (int j = 0; j < kStatRegs; ++j) {
        const int sj = lane + 64 * j;
        const int sc = sj < nseg ? sj : nseg - 1;
        const float x = sm[sc];
        sv[j] = ss[sc];
        mv[j] = sj < nseg ? x : -INFINITY;
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kStatRegs; ++j) m = fmaxf(m, mv[j]);
    for (int s = lane + 64 * kStatRegs; s < nseg; s += 64) m = fmaxf(m, sm[s]);
    M = wave_max(m);
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < kStatRegs; ++j)
        if (mv[j] != -INFINITY) acc += sv[j] * (double)fast_exp2((mv[j] - M) * c2);
    for (int s = lane + 64 * kStatRegs; s < nseg; s += 64)
        if (sm[s] != -INFINITY) acc += ss[s] * (double)fast_exp2((sm[s] - M) * c2);
    S = wave_sum(acc);
}

// Smallest element index of segment `seg` whose running weight (increasing
// index) exceeds tgt; wfn.w4(v) gives the fp32 weights of elements v..v+3
// (the same arithmetic that produced the segment sums), summed in fp64.
// Falls back to the last positive-weight element of the segment when
// rounding leaves no crossing.  Wave-wide; every lane returns the index.
template <class WFn>
__device__ __forceinline__ int draw_in_segment(int seg, int V, double tgt, const WFn& wfn, int lane) {
    const int lo = seg * kSeg + lane * 32;
    float w[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        // a quad past the row's end reads the last quad (V % 4 == 0) and weighs
        // nothing, so the eight loads are issued together
        const int v = lo + 4 * q;
        const f32x4 w4 = wfn.w4(v < V ? v : V - 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) w[4 * q + c] = v < V ? w4[c] : 0.f;
    }
    double mine = 0.0;
#pragma unroll
    for (int j = 0; j < 32; ++j) mine += (double)w[j];
    const double incl = wave_inclusive_scan(mine);
    const double excl = incl - mine;
    const uint64_t hit = ballot(mine > 0.0 && incl > tgt);
    int result = -1;
    if (hit) {
        const int src = __builtin_ctzll(hit);
        int found = -1;
        if (lane == src) {
            double acc = excl;
            int lastpos = -1;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                if (w[j] > 0.f) lastpos = lo + j;
                acc += (double)w[j];
                if (found < 0 && w[j] > 0.f && acc > tgt) found = lo + j;
            }
            if (found < 0) found = lastpos;
        }
        result = lane_value(found, src);
    } else {
        const uint64_t pos = ballot(mine > 0.0);
        if (pos) {
            const int src = 63 - __builtin_clzll(pos);
            int last = -1;
            if (lane == src) {
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    if (w[j] > 0.f) last = lo + j;
            }
            result = lane_value(last, src);
        }
    }
    return result;
}

// Pick the segment whose cumulative weight crosses `target`.  seg_w(s) is a
// segment's weight in the units of target.  Returns the segment and the
// weight before it.
template <class SegW>
__device__ __forceinline__ int find_segment(int nseg, double target, const SegW& seg_w, int lane, double& before) {
    double carry = 0.0;
    int last_pos_seg = -1;
    double before_last = 0.0;
    for (int s0 = 0; s0 < nseg; s0 += 64) {
        const int s = s0 + lane;
        const double w = s < nseg ? seg_w(s) : 0.0;
        const double incl = wave_inclusive_scan(w);
        const uint64_t hit = ballot(w > 0.0 && carry + incl > target);
        if (hit) {
            const int src = __builtin_ctzll(hit);
            before = carry + lane_value(incl - w, src);
            return s0 + src;
        }
        const uint64_t pos = ballot(w > 0.0);
        if (pos) {
            const int src = 63 - __builtin_clzll(pos);
            last_pos_seg = s0 + src;
            before_last = carry + lane_value(incl - w, src);
        }
        carry += lane_value(incl, 63);
    }
    before = before_last;
    return last_pos_seg;
}

// Weight 2^((z - m_s) * c2) of softmax(z / T) relative to a segment maximum.
struct SoftmaxW {
    const float* zr;
    float ms, c2;
    __device__ __forceinline__ f32x4 w4(int v) const {
        const f32x4 z = *reinterpret_cast<const f32x4*>(zr + v);
        f32x4 r;
        r[0] = fast_exp2((z[0] - ms) * c2);
        r[1] = fast_exp2((z[1] - ms) * c2);
        r[2] = fast_exp2((z[2] - ms) * c2);
        r[3] = fast_exp2((z[3] - ms) * c2);
        return r;
    }
};

// Draw from softmax(z / T) of one row using its segment statistics.
__device__ __forceinline__ int draw_softmax_row(const float* zr, int V, const float* sm, const double* ss,
                                int nseg, float c2, float M, double S, double u, int lane) {
    const double target = u * S;
    double before = 0.0;
    auto segw = [&](int s) -> double {
        return sm[s] == -INFINITY ? 0.0 : ss[s] * (double)fast_exp2((sm[s] - M) * c2);
    };
    const int seg = find_segment(nseg, target, segw, lane, before);
    if (seg < 0) return 0;
    const float ms = sm[seg];
    const double f = (double)fast_exp2((ms - M) * c2);
    const double tgt = (target - before) / f;
    const SoftmaxW wfn{zr, ms, c2};
    return draw_in_segment(seg, V, tgt, wfn, lane);
}

// ------------------------------------------------------- top-k finalize
struct TopKFin {
    const float* z;
    int B, G, V, nseg, k;
    float T, c2;
    const uint64_t* seeds;
    uint64_t step;
    const float* seg_m;
    const double* seg_s;
    int32_t* topk_idx;
    float* topk_val;
    double* lse;
    int32_t* draft;
};

constexpr int kSegCache = 4;  // segment maxima per lane held in registers by the finalize

// The k-th largest of a row's segment maxima, counting repeats; -inf when
// fewer than k of them are above -inf.  Each round takes the largest maximum
// below the previous one and counts its copies, so at most k rounds.  The
// first 64 * kSegCache maxima come from registers (c), the rest from memory.
__device__ __forceinline__ float kth_segment_max(const float (&c)[kSegCache], const float* sm, int nseg,
                                                 int k, int lane) {
    float t = INFINITY;
    int counted = 0;
    for (;;) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < kSegCache; ++j)
            if (c[j] < t) m = fmaxf(m, c[j]);
        for (int s = 64 * kSegCache + lane; s < nseg; s += 64) {
            const float x = sm[s];
            if (x < t) m = fmaxf(m, x);
        }
        m = wave_max(m);
        if (m == -INFINITY) return -INFINITY;
#pragma unroll
        for (int j = 0; j < kSegCache; ++j) counted += __popcll(ballot(c[j] == m));
        for (int s0 = 64 * kSegCache; s0 < nseg; s0 += 64)
            counted += __popcll(ballot(s0 + lane < nseg && sm[s0 + lane] == m));
        if (counted >= k) return m;
        t = m;
    }
}

// One row per workgroup of five waves.  Waves 0-3 find tau; the segments with
// m_s >= tau are dealt to them in index order (the i-th such segment to wave
// i mod 4), and each re-reads its segments (two in flight) and keeps a top-k
// list over the quads whose maximum passes its filter (tau, raised to the
// wave's own k-th best once it holds k entries).  Meanwhile, at T > 0, wave 4
// merges the segment statistics into the log-normaliser and draws the drafted
// token.  Wave 0 then merges the four lists into the row's top-k.
__global__ void __launch_bounds__(64 * (kFinWaves + 1)) topk_finalize_kernel(TopKFin a) {
    __shared__ float s_lv[kFinWaves][64];
    __shared__ int s_li[kFinWaves][64];
    __shared__ __attribute__((aligned(16))) float s_bv[kFinWaves][kBuf];
    __shared__ __attribute__((aligned(16))) int s_bi[kFinWaves][kBuf];
    __shared__ int s_len[kFinWaves], s_lc[kFinWaves];
    const int row = blockIdx.x, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = row / a.G, r = row % a.G;
    const float* sm = a.seg_m + (size_t)row * a.nseg;
    const float* zr = a.z + (size_t)row * a.V;

    TopKRegs tk{0, 0, -INFINITY};
    float tau = -INFINITY;
    if (wave == kFinWaves) {
        if (a.T > 0.f) {
            float M;
            double S;
            const double* ss = a.seg_s + (size_t)row * a.nseg;
            merge_row_stats(sm, ss, a.nseg, a.c2, lane, M, S);
            if (a.lse && lane == 0) a.lse[row] = (double)M / (double)a.T + log(S);
            if (a.draft) {
                const double u = philox_uniform(a.seeds[b], a.step, (uint64_t)b, (uint64_t)r, kDraftDraw);
                const int tok = draw_softmax_row(zr, a.V, sm, ss, a.nseg, a.c2, M, S, u, lane);
                if (lane == 0) a.draft[row] = tok;
            }
        }
    } else {
        float cache[kSegCache];
#pragma unroll
        for (int j = 0; j < kSegCache; ++j) {
            const int sj = 64 * j + lane;
            cache[j] = sj < a.nseg ? sm[sj] : -INFINITY;
        }
        tau = kth_segment_max(cache, sm, a.nseg, a.k, lane);

        const __amdgpu_buffer_rsrc_t zr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(zr), (short)0, a.V * 4, kRsrcWord3);
        auto load = [&](f32x4 (&v)[kIters], int seg) {
            const uint32_t base = (uint32_t)(seg * kSeg + 4 * lane) * 4u;  // < 2^32: V <= 2^29
#pragma unroll
            for (int it = 0; it < kIters; ++it)
                v[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     zr_rsrc, (int)(base + it * 1024u), 0, kLoadStream));
        };
        tk.tv = tau;
        // a lane whose 4 elements of load group `it` include one that can pass
        // the filter appends all 4 (16-byte LDS writes); the rebuild ranks
        // them exactly, and elements past the row's end go in as empties
        auto append = [&](const f32x4& q, bool pass, uint64_t mask, int idx) {
            if (pass) {
                const int pos = tk.cnt + 4 * lanes_below(mask);
                i32x4 ii;
#pragma unroll
                for (int c = 0; c < 4; ++c) ii[c] = idx + c < a.V ? idx + c : -1;
                *reinterpret_cast<f32x4*>(&s_bv[wave][pos]) = q;
                *reinterpret_cast<i32x4*>(&s_bi[wave][pos]) = ii;
            }
            tk.cnt += 4 * __popcll(mask);
        };
        auto process = [&](f32x4 (&v)[kIters], int seg) {
            const int base = seg * kSeg + 4 * lane;
            bool pass[kIters];
            uint64_t mask[kIters];
            int total = 0;
#pragma unroll
            for (int it = 0; it < kIters; ++it) {
                // quads past the row's end read as zeros: they take no part
                if (base + it * 256 >= a.V) v[it] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                pass[it] = fmaxf(fmaxf(v[it][0], v[it][1]), fmaxf(v[it][2], v[it][3])) >= tk.tv;
                mask[it] = ballot(pass[it]);
                total += __popcll(mask[it]);
            }
            if (!total) return;
            if (tk.cnt + 4 * total <= kBuf) {
                // the whole segment's quads fit: append, then rebuild once
#pragma unroll
                for (int it = 0; it < kIters; ++it)
                    if (mask[it]) append(v[it], pass[it], mask[it], base + it * 256);
                if (tk.cnt > kCap) topk_compact(tk, s_lv, s_li, s_bv, s_bi, wave, a.k, lane, tau);
                return;
            }
            // many passing quads (e.g. long runs of equal logits): one load
            // group at a time, rebuilding whenever the buffer fills
#pragma unroll 1
            for (int it = 0; it < kIters; ++it) {
                f32x4 q = v[0];
#pragma unroll
                for (int j = 1; j < kIters; ++j)
                    if (j == it) q = v[j];
                const bool p = fmaxf(fmaxf(q[0], q[1]), fmaxf(q[2], q[3])) >= tk.tv;
                const uint64_t m = ballot(p);
                if (m) {
                    append(q, p, m, base + it * 256);
                    if (tk.cnt > kCap) topk_compact(tk, s_lv, s_li, s_bv, s_bi, wave, a.k, lane, tau);
                }
            }
        };

        // Collect up to 64 of this wave's segments (lane i holds the i-th),
        // then stream them two at a time; repeat while segments remain.
        const int dead = a.nseg;  // a segment past the row's end: loads read zeros
        int s0 = 0, group = 0, dealt = 0;
        uint64_t pick = 0;
        for (;;) {
            int n_own = 0, my_seg = dead;
            while (n_own < 64) {
                if (!pick) {
                    if (s0 >= a.nseg) break;
                    group = s0;
                    const int sl = s0 + lane;
                    float m = sl < a.nseg && s0 >= 64 * kSegCache ? sm[sl] : -INFINITY;
#pragma unroll
                    for (int j = 0; j < kSegCache; ++j)
                        if (s0 == 64 * j) m = cache[j];
                    pick = ballot(sl < a.nseg && m >= tau);
                    s0 += 64;
                    continue;
                }
                const int p = __builtin_ctzll(pick);
                pick &= pick - 1;
                if ((dealt++ % kFinWaves) == wave) {
                    if (lane == n_own) my_seg = group + p;
                    ++n_own;
                }
            }
            if (n_own == 0) break;
            f32x4 va[kIters], vb[kIters];
            load(va, lane_value(my_seg, 0));
            for (int i = 0; i < n_own; i += 2) {
                const int sa = lane_value(my_seg, i);
                const int sb = i + 1 < 64 ? lane_value(my_seg, i + 1) : dead;  // dead past n_own
                load(vb, sb);
                process(va, sa);
                load(va, i + 2 < 64 ? lane_value(my_seg, i + 2) : dead);
                if (i + 1 < n_own) process(vb, sb);
            }
            if (n_own < 64) break;
        }
        if (lane == 0) { s_len[wave] = tk.lcount + tk.cnt; s_lc[wave] = tk.lcount; }
    }
    __syncthreads();
    // A wave's entries are its list (s_lc of them) followed by its buffer.
    // Usually the four waves hold a few dozen in all; otherwise each wave
    // first reduces its own to at most k.
    int n_tot = 0;
#pragma unroll
    for (int w = 0; w < kFinWaves; ++w) n_tot += s_len[w];
    if (n_tot > 64) {
        if (wave < kFinWaves) {
            if (tk.cnt > 0) topk_compact(tk, s_lv, s_li, s_bv, s_bi, wave, a.k, lane, -INFINITY);
            if (lane == 0) { s_len[wave] = tk.lcount; s_lc[wave] = tk.lcount; }
        }
        __syncthreads();
        n_tot = 0;
#pragma unroll
        for (int w = 0; w < kFinWaves; ++w) n_tot += s_len[w];
    }
    if (wave != 0) return;

    // entry e of the waves' concatenated entries
    auto entry = [&](int e, float& v, int& i) {
        v = -INFINITY;
        i = -1;
        int off = 0;
#pragma unroll
        for (int w = 0; w < kFinWaves; ++w) {
            const int loc = e - off;
            if (loc >= 0 && loc < s_len[w]) {
                v = loc < s_lc[w] ? s_lv[w][loc] : s_bv[w][loc - s_lc[w]];
                i = loc < s_lc[w] ? s_li[w][loc] : s_bi[w][loc - s_lc[w]];
            }
            off += s_len[w];
        }
    };
    auto emit = [&](int rank, float v, int i) {
        a.topk_idx[(size_t)row * a.k + rank] = i;
        a.topk_val[(size_t)row * a.k + rank] = v;
        if (rank == 0 && a.T == 0.f) {
            if (a.lse) a.lse[row] = NAN;
            if (a.draft) a.draft[row] = i;
        }
    };
    if (n_tot <= 64) {
        // One entry per lane.  Only entries >= tau can rank, and the row's
        // top k are among them (k <= V entries of the row exist, so no empty
        // ranks); each of those counts the others ranking ahead of it, so the
        // ranks are 0, 1, ... without repeats (every index appears once).
        float v;
        int i;
        entry(lane, v, i);
        const bool keep = lane < n_tot && v >= tau && i != -1;
        uint64_t kept = ballot(keep);
        int rank = 0;
        while (kept) {
            const int j = __builtin_ctzll(kept);
            kept &= kept - 1;
            const float vj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
            const int ij = __builtin_amdgcn_readlane(i, j);
            rank += ranks_ahead(vj, ij, v, i) ? 1 : 0;
        }
        if (keep && rank < a.k) emit(rank, v, i);
        return;
    }
    // more than 64 entries (k > 16): k rounds of a wave-wide reduction
    float cv[kFinWaves];
    int ci[kFinWaves];
#pragma unroll
    for (int q = 0; q < kFinWaves; ++q) entry(q * 64 + lane, cv[q], ci[q]);
    for (int rr = 0; rr < a.k; ++rr) {
        float bv = cv[0];
        int bi = ci[0];
#pragma unroll
        for (int q = 1; q < kFinWaves; ++q)
            if (ranks_ahead(cv[q], ci[q], bv, bi)) { bv = cv[q]; bi = ci[q]; }
        wave_best(bv, bi);
#pragma unroll
        for (int q = 0; q < kFinWaves; ++q)
            if (ci[q] == bi && ci[q] != -1) { cv[q] = -INFINITY; ci[q] = -1; }
        if (lane == 0) emit(rr, bv, bi);
    }
}

// --------------------------------------------------------- verification
struct VerifyArgs {
    const float* zp;   // target logits [B, G, V]
    const float* zq;   // draft logits  [B, G, V]
    const int32_t* drafts;  // [B, G]
    const double* draft_lse;  // [B, G] or null
    int B, G, V, nseg, wpr;
    float T, c2;
    const uint64_t* seeds;
    uint64_t step;
    const float* p_seg_m;   // target rows' segment stats
    const double* p_seg_s;
    const float* q_seg_m;   // draft rows' segment stats (when draft_lse is null)
    const double* q_seg_s;
    const float* cand_v;    // target rows' per-wave argmax
    const int* cand_i;
    int* seq_j;             // [B]
    f32x4* seq_w;           // [B]: residual weight constants (R_p, R_q, F_p, F_q) of row j
    double* resid_s;        // [B][nseg]
    int32_t* accept_len;
    int32_t* out_tokens;
    uint8_t* accepted;
};

__device__ __forceinline__ int clamp_tok(int d, int V) { return d < 0 ? 0 : (d >= V ? V - 1 : d); }

constexpr int kCommitWaves = 8;  // one wave per block row (gamma <= 8 in one round)

// Verification of one sequence.  The block's rows are spread over the eight
// waves: each merges its rows' statistics with all 64 lanes (target argmax for
// greedy; max and fp64 exp-sum for sampled), gathers p and q at the draft and
// takes the fp64 accept decision.  Wave 0 then forms the accepted prefix and,
// when every draft survived, draws the bonus token from the target's last row.
__global__ void __launch_bounds__(64 * kCommitWaves) verify_commit_kernel(VerifyArgs a) {
    __shared__ int s_acc[32], s_tok[32];
    __shared__ float s_M[32];
    __shared__ double s_S[32], s_lsep[32], s_lseq[32];
    const int b = blockIdx.x, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.G;
    const double Td = (double)a.T;
    for (int r = wave; r < G; r += kCommitWaves) {
        const bool is_draft = r < G - 1;
        // the row's inputs that do not depend on each other are loaded together
        const int d = is_draft ? clamp_tok(a.drafts[(size_t)b * G + r], a.V) : 0;
        const double lseq_in =
            is_draft && a.zq && a.draft_lse && a.T > 0.f ? a.draft_lse[(size_t)b * G + r] : 0.0;
        if (a.T == 0.f) {
            const size_t cb = ((size_t)b * G + r) * a.wpr;
            float bv = -INFINITY;
            int bi = -1;
            for (int w = lane; w < a.wpr; w += 64)
                if (ranks_ahead(a.cand_v[cb + w], a.cand_i[cb + w], bv, bi)) {
                    bv = a.cand_v[cb + w];
                    bi = a.cand_i[cb + w];
                }
            wave_best(bv, bi);
            if (lane == 0) {
                s_tok[r] = bi;
                s_acc[r] = is_draft && d == bi;
            }
            continue;
        }
        // the two logits at the draft are loaded before the row statistics are merged
        float zpd = 0.f, zqd = 0.f;
        if (is_draft && lane == 0) {
            const size_t off = ((size_t)b * G + r) * a.V + d;
            zpd = a.zp[off];
            if (a.zq) zqd = a.zq[off];
        }
        const size_t rb = ((size_t)b * G + r) * a.nseg;
        float M;
        double S;
        merge_row_stats(a.p_seg_m + rb, a.p_seg_s + rb, a.nseg, a.c2, lane, M, S);
        const double lsep = (double)M / Td + log(S);
        double lseq = 0.0;
        if (is_draft && a.zq) {
            if (a.draft_lse) {
                lseq = lseq_in;
            } else {
                float Mq;
                double Sq;
                merge_row_stats(a.q_seg_m + rb, a.q_seg_s + rb, a.nseg, a.c2, lane, Mq, Sq);
                lseq = (double)Mq / Td + log(Sq);
            }
        }
        if (lane == 0) {
            int acc = 0;
            if (is_draft) {
                // deterministic drafts (no draft logits): q is the point mass at d
                const double ratio = a.zq ? exp(((double)zpd - (double)zqd) / Td - lsep + lseq)
                                          : exp((double)zpd / Td - lsep);
                const double u =
                    philox_uniform(a.seeds[b], a.step, (uint64_t)b, (uint64_t)r, kAcceptTest);
                // u < min(1, ratio); a ratio that is NaN (p and q both zero at the
                // draft, e.g. a draft outside a truncated target row) rejects
                acc = ratio >= 1.0 || u < ratio;
            }
            s_acc[r] = acc;
            s_M[r] = M;
            s_S[r] = S;
            s_lsep[r] = lsep;
            s_lseq[r] = lseq;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    const int r = lane;
    const bool is_row = r < G, is_draft = r < G - 1;
    const bool acc = is_draft && s_acc[r];
    const uint64_t accmask = ballot(acc);
    const int lead = __builtin_ctzll(~accmask);
    const int j = lead < G - 1 ? lead : G - 1;
    if (is_draft && a.accepted) a.accepted[(size_t)b * (G - 1) + r] = acc ? 1 : 0;
    int final_tok = -1;
    bool final_known = true;
    if (a.T == 0.f) {
        final_tok = s_tok[j];
    } else if (j == G - 1) {
        const int row = b * G + (G - 1);
        const double u = philox_uniform(a.seeds[b], a.step, (uint64_t)b, (uint64_t)(G - 1), kFinalDraw);
        final_tok = draw_softmax_row(a.zp + (size_t)row * a.V, a.V, a.p_seg_m + (size_t)row * a.nseg,
                                     a.p_seg_s + (size_t)row * a.nseg, a.nseg, a.c2, s_M[G - 1],
                                     s_S[G - 1], u, lane);
    } else {
        final_known = false;  // correction drawn by the residual kernels
        if (lane == 0) {
            // 2^((z - R) c2) F = exp(z / T - LSE) with R = LSE T rounded to fp32, so that the
            // exponent stays near zero; computed once here, loaded by the residual passes
            const double lp = s_lsep[j], lq = s_lseq[j];
            const float Rp = (float)(lp * Td), Rq = (float)(lq * Td);
            a.seq_w[b] = f32x4{Rp, Rq, (float)exp((double)Rp / Td - lp), (float)exp((double)Rq / Td - lq)};
        }
    }
    if (lane == 0) {
        a.accept_len[b] = j;
        a.seq_j[b] = final_known ? -1 : j;
    }
    if (is_row) {
        int tok = r < j ? clamp_tok(a.drafts[(size_t)b * G + r], a.V) : -1;
        if (r == j) tok = final_known ? final_tok : -1;
        a.out_tokens[(size_t)b * G + r] = tok;
    }
}

// Element weight of the residual [p - q]_+ at row j, from the row log-normalisers.
struct ResidualW {
    const float* zpr;
    const float* zqr;  // null: deterministic draft, q = point mass at dq
    int dq;
    float Rp, Rq, Fp, Fq, c2;
    __device__ __forceinline__ f32x4 w4(int v) const {
        const f32x4 zp = *reinterpret_cast<const f32x4*>(zpr + v);
        f32x4 r;
        if (zqr) {
            const f32x4 zq = *reinterpret_cast<const f32x4*>(zqr + v);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float p = fast_exp2((zp[c] - Rp) * c2) * Fp;
                const float q = fast_exp2((zq[c] - Rq) * c2) * Fq;
                r[c] = fmaxf(p - q, 0.f);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float p = fast_exp2((zp[c] - Rp) * c2) * Fp;
                r[c] = v + c == dq ? 0.f : p;  // p - 1 < 0 at the draft, p - 0 elsewhere
            }
        }
        return r;
    }
};

__device__ __forceinline__ ResidualW make_residual(const VerifyArgs& a, int b, int j) {
    ResidualW w;
    const size_t row = (size_t)b * a.G + j;
    w.zpr = a.zp + row * a.V;
    w.zqr = a.zq ? a.zq + row * a.V : nullptr;
    w.dq = a.zq ? -1 : clamp_tok(a.drafts[row], a.V);
    const f32x4 c = a.seq_w[b];
    w.Rp = c[0];
    w.Rq = c[1];
    w.Fp = c[2];
    w.Fq = c[3];
    w.c2 = a.c2;
    return w;
}

// Residual mass per segment of row j, for sequences that rejected a draft.
__global__ void __launch_bounds__(256) verify_residual_kernel(VerifyArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int gw = blockIdx.x * kScanWaves + wave;
    const int b = gw / a.nseg, seg = gw % a.nseg;
    if (b >= a.B) return;
    const int j = a.seq_j[b];
    if (j < 0) return;
    const ResidualW w = make_residual(a, b, j);
    const int base = seg * kSeg + 4 * lane;
    f32x4 t4[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
        // a quad past the row's end reads the last quad and weighs nothing
        const int e = base + it * 256;
        const f32x4 x = w.w4(e < a.V ? e : a.V - 4);
        t4[it] = e < a.V ? x : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    double s = 0.0;
#pragma unroll
    for (int h = 0; h < kIters / 2; ++h) {
        const f32x4 x = t4[2 * h], y = t4[2 * h + 1];
        s += (double)(((x[0] + x[1]) + (x[2] + x[3])) + ((y[0] + y[1]) + (y[2] + y[3])));
    }
    s = wave_sum(s);
    if (lane == 0) a.resid_s[(size_t)b * a.nseg + seg] = s;
}

// Correction draw from [p_j - q_j]_+ (or from p_j when it has no mass).
__global__ void __launch_bounds__(64) verify_draw_kernel(VerifyArgs a) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const int j = a.seq_j[b];
    if (j < 0) return;
    const double u = philox_uniform(a.seeds[b], a.step, (uint64_t)b, (uint64_t)j, kFinalDraw);
    const double* rs = a.resid_s + (size_t)b * a.nseg;
    double tot = 0.0;
    for (int s = lane; s < a.nseg; s += 64) tot += rs[s];
    tot = wave_sum(tot);
    int tok;
    if (tot > 0.0) {
        const ResidualW w = make_residual(a, b, j);
        double before = 0.0;
        auto segw = [&](int s) -> double { return rs[s]; };
        const double target = u * tot;
        const int seg = find_segment(a.nseg, target, segw, lane, before);
        tok = seg < 0 ? 0 : draw_in_segment(seg, a.V, target - before, w, lane);
    } else {
        const int row = b * a.G + j;
        const float* sm = a.p_seg_m + (size_t)row * a.nseg;
        const double* ss = a.p_seg_s + (size_t)row * a.nseg;
        float M;
        double S;
        merge_row_stats(sm, ss, a.nseg, a.c2, lane, M, S);
        tok = draw_softmax_row(a.zp + (size_t)row * a.V, a.V, sm, ss, a.nseg, a.c2, M, S, u, lane);
    }
    if (lane == 0) a.out_tokens[(size_t)b * a.G + j] = tok;
}

// ------------------------------------------------------------- planning
struct ScanPlan {
    int nseg, spw, wpr;
};

ScanPlan plan_scan(long rows, int V) {
    ScanPlan p;
    p.nseg = (V + kSeg - 1) / kSeg;
    long spw = (rows * p.nseg + kTargetWaves - 1) / kTargetWaves;
    if (spw < 1) spw = 1;
    if (spw > p.nseg) spw = p.nseg;
    p.spw = (int)spw;
    p.wpr = (p.nseg + p.spw - 1) / p.spw;
    return p;
}

struct TopKLayout {
    ScanPlan sp;
    size_t seg_m, seg_s, bytes;
};

TopKLayout topk_layout(int batch, int gamma, int vocab) {
    TopKLayout L{};
    const long rows = (long)batch * gamma;
    L.sp = plan_scan(rows, vocab);
    Carve c;
    L.seg_m = c.take<float>((size_t)rows * L.sp.nseg);
    L.seg_s = c.take<double>((size_t)rows * L.sp.nseg);
    L.bytes = c.total();
    return L;
}

struct VerifyLayout {
    ScanPlan sp;
    size_t p_m, p_s, q_m, q_s, cand_v, cand_i, seq_j, seq_w, resid, bytes;
};

VerifyLayout verify_layout(int batch, int gamma, int vocab) {
    VerifyLayout L{};
    const long rows = (long)batch * gamma;
    L.sp = plan_scan(rows, vocab);
    const size_t rs = (size_t)rows * L.sp.nseg;
    Carve c;
    L.p_m = c.take<float>(rs);
    L.p_s = c.take<double>(rs);
    L.q_m = c.take<float>(rs);
    L.q_s = c.take<double>(rs);
    L.cand_v = c.take<float>((size_t)rows * L.sp.wpr);
    L.cand_i = c.take<int>((size_t)rows * L.sp.wpr);
    L.seq_j = c.take<int>((size_t)batch);
    L.seq_w = c.take<f32x4>((size_t)batch);
    L.resid = c.take<double>((size_t)batch * L.sp.nseg);
    L.bytes = c.total();
    return L;
}

bool ws_ok(const void* ws, size_t have, size_t need) {
    return ws && !(reinterpret_cast<uintptr_t>(ws) & 255) && have >= need;
}

template <int MODE>
void launch_scan(const ScanArgs& s, hipStream_t st) {
    const long waves = (long)s.rows * s.wpr;
    hipLaunchKernelGGL((row_scan_kernel<MODE>), dim3((unsigned)((waves + kScanWaves - 1) / kScanWaves)),
                       dim3(64 * kScanWaves), 0, st, s);
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" size_t dflash_topk_workspace_size(int batch, int gamma, int vocab, int k) {
    if (batch < 0 || gamma < 1 || vocab < 1 || k < 1) return 0;
    return topk_layout(batch, gamma, vocab).bytes;
}

extern "C" int dflash_topk(const float* logits, int batch, int gamma, int vocab, int k,
                           float temperature, const uint64_t* seeds, uint64_t step,
                           int32_t* topk_idx, float* topk_val, double* lse, int32_t* draft,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (batch < 0 || gamma < 1 || vocab < 1 || k < 1 || k > vocab) return DFLASH_ERR_SHAPE;
    if (!(temperature >= 0.f) || !std::isfinite(temperature)) return DFLASH_ERR_SHAPE;
    if (batch == 0) return DFLASH_OK;
    if (!logits || !topk_idx || !topk_val) return DFLASH_ERR_NULL;
    if (temperature > 0.f && draft && !seeds) return DFLASH_ERR_NULL;
    if (k > 64 || gamma > 32 || vocab % 4 != 0 || vocab > kMaxVocab) return DFLASH_ERR_UNSUPPORTED;
    const TopKLayout L = topk_layout(batch, gamma, vocab);
    if (!ws_ok(workspace, workspace_bytes, L.bytes)) return DFLASH_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const float c2 = temperature > 0.f ? (float)(1.4426950408889634 / (double)temperature) : 0.f;
    ScanArgs s{logits, batch * gamma, vocab, L.sp.nseg, L.sp.spw, L.sp.wpr, c2,
               reinterpret_cast<float*>(ws + L.seg_m), reinterpret_cast<double*>(ws + L.seg_s),
               nullptr, nullptr};
    if (temperature > 0.f) launch_scan<kSumExp>(s, st);
    else launch_scan<kSegMax>(s, st);
    int rc = launch_status();
    if (rc) return rc;
    TopKFin f{logits, batch, gamma, vocab, L.sp.nseg, k, temperature, c2, seeds, step,
              s.seg_m, s.seg_s, topk_idx, topk_val, lse, draft};
    hipLaunchKernelGGL(topk_finalize_kernel, dim3(batch * gamma), dim3(64 * (kFinWaves + 1)), 0, st, f);
    return launch_status();
}

extern "C" size_t spec_verify_workspace_size(int batch, int gamma, int vocab) {
    if (batch < 0 || gamma < 1 || vocab < 1) return 0;
    return verify_layout(batch, gamma, vocab).bytes;
}

namespace dfl {

int verify_check(const float* target_logits, const int32_t* draft_tokens, float temperature,
                 const uint64_t* seeds, const int32_t* accept_len, const int32_t* out_tokens,
                 int batch, int gamma, int vocab) {
    if (batch < 0 || gamma < 1 || vocab < 1) return DFLASH_ERR_SHAPE;
    if (!(temperature >= 0.f) || !std::isfinite(temperature)) return DFLASH_ERR_SHAPE;
    if (batch == 0) return DFLASH_OK;
    if (!target_logits || !draft_tokens || !accept_len || !out_tokens) return DFLASH_ERR_NULL;
    if (temperature > 0.f && !seeds) return DFLASH_ERR_NULL;
    if (gamma > 32 || vocab % 4 != 0 || vocab > kMaxVocab) return DFLASH_ERR_UNSUPPORTED;
    return DFLASH_OK;
}

size_t verify_scratch_bytes(int batch, int gamma, int vocab) {
    return verify_layout(batch, gamma, vocab).bytes;
}

int verify_enqueue(const float* target_logits, const float* draft_logits,
                   const int32_t* draft_tokens, const double* draft_lse, float temperature,
                   const uint64_t* seeds, uint64_t step, int32_t* accept_len, int32_t* out_tokens,
                   uint8_t* accepted, int batch, int gamma, int vocab, void* scratch_ws,
                   hipStream_t st) {
    const VerifyLayout L = verify_layout(batch, gamma, vocab);
    char* ws = static_cast<char*>(scratch_ws);
    const float c2 = temperature > 0.f ? (float)(1.4426950408889634 / (double)temperature) : 0.f;
    VerifyArgs v{};
    v.zp = target_logits; v.zq = draft_logits; v.drafts = draft_tokens; v.draft_lse = draft_lse;
    v.B = batch; v.G = gamma; v.V = vocab; v.nseg = L.sp.nseg; v.wpr = L.sp.wpr;
    v.T = temperature; v.c2 = c2; v.seeds = seeds; v.step = step;
    v.p_seg_m = reinterpret_cast<float*>(ws + L.p_m);
    v.p_seg_s = reinterpret_cast<double*>(ws + L.p_s);
    v.q_seg_m = reinterpret_cast<float*>(ws + L.q_m);
    v.q_seg_s = reinterpret_cast<double*>(ws + L.q_s);
    v.cand_v = reinterpret_cast<float*>(ws + L.cand_v);
    v.cand_i = reinterpret_cast<int*>(ws + L.cand_i);
    v.seq_j = reinterpret_cast<int*>(ws + L.seq_j);
    v.seq_w = reinterpret_cast<f32x4*>(ws + L.seq_w);
    v.resid_s = reinterpret_cast<double*>(ws + L.resid);
    v.accept_len = accept_len; v.out_tokens = out_tokens; v.accepted = accepted;
    ScanArgs s{target_logits, batch * gamma, vocab, L.sp.nseg, L.sp.spw, L.sp.wpr, c2,
               const_cast<float*>(v.p_seg_m), const_cast<double*>(v.p_seg_s),
               const_cast<float*>(v.cand_v), const_cast<int*>(v.cand_i)};
    if (temperature == 0.f) {
        launch_scan<kArgmax>(s, st);
    } else {
        launch_scan<kSumExp>(s, st);
        if (!draft_lse && draft_logits) {
            ScanArgs q = s;
            q.z = draft_logits;
            q.seg_m = const_cast<float*>(v.q_seg_m);
            q.seg_s = const_cast<double*>(v.q_seg_s);
            launch_scan<kSumExp>(q, st);
        }
    }
    int rc = launch_status();
    if (rc) return rc;
    hipLaunchKernelGGL(verify_commit_kernel, dim3(batch), dim3(64 * kCommitWaves), 0, st, v);
    rc = launch_status();
    if (rc || temperature == 0.f) return rc;
    const long waves = (long)batch * L.sp.nseg;
    hipLaunchKernelGGL(verify_residual_kernel, dim3((unsigned)((waves + kScanWaves - 1) / kScanWaves)),
                       dim3(64 * kScanWaves), 0, st, v);
    rc = launch_status();
    if (rc) return rc;
    hipLaunchKernelGGL(verify_draw_kernel, dim3(batch), dim3(64), 0, st, v);
    return launch_status();
}

}  // namespace dfl

extern "C" int spec_verify(const float* target_logits, const float* draft_logits,
                           const int32_t* draft_tokens, const double* draft_lse,
                           float temperature, const uint64_t* seeds, uint64_t step,
                           int32_t* accept_len, int32_t* out_tokens, uint8_t* accepted,
                           int batch, int gamma, int vocab, void* workspace,
                           size_t workspace_bytes, void* stream) {
    const int rc = verify_check(target_logits, draft_tokens, temperature, seeds, accept_len,
                                out_tokens, batch, gamma, vocab);
    if (rc || batch == 0) return rc;
    if (!ws_ok(workspace, workspace_bytes, verify_scratch_bytes(batch, gamma, vocab)))
        return DFLASH_ERR_WORKSPACE;
    return verify_enqueue(target_logits, draft_logits, draft_tokens, draft_lse, temperature, seeds,
                          step, accept_len, out_tokens, accepted, batch, gamma, vocab, workspace,
                          reinterpret_cast<hipStream_t>(stream));
}
