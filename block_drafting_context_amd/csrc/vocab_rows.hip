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
// One workgroup of 16 waves streams one row, split into 2,048-element
// segments; each wave owns a contiguous run of segments and, per segment,
// holds all 32 of each lane's elements in registers (8 float4 loads issued
// together), so it can take an exact wave-uniform segment maximum m_s before
// exponentiating.  Per segment it produces m_s and, at T > 0,
// s_s = sum 2^((z - m_s) * log2(e)/T) (fp32 pairwise sums, fp64 across); the
// greedy verify scan takes each wave's argmax instead.
//
// dflash_topk is one launch: after the scan the same workgroup finishes its
// row.  tau = the k-th largest m_s of the row (counting repeats) is a lower
// bound of the row's k-th largest entry, since those k maxima are k distinct
// entries, so every top-k entry lies in a segment with m_s >= tau; fifteen
// waves re-read just those segments (about k of them) with tau as the first
// filter, keeping the entries that can still rank in LDS buffers, whose lists
// are rebuilt by k rounds of a wave-wide (value desc, index asc) reduction
// when they fill; the sixteenth wave meanwhile merges the segment statistics
// into the log-normaliser and draws: an inverse-CDF draw needs only the
// segment sums plus one re-read of the single segment holding the crossing,
// recomputing the element weights with exactly the arithmetic that produced
// the sums.
//
// spec_verify is three launches: the row scan (per-row max and fp64
// exp-sum, or argmax, and the segment statistics the draws use); a tail with
// a group of workgroups per sequence, each of which takes the same accept
// decisions from the row statistics (the same arithmetic on the same values,
// so they agree), the first writing the committed tokens and drawing the
// bonus token, and, when a draft was rejected, each wave summing the residual
// [p - q]_+ over one segment of the rejected row; then the correction draw,
// one wave per rejecting sequence.  (Handing the sums to the last workgroup
// of a sequence through a per-sequence atomic counter instead was slower:
// the counters serialise and the device-scope handoff costs a memory round
// trip per wave.)
#include <climits>
#include <cmath>
#include <type_traits>

#include "common.hpp"
#include "verify_run.hpp"

namespace dfl {
DFL_VIOLATION_WORD(violations_rows)
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kSeg = 2048;             // elements per segment (8 x 64 lanes x 4)
constexpr int kIters = kSeg / 256;     // float4 loads per lane per segment
constexpr int kRowWaves = 16;          // waves per row workgroup
constexpr int kRowThreads = 64 * kRowWaves;
constexpr int kFinWaves = kRowWaves - 1;  // top-k candidate waves (the last one draws)
constexpr int kCap = 256;              // top-k candidate buffer fill that triggers a rebuild
constexpr int kBuf = kCap + 256;       // buffer size: one load group (4 x 64) of slack
constexpr int kMaxTopkSeg = 4096;      // top-k: segment statistics held in LDS (V <= 2^23)
constexpr int kTailWaves = 4;          // waves per verification tail workgroup
constexpr int kRsrcWord3 = 0x00020000; // buffer resource word 3 for raw byte buffers on gfx9 parts
constexpr int kMaxVocab = 1 << 29;     // a row's bytes, and a segment past it, fit 32-bit offsets
constexpr int kMaxTopkVocab = kMaxTopkSeg * kSeg;

enum : int { kArgmax = 1, kSumExp = 2, kSegMax = 4 };

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

// raw buffer over one row (V % 4 == 0, V <= 2^29: V * 4 bytes fit 32 bits)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* zr, int V) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(zr), (short)0,
                                             (int)((uint32_t)V * 4u), kRsrcWord3);
}

// The 32 elements of this lane in segment `seg`: base + it*256 + c.  Every
// load is issued unconditionally: a quad past the row's end (V % 4 == 0, so
// quads are whole) or of a segment past a wave's run reads as zeros without
// touching memory, and the compiler counts the loads in flight exactly.
__device__ __forceinline__ void load_segment(f32x4 (&v)[kIters], __amdgpu_buffer_rsrc_t rsrc, int seg,
                                             int lane) {
    const uint32_t base = (uint32_t)(seg * kSeg + 4 * lane) * 4u;  // < 2^32: V <= 2^29
#pragma unroll
    for (int it = 0; it < kIters; ++it)
        // logits rows are streamed once: non-temporal loads
        v[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              rsrc, (int)(base + it * 1024u), 0, kLoadStream));
}

// The nucleus inside a run of entries that lies wholly at or below a cut's
// index (keep z >= logit) or wholly above it (keep z > logit, which for the
// finite or -inf logits of the domain is z >= the next float up; denormals
// are not flushed): one comparison per entry.
struct ThrCut {
    float thr;
    __device__ __forceinline__ float one(float z, int) const { return z >= thr ? z : -INFINITY; }
};
// Top-p nucleus of a row (dflash_nucleus_cut): entry (z, v) is kept iff
// z > logit, or z == logit and v <= index; an entry outside it is taken as
// -inf, exactly as in a row masked to its nucleus.  NoCut keeps every entry
// and compiles to nothing.
struct RowCut {
    float logit;
    int index;
    __device__ __forceinline__ float one(float z, int v) const {
        return (z > logit || (z == logit && v <= index)) ? z : -INFINITY;
    }
    __device__ __forceinline__ void quad(f32x4& q, int v0) const {
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = one(q[c], v0 + c);
    }
    // Entries s0 .. s0 + len - 1 as one threshold, when they lie wholly on
    // one side of the index.
    __device__ __forceinline__ bool seg_uniform(int s0, int len, ThrCut& t) const {
        if (s0 + len - 1 <= index) {
            t.thr = logit;
            return true;
        }
        if (s0 > index) {
            // the next float above logit; above either zero, the smallest
            // positive float (-inf: -FLT_MAX)
            const uint32_t bits = __float_as_uint(logit);
            t.thr = logit == 0.f ? __uint_as_float(1u)
                                 : __uint_as_float((bits & 0x80000000u) ? bits - 1u : bits + 1u);
            return true;
        }
        return false;
    }
    // The lane's entries v[it][c] = entry base + it*256 + c of segment `seg`
    // (wave-uniform).  Within a segment v <= index holds for every entry or
    // for none, except in the one segment holding `index`: one comparison
    // per entry elsewhere.
    __device__ __forceinline__ void segment(f32x4 (&v)[kIters], int seg, int base) const {
        const int s0 = seg * kSeg;
        if (s0 + kSeg - 1 <= index) {
#pragma unroll
            for (int it = 0; it < kIters; ++it)
#pragma unroll
                for (int c = 0; c < 4; ++c) v[it][c] = v[it][c] >= logit ? v[it][c] : -INFINITY;
        } else if (s0 > index) {
#pragma unroll
            for (int it = 0; it < kIters; ++it)
#pragma unroll
                for (int c = 0; c < 4; ++c) v[it][c] = v[it][c] > logit ? v[it][c] : -INFINITY;
        } else {
#pragma unroll
            for (int it = 0; it < kIters; ++it) quad(v[it], base + it * 256);
        }
    }
};
struct NoCut {
    __device__ __forceinline__ float one(float z, int) const { return z; }
    __device__ __forceinline__ void quad(f32x4&, int) const {}
    __device__ __forceinline__ void segment(f32x4 (&)[kIters], int, int) const {}
};
// The cut of row `row`, or one that keeps everything when the caller gave no
// cuts; the load is issued either way (from `valid`, any readable 8 bytes).
__device__ __forceinline__ RowCut row_cut(const dflash_nucleus_cut* cuts, size_t row, const void* valid) {
    const dflash_nucleus_cut c = *(cuts ? cuts + row : reinterpret_cast<const dflash_nucleus_cut*>(valid));
    return cuts ? RowCut{c.logit, c.index} : RowCut{-INFINITY, INT_MAX};
}
// Kernels that take cuts are instantiated twice: with RowCut when the caller
// gave cuts, with NoCut (no per-entry test at all) when not.
template <bool CUT>
using CutOf = typename std::conditional<CUT, RowCut, NoCut>::type;
template <bool CUT>
__device__ __forceinline__ CutOf<CUT> cut_of(const dflash_nucleus_cut* cuts, size_t row, const void* valid) {
    if constexpr (CUT) return row_cut(cuts, row, valid);
    else return NoCut{};
}
// lane j's cut, in every lane
__device__ __forceinline__ RowCut cut_from_lane(const RowCut& c, int j) {
    return RowCut{__builtin_bit_cast(float, lane_value(__builtin_bit_cast(int, c.logit), j)), lane_value(c.index, j)};
}
__device__ __forceinline__ NoCut cut_from_lane(const NoCut&, int) { return NoCut{}; }

// ------------------------------------------------------------ row scan
// Wave `wave` of a row workgroup streams its run of segments and stores each
// segment's maximum (and, with kSumExp, its exp-sum) through lane 0 into
// sm[seg] / ss[seg] (LDS or global); with kArgmax it keeps its argmax.
// hook(v, qm, seg) then sees the segment's values (entries past the row's end
// and, with a cut, entries outside the row's nucleus set to -inf) and the
// lane's quad maxima qm[it] = max of v[it].
struct NoHook {
    __device__ __forceinline__ void operator()(f32x4 (&)[kIters], const float (&)[kIters], int) const {}
};
template <int MODE, class MArr, class SArr, class Hook = NoHook, class CutT = NoCut>
__device__ __forceinline__ void scan_row(const float* zr, int V, int nseg, float c2, MArr sm, SArr ss,
                                         float& best_v, int& best_i, int wave, int lane,
                                         Hook hook = Hook(), CutT cut = CutT()) {
    const int seg0 = (int)((long)wave * nseg / kRowWaves);
    const int seg1 = (int)((long)(wave + 1) * nseg / kRowWaves);
    const __amdgpu_buffer_rsrc_t rsrc = row_rsrc(zr, V);
    best_v = -INFINITY;
    best_i = -1;
    auto process = [&](f32x4 (&v)[kIters], int seg) {
        const int base = seg * kSeg + 4 * lane;
        if (seg * kSeg + kSeg > V) {
            // quads past the row's end read as zeros: they take no part
#pragma unroll
            for (int it = 0; it < kIters; ++it)
                if (base + it * 256 >= V) v[it] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
        cut.segment(v, seg, base);
        if (MODE & kArgmax) {
#pragma unroll
            for (int it = 0; it < kIters; ++it)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (v[it][c] > best_v) { best_v = v[it][c]; best_i = base + it * 256 + c; }
        }
        float qm[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) qm[it] = fmaxf(fmaxf(v[it][0], v[it][1]), fmaxf(v[it][2], v[it][3]));
        if (MODE & (kSumExp | kSegMax)) {
            float lane_m = -INFINITY;
#pragma unroll
            for (int it = 0; it < kIters; ++it) lane_m = fmaxf(lane_m, qm[it]);
            const float m = wave_max(lane_m);
            double sacc = 0.0;
            if ((MODE & kSumExp) && m != -INFINITY) {
#pragma unroll
                for (int h = 0; h < kIters / 2; ++h) {
                    float w[8];
#pragma unroll
                    for (int q = 0; q < 2; ++q)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            w[q * 4 + c] = fast_exp2((v[2 * h + q][c] - m) * c2);
                    const float t = ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
                    sacc += (double)t;
                }
            }
            if (MODE & kSumExp) sacc = wave_sum(sacc);
            if (lane == 0) {
                sm[seg] = m;
                if (MODE & kSumExp) ss[seg] = sacc;
            }
        }
        hook(v, qm, seg);
    };
    // two segments per trip, each one's loads issued before the other is
    // processed; a segment past the run is loaded from past the row's end
    const int dead = nseg;
    f32x4 va[kIters], vb[kIters];
    load_segment(va, rsrc, seg0 < seg1 ? seg0 : dead, lane);
    for (int seg = seg0; seg < seg1; seg += 2) {
        const bool has_b = seg + 1 < seg1;
        load_segment(vb, rsrc, has_b ? seg + 1 : dead, lane);
        process(va, seg);
        load_segment(va, rsrc, seg + 2 < seg1 ? seg + 2 : dead, lane);
        if (has_b) process(vb, seg + 1);
    }
}

// ----------------------------------------------------------- draws
// Merge a row's segment statistics: M = max m_s, S = sum s_s 2^((m_s - M) c2)
// (each lane sums its segments lane, lane + 64, ... in that order).  The
// first 64 * kStatRegs segments are loaded at once into registers (addresses
// clamped into the row, so no load sits behind a branch), the rest in a loop.
constexpr int kStatRegs = 4;
template <class MArr, class SArr>
__device__ __forceinline__ void merge_row_stats(MArr sm, SArr ss, int nseg, float c2, int lane, float& M,
                                                double& S) {
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
// index) exceeds tgt; wfn.load(v) reads what elements v..v+3 need and
// wfn.w4(raw, v) gives their fp32 weights (the same arithmetic that produced
// the segment sums), summed in fp64.  Falls back to the last positive-weight
// element of the segment when rounding leaves no crossing.  Wave-wide; every
// lane returns the index.
template <class WFn>
__device__ __forceinline__ int draw_in_segment(int seg, int V, double tgt, const WFn& wfn, int lane) {
    const int lo = seg * kSeg + lane * 32;
    float w[32];
    // all eight quads' loads are issued before any is used (raw buffer loads:
    // a quad past the row's end reads zeros and weighs nothing)
    typename WFn::Raw raw[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) raw[q] = wfn.load(lo + 4 * q);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int v = lo + 4 * q;
        const f32x4 w4 = wfn.w4(raw[q], v);
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

// 16 bytes at element v of a row (zeros past its end)
__device__ __forceinline__ f32x4 load_quad(__amdgpu_buffer_rsrc_t rsrc, int v) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)((uint32_t)v * 4u), 0,
                                                                           kLoadDefault));
}

// Weight 2^((z - m_s) * c2) of softmax(z / T) relative to a segment maximum
// (0 outside the row's nucleus).
template <class CutT>
struct SoftmaxW {
    __amdgpu_buffer_rsrc_t zr;
    float ms, c2;
    CutT cut;
    typedef f32x4 Raw;
    __device__ __forceinline__ Raw load(int v) const { return load_quad(zr, v); }
    __device__ __forceinline__ f32x4 w4(const Raw& z, int v) const {
        f32x4 r;
#pragma unroll
        for (int c = 0; c < 4; ++c) r[c] = fast_exp2((cut.one(z[c], v + c) - ms) * c2);
        return r;
    }
};

// Draw from softmax(z / T) of one row (restricted to its nucleus, with a
// cut) using its segment statistics.
template <class MArr, class SArr, class CutT = NoCut>
__device__ __forceinline__ int draw_softmax_row(const float* zr, int V, MArr sm, SArr ss, int nseg, float c2,
                                                float M, double S, double u, int lane, CutT cut = CutT()) {
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
    if constexpr (std::is_same<CutT, RowCut>::value) {
        ThrCut t;
        if (cut.seg_uniform(seg * kSeg, kSeg, t)) {
            const SoftmaxW<ThrCut> wfn{row_rsrc(zr, V), ms, c2, t};
            return draw_in_segment(seg, V, tgt, wfn, lane);
        }
    }
    const SoftmaxW<CutT> wfn{row_rsrc(zr, V), ms, c2, cut};
    return draw_in_segment(seg, V, tgt, wfn, lane);
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
    // both the old filter and the new one bound the row's k-th largest entry from below
    s.tv = fmaxf(s.tv, newcount == k ? fmaxf(lastv, floor) : floor);
}

// The k-th largest of a row's segment maxima (LDS), counting repeats; -inf
// when fewer than k of them are above -inf.  Each round takes the largest
// maximum below the previous one and counts its copies, so at most k rounds.
__device__ __forceinline__ float kth_segment_max(const float* sm, int nseg, int k, int lane) {
    float t = INFINITY;
    int counted = 0;
    for (;;) {
        float m = -INFINITY;
        for (int s = lane; s < nseg; s += 64) {
            const float x = sm[s];
            if (x < t) m = fmaxf(m, x);
        }
        m = wave_max(m);
        if (m == -INFINITY) return -INFINITY;
        for (int s0 = 0; s0 < nseg; s0 += 64)
            counted += __popcll(ballot(s0 + lane < nseg && sm[s0 + lane] == m));
        if (counted >= k) return m;
        t = m;
    }
}

// The k-th largest of the wave's 64 values counting repeats, or -inf when
// fewer than k are above -inf: at most k rounds, each taking the largest
// value left and counting its copies.
__device__ __forceinline__ float wave_kth_largest(float x, int k) {
    int counted = 0;
    for (;;) {
        const float m = wave_max(x);
        if (m == -INFINITY) return -INFINITY;
        const uint64_t at = ballot(x == m);
        counted += __popcll(at);
        if (counted >= k) return m;
        x = x == m ? -INFINITY : x;
    }
}

// --------------------------------------------------------------- top-k
struct TopKArgs {
    const float* z;
    const dflash_nucleus_cut* cut;  // [rows] (CUT instantiations only)
    int B, G, V, nseg, k;
    float T, c2;
    const uint64_t* seeds;
    uint64_t step;
    int32_t* topk_idx;
    float* topk_val;
    double* lse;
    int32_t* draft;
};

// One row per workgroup of sixteen waves: the scan, then waves 0-14 find tau
// and the top k while wave 15 merges the log-normaliser and draws.  CUT: every
// read of the row applies the row's nucleus cut.
template <int MODE, bool CUT>
__global__ void __launch_bounds__(kRowThreads) topk_row_kernel(TopKArgs a) {
    __shared__ __attribute__((aligned(16))) float s_m[kMaxTopkSeg];
    __shared__ double s_s[kMaxTopkSeg];
    __shared__ float s_lv[kFinWaves][64];
    __shared__ int s_li[kFinWaves][64];
    __shared__ __attribute__((aligned(16))) float s_bv[kFinWaves][kBuf];
    __shared__ __attribute__((aligned(16))) int s_bi[kFinWaves][kBuf];
    __shared__ int s_len[kFinWaves], s_lc[kFinWaves];
    __shared__ __attribute__((aligned(16))) float f_v[kRowThreads];
    __shared__ __attribute__((aligned(16))) int f_i[kRowThreads];
    __shared__ float s_tau;
    __shared__ int s_nf;
    const int row = blockIdx.x, lane = threadIdx.x & 63, tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b = row / a.G, r = row % a.G;
    const float* zr = a.z + (size_t)row * a.V;
    // the draw's uniform depends on no data: computed before the scan
    const bool draws = wave == kFinWaves && a.T > 0.f && a.draft;
    const double u_draw = draws ? philox_uniform(a.seeds[b], a.step, (uint64_t)b, (uint64_t)r, kDraftDraw) : 0.0;
    typedef typename std::conditional<CUT, RowCut, NoCut>::type CutT;
    CutT cut{};
    if constexpr (CUT) cut = RowCut{a.cut[row].logit, a.cut[row].index};

    {
        float bv;
        int bi;
        scan_row<MODE>(zr, a.V, a.nseg, a.c2, s_m, s_s, bv, bi, wave, lane, NoHook(), cut);
    }
    if (tid == 0) { s_tau = -INFINITY; s_nf = 0; }
    __syncthreads();

    // tau: the k-th largest segment maximum counting repeats, i.e. the one
    // ranked k-1 in (value desc, segment asc) order; each thread ranks its
    // segments by counting the ones ahead (-inf stays when fewer than k
    // segments exist).  Rows of more than 1,024 segments take k rounds of a
    // wave-wide maximum instead.
    if (a.nseg <= kRowThreads) {
        if (tid < a.nseg) {
            const float mt = s_m[tid];
            int rank = 0;
            int q = 0;
            for (; q + 4 <= a.nseg; q += 4) {
                const f32x4 m4 = *reinterpret_cast<const f32x4*>(&s_m[q]);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    rank += (m4[c] > mt || (m4[c] == mt && q + c < tid)) ? 1 : 0;
            }
            for (; q < a.nseg; ++q) rank += (s_m[q] > mt || (s_m[q] == mt && q < tid)) ? 1 : 0;
            if (rank == a.k - 1) s_tau = mt;
        }
    } else if (wave == 0) {
        const float t = kth_segment_max(s_m, a.nseg, a.k, lane);
        if (lane == 0) s_tau = t;
    }
    __syncthreads();
    const float tau = s_tau;

    TopKRegs tk{0, 0, -INFINITY};
    if (wave == kFinWaves) {
        if (a.T > 0.f) {
            float M;
            double S;
            merge_row_stats(s_m, s_s, a.nseg, a.c2, lane, M, S);
            if (a.lse && lane == 0) a.lse[row] = (double)M / (double)a.T + log(S);
            if (a.draft) {
                const int tok = draw_softmax_row(zr, a.V, s_m, s_s, a.nseg, a.c2, M, S, u_draw, lane, cut);
                if (lane == 0) a.draft[row] = tok;
            }
        }
    } else {
        const __amdgpu_buffer_rsrc_t zr_rsrc = row_rsrc(zr, a.V);
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
            cut.segment(v, seg, base);
            float qm[kIters];
#pragma unroll
            for (int it = 0; it < kIters; ++it) {
                // quads past the row's end read as zeros: they take no part
                if (base + it * 256 >= a.V) v[it] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                qm[it] = fmaxf(fmaxf(v[it][0], v[it][1]), fmaxf(v[it][2], v[it][3]));
            }
            if (tk.tv == -INFINITY && a.k <= 64) {
                // no bound yet (fewer than k segments above -inf, e.g. a
                // short row): k of the 64 lanes each hold an entry >= the
                // k-th largest lane maximum, so it bounds the row's k-th
                // largest entry from below and the filter may start there
                float lm = qm[0];
#pragma unroll
                for (int it = 1; it < kIters; ++it) lm = fmaxf(lm, qm[it]);
                tk.tv = wave_kth_largest(lm, a.k);
            }
#pragma unroll
            for (int it = 0; it < kIters; ++it) {
                pass[it] = qm[it] >= tk.tv;
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

        // The segments with m_s >= tau are dealt to the candidate waves in
        // index order (the i-th to wave i mod kFinWaves).  Collect up to 64 of
        // this wave's segments (lane i holds the i-th), then stream them two
        // at a time; repeat while segments remain.
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
                    const float m = sl < a.nseg ? s_m[sl] : -INFINITY;
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
            load_segment(va, zr_rsrc, lane_value(my_seg, 0), lane);
            for (int i = 0; i < n_own; i += 2) {
                const int sa = lane_value(my_seg, i);
                const int sb = i + 1 < 64 ? lane_value(my_seg, i + 1) : dead;  // dead past n_own
                load_segment(vb, zr_rsrc, sb, lane);
                process(va, sa);
                load_segment(va, zr_rsrc, i + 2 < 64 ? lane_value(my_seg, i + 2) : dead, lane);
                if (i + 1 < n_own) process(vb, sb);
            }
            if (n_own < 64) break;
        }
        if (lane == 0) { s_len[wave] = tk.lcount + tk.cnt; s_lc[wave] = tk.lcount; }
    }
    __syncthreads();
    // A wave's entries are its list (s_lc of them) followed by its buffer.
    // When they fit one per thread, the entries >= tau are gathered into one
    // flat array and each thread ranks one of them by counting the entries
    // ranked ahead of it: only entries >= tau can rank (tau is at most the
    // row's k-th largest value), the row's top k are among them (k <= V
    // entries exist, so no empty ranks), and every index appears once, so the
    // ranks are 0, 1, ...
    int n_tot = 0;
#pragma unroll
    for (int w = 0; w < kFinWaves; ++w) n_tot += s_len[w];
    auto emit = [&](int rank, float v, int i) {
        a.topk_idx[(size_t)row * a.k + rank] = i;
        a.topk_val[(size_t)row * a.k + rank] = v;
        if (rank == 0 && a.T == 0.f) {
            if (a.lse) a.lse[row] = NAN;
            if (a.draft) a.draft[row] = i;
        }
    };
    if (n_tot <= kRowThreads) {
        if (wave < kFinWaves) {
            const int len = s_len[wave], lc = s_lc[wave];
            for (int e0 = 0; e0 < len; e0 += 64) {
                const int e = e0 + lane;
                float v = -INFINITY;
                int i = -1;
                if (e < len) {
                    v = e < lc ? s_lv[wave][e] : s_bv[wave][e - lc];
                    i = e < lc ? s_li[wave][e] : s_bi[wave][e - lc];
                }
                const bool keep = e < len && v >= tau && i != -1;
                const uint64_t m = ballot(keep);
                int at = 0;
                if (lane == 0 && m) at = atomicAdd(&s_nf, __popcll(m));
                at = lane_value(at, 0) + lanes_below(m);
                if (keep) { f_v[at] = v; f_i[at] = i; }
            }
        }
        __syncthreads();
        const int nf = s_nf;
        if (tid < nf) {
            const float v = f_v[tid];
            const int i = f_i[tid];
            int rank = 0;
            int e = 0;
            for (; e + 4 <= nf; e += 4) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(&f_v[e]);
                const i32x4 i4 = *reinterpret_cast<const i32x4*>(&f_i[e]);
#pragma unroll
                for (int c = 0; c < 4; ++c) rank += ranks_ahead(v4[c], i4[c], v, i) ? 1 : 0;
            }
            for (; e < nf; ++e) rank += ranks_ahead(f_v[e], f_i[e], v, i) ? 1 : 0;
            if (rank < a.k) emit(rank, v, i);
        }
        return;
    }
    // many entries (long runs of equal logits): each wave first reduces its
    // own to at most k, then wave 0 takes k rounds over the lists
    if (wave < kFinWaves) {
        if (tk.cnt > 0) topk_compact(tk, s_lv, s_li, s_bv, s_bi, wave, a.k, lane, -INFINITY);
        if (lane == 0) { s_len[wave] = tk.lcount; s_lc[wave] = tk.lcount; }
    }
    __syncthreads();
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
    // k rounds of a wave-wide reduction over the waves' lists (each at most
    // k <= 64 entries)
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
struct RowArgs {
    const float* zp;    // target logits [B, G, V]: rows 0 .. rows-1 of the launch
    const float* zq;    // drafter logits [B, G, V]: rows rows .. 2 rows-1 (log-normaliser only)
    const dflash_nucleus_cut* tcut;  // [B G] or null, for the target rows (CUT only)
    const dflash_nucleus_cut* dcut;  // [B G] or null, for the drafter rows
    int rows, V, nseg, B;
    float c2;
    float* seg_m;       // [launch rows][nseg]
    double* seg_s;
    float* row_M;       // [launch rows]
    double* row_S;
    int* row_arg;       // [rows] (greedy)
};

// Statistics of one target (or drafter) row per workgroup: the segment
// statistics (global, for the draws) and the row's M and S, or its argmax.
// CUT: the row is read through its nucleus cut (if its side has cuts).
template <int MODE, bool CUT>
__global__ void __launch_bounds__(kRowThreads) verify_row_kernel(RowArgs a) {
    __shared__ float s_v[kRowWaves];
    __shared__ int s_i[kRowWaves];
    const int row = blockIdx.x, lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float* zr = row < a.rows ? a.zp + (size_t)row * a.V : a.zq + (size_t)(row - a.rows) * a.V;
    float* sm = a.seg_m + (size_t)row * a.nseg;
    double* ss = a.seg_s + (size_t)row * a.nseg;
    float bv;
    int bi;
    if constexpr (CUT) {
        const RowCut cut = row < a.rows ? row_cut(a.tcut, row, zr) : row_cut(a.dcut, row - a.rows, zr);
        scan_row<MODE>(zr, a.V, a.nseg, a.c2, sm, ss, bv, bi, wave, lane, NoHook(), cut);
    } else {
        scan_row<MODE>(zr, a.V, a.nseg, a.c2, sm, ss, bv, bi, wave, lane);
    }
    if (MODE & kArgmax) {
        wave_best(bv, bi);
        if (lane == 0) { s_v[wave] = bv; s_i[wave] = bi; }
        __syncthreads();
        if (threadIdx.x == 0) {
            float v = s_v[0];
            int i = s_i[0];
#pragma unroll
            for (int w = 1; w < kRowWaves; ++w) best_of(v, i, s_v[w], s_i[w]);
            a.row_arg[row] = i;
        }
    } else {
        // the segment statistics were stored by the waves of this workgroup
        __syncthreads();
        if (wave == 0) {
            float M;
            double S;
            merge_row_stats(sm, ss, a.nseg, a.c2, lane, M, S);
            if (lane == 0) {
                a.row_M[row] = M;
                a.row_S[row] = S;
            }
        }
    }
}

// What the correction draw needs of a sequence that rejected a draft (j < 0:
// nothing to draw).
struct SeqDraw {
    int j, dq;              // first rejected row; the deterministic draft there (-1 with draft logits)
    float Rp, Rq, Fp, Fq;   // residual weight constants of row j
    float Mj;               // row j's maximum and exp-sum (fallback draw from p_j)
    double Sj;
};

struct TailArgs {
    const float* zp;   // target logits [B, G, V]
    const float* zq;   // draft logits  [B, G, V] or null
    const int32_t* drafts;  // [B, G]
    const double* draft_lse;  // [B, G] or null
    const dflash_nucleus_cut* tcut;  // [B, G] or null: nuclei of the target rows
    const dflash_nucleus_cut* dcut;  // [B, G] or null: nuclei of the drafter rows
    int B, G, V, nseg, nr;    // nr: workgroups per sequence
    float T, c2;
    const uint64_t* seeds;
    uint64_t step;
    const float* seg_m;     // target rows' segment statistics
    const double* seg_s;
    const float* row_M;     // [2 B G]: target rows, then drafter rows
    const double* row_S;
    const int* row_arg;     // [B G]
    double* resid_s;        // [B][nseg]
    SeqDraw* seq;           // [B]
    int32_t* accept_len;
    int32_t* out_tokens;
    uint8_t* accepted;
};

__device__ __forceinline__ int clamp_tok(int d, int V) { return d < 0 ? 0 : (d >= V ? V - 1 : d); }

// Element weight of the residual [p - q]_+ at row j, from the row
// log-normalisers.  Both rows are read through raw buffers; without draft
// logits (deterministic draft, q = point mass at dq) the drafter's buffer is
// empty and reads as zeros.
template <class CutT>
struct ResidualW {
    __amdgpu_buffer_rsrc_t zp, zq;
    bool has_q;
    int dq;
    float Rp, Rq, Fp, Fq, c2;
    CutT cp, cq;  // the rows' nuclei (NoCut: keep everything)
    struct Raw {
        f32x4 p, q;
    };
    __device__ __forceinline__ Raw load(int v) const { return Raw{load_quad(zp, v), load_quad(zq, v)}; }
    __device__ __forceinline__ f32x4 w4(const Raw& z, int v) const {
        f32x4 r;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float p = fast_exp2((cp.one(z.p[c], v + c) - Rp) * c2) * Fp;
            const float q = fast_exp2((cq.one(z.q[c], v + c) - Rq) * c2) * Fq;
            // point-mass q: p - 1 < 0 at the draft, p - 0 elsewhere
            r[c] = has_q ? fmaxf(p - q, 0.f) : (v + c == dq ? 0.f : p);
        }
        return r;
    }
};

// The same weights with other cut tests.
template <class CutT, class CutU>
__device__ __forceinline__ ResidualW<CutU> with_cuts(const ResidualW<CutT>& w, CutU cp, CutU cq) {
    ResidualW<CutU> r;
    r.zp = w.zp;
    r.zq = w.zq;
    r.has_q = w.has_q;
    r.dq = w.dq;
    r.Rp = w.Rp;
    r.Rq = w.Rq;
    r.Fp = w.Fp;
    r.Fq = w.Fq;
    r.c2 = w.c2;
    r.cp = cp;
    r.cq = cq;
    return r;
}

// Verification tail: a group of a.nr workgroups per sequence (one when
// greedy).  Every wave takes the accept decisions of the whole block, lane r
// for block row r (the same arithmetic on the same values in every wave, so
// all agree); workgroup 0's first wave writes the committed tokens, draws the
// bonus and records what the correction draw needs; on a rejection every wave
// sums the residual over one segment of the rejected row.
template <bool CUT>
__global__ void __launch_bounds__(64 * kTailWaves) verify_tail_kernel(TailArgs a) {
    typedef CutOf<CUT> CutT;
    const int b = blockIdx.x / a.nr, n = blockIdx.x % a.nr;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = a.G;
    const double Td = (double)a.T;
    const size_t BG = (size_t)a.B * G;

    // ---- the block's decisions: lane r for row r.  Every load that does not
    // depend on the draft is issued with it, unconditionally (pointers that
    // do not apply are replaced by valid ones whose values go unused), then
    // the two logits at the draft.
    const int r = lane;
    const bool is_row = r < G, is_draft = r < G - 1;
    const size_t row = (size_t)b * G + (is_row ? r : G - 1);
    const int d_raw = a.drafts[row];
    const int tok_arg = a.row_arg[row];
    const float M = a.row_M[row];
    const double S = a.row_S[row];
    const float Mq = a.row_M[BG + row];
    const double Sq = a.row_S[BG + row];
    const double lse_given = (a.draft_lse ? a.draft_lse : a.row_S)[row];
    const uint64_t seed = *(a.seeds ? a.seeds + b : reinterpret_cast<const uint64_t*>(a.row_S));
    const int d = is_draft ? clamp_tok(d_raw, a.V) : 0;
    const CutT tc = cut_of<CUT>(a.tcut, row, a.row_S);
    const CutT dc = cut_of<CUT>(a.dcut, row, a.row_S);
    const float zpd = tc.one(a.zp[row * a.V + d], d);
    const float zqd = dc.one((a.zq ? a.zq : a.zp)[row * a.V + d], d);
    int acc = 0;
    double lsep = 0.0, lseq = 0.0;
    if (a.T == 0.f) {
        acc = is_draft && d == tok_arg;
    } else {
        lsep = (double)M / Td + log(S);
        if (a.zq) lseq = a.draft_lse ? lse_given : (double)Mq / Td + log(Sq);
        if (is_draft) {
            // deterministic drafts (no draft logits): q is the point mass at d
            const double ratio = a.zq ? exp(((double)zpd - (double)zqd) / Td - lsep + lseq)
                                      : exp((double)zpd / Td - lsep);
            const double u = philox_uniform(seed, a.step, (uint64_t)b, (uint64_t)r, kAcceptTest);
            // u < min(1, ratio); a ratio that is NaN (p and q both zero at the
            // draft, e.g. a draft outside a truncated target row) rejects
            acc = ratio >= 1.0 || u < ratio;
        }
    }
    const uint64_t accmask = ballot(is_draft && acc);
    const int lead = __builtin_ctzll(~accmask);
    const int j = lead < G - 1 ? lead : G - 1;
    const bool rejected = a.T > 0.f && j < G - 1;

    if (n == 0 && wave == 0) {
        if (DFLASH_DEVICE_CHECKS && is_draft && (d_raw < 0 || d_raw >= a.V)) DFL_VIOLATION(DFLASH_VIOLATION_TOKEN);
        if (is_draft && a.accepted) a.accepted[(size_t)b * (G - 1) + r] = acc ? 1 : 0;
        int final_tok = -1;
        if (a.T == 0.f) {
            final_tok = lane_value(tok_arg, j);
        } else if (!rejected) {
            const size_t rl = (size_t)b * G + (G - 1);
            const float Ml = __builtin_bit_cast(float, lane_value(__builtin_bit_cast(int, M), G - 1));
            const double Sl = lane_value(S, G - 1);
            const double u = philox_uniform(seed, a.step, (uint64_t)b, (uint64_t)(G - 1), kFinalDraw);
            const CutT cl = cut_from_lane(tc, G - 1);
            final_tok = draw_softmax_row(a.zp + rl * a.V, a.V, a.seg_m + rl * a.nseg, a.seg_s + rl * a.nseg,
                                         a.nseg, a.c2, Ml, Sl, u, lane, cl);
        }
        if (lane == 0) a.accept_len[b] = j;
        if (a.T > 0.f) {
            // the correction draw's record (j = -1: nothing to draw)
            const double lpj = lane_value(lsep, j), lqj = lane_value(lseq, j);
            SeqDraw sd;
            sd.j = rejected ? j : -1;
            sd.dq = a.zq ? -1 : lane_value(d, j);
            sd.Rp = (float)(lpj * Td);
            sd.Rq = (float)(lqj * Td);
            sd.Fp = (float)exp((double)sd.Rp / Td - lpj);
            sd.Fq = (float)exp((double)sd.Rq / Td - lqj);
            sd.Mj = __builtin_bit_cast(float, lane_value(__builtin_bit_cast(int, M), j));
            sd.Sj = lane_value(S, j);
            if (lane == 0) a.seq[b] = sd;
        }
        // position j of a rejecting sequence is written by the correction draw
        if (is_row && !(rejected && r == j)) {
            int tok = r < j ? d : -1;
            if (r == j) tok = final_tok;
            a.out_tokens[(size_t)b * G + r] = tok;
        }
    }
    if (!rejected) return;
    const int seg = n * kTailWaves + wave;
    if (seg >= a.nseg) return;

    // residual [p_j - q_j]_+: weights 2^((z - R) c2) F = exp(z / T - LSE) with
    // R = LSE T rounded to fp32, so that the exponent stays near zero
    const double lp = lane_value(lsep, j), lq = lane_value(lseq, j);
    ResidualW<CutT> w;
    const size_t rowj = (size_t)b * G + j;
    const float* zpr = a.zp + rowj * a.V;
    w.zp = row_rsrc(zpr, a.V);
    w.zq = row_rsrc(a.zq ? a.zq + rowj * a.V : zpr, a.zq ? a.V : 0);
    w.has_q = a.zq != nullptr;
    w.dq = a.zq ? -1 : lane_value(d, j);
    w.Rp = (float)(lp * Td);
    w.Rq = (float)(lq * Td);
    w.Fp = (float)exp((double)w.Rp / Td - lp);
    w.Fq = (float)exp((double)w.Rq / Td - lq);
    w.c2 = a.c2;
    w.cp = cut_from_lane(tc, j);
    w.cq = cut_from_lane(dc, j);
    const int base = seg * kSeg + 4 * lane;
    auto segment_sum = [&](const auto& wfn) {
        // the segment's loads of both rows are issued before any is used (a
        // quad past the row's end reads zeros and weighs nothing)
        typename std::decay<decltype(wfn)>::type::Raw raw[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) raw[it] = wfn.load(base + it * 256);
        f32x4 t4[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = base + it * 256;
            const f32x4 x = wfn.w4(raw[it], e);
            t4[it] = e < a.V ? x : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        double s = 0.0;
#pragma unroll
        for (int h = 0; h < kIters / 2; ++h) {
            const f32x4 x = t4[2 * h], y = t4[2 * h + 1];
            s += (double)(((x[0] + x[1]) + (x[2] + x[3])) + ((y[0] + y[1]) + (y[2] + y[3])));
        }
        return wave_sum(s);
    };
    double s;
    if constexpr (CUT) {
        // outside the segment holding a cut's index, its test is one comparison
        ThrCut tp, tq;
        if (w.cp.seg_uniform(seg * kSeg, kSeg, tp) && w.cq.seg_uniform(seg * kSeg, kSeg, tq))
            s = segment_sum(with_cuts(w, tp, tq));
        else
            s = segment_sum(w);
    } else {
        s = segment_sum(w);
    }
    if (lane == 0) a.resid_s[(size_t)b * a.nseg + seg] = s;
}

// Correction draw of one rejecting sequence per workgroup (one wave): the
// segment where the running residual mass first exceeds u times the total,
// then the element inside it, by the residual weights recomputed with the
// arithmetic that produced the segment sums.  Falls back to p_j when the
// residual has no mass.
constexpr int kResidRegs = 4;  // residual sums per lane held in registers
template <bool CUT>
__global__ void __launch_bounds__(64) verify_draw_kernel(TailArgs a) {
    typedef CutOf<CUT> CutT;
    const int b = blockIdx.x, lane = threadIdx.x;
    // every load that does not depend on the record is issued with it
    const SeqDraw sd = a.seq[b];
    const double* rs = a.resid_s + (size_t)b * a.nseg;
    double rv[kResidRegs];
#pragma unroll
    for (int c = 0; c < kResidRegs; ++c) {
        const int q = c * 64 + lane;
        rv[c] = rs[q < a.nseg ? q : a.nseg - 1];
        if (q >= a.nseg) rv[c] = 0.0;
    }
    const uint64_t seed = a.seeds[b];
    if (sd.j < 0) return;
    const int j = sd.j;
    const size_t rj = (size_t)b * a.G + j;
    const CutT tc = cut_of<CUT>(a.tcut, rj, a.row_S);
    const CutT dc = cut_of<CUT>(a.dcut, rj, a.row_S);
    double tot = 0.0;
#pragma unroll
    for (int c = 0; c < kResidRegs; ++c) tot += rv[c];
    for (int q = 64 * kResidRegs + lane; q < a.nseg; q += 64) tot += rs[q];
    tot = wave_sum(tot);
    const double u = philox_uniform(seed, a.step, (uint64_t)b, (uint64_t)j, kFinalDraw);
    const size_t rowj = (size_t)b * a.G + j;
    const float* zpr = a.zp + rowj * a.V;
    int tok;
    if (tot > 0.0) {
        ResidualW<CutT> w;
        w.zp = row_rsrc(zpr, a.V);
        w.zq = row_rsrc(a.zq ? a.zq + rowj * a.V : zpr, a.zq ? a.V : 0);
        w.has_q = a.zq != nullptr;
        w.dq = sd.dq;
        w.Rp = sd.Rp;
        w.Rq = sd.Rq;
        w.Fp = sd.Fp;
        w.Fq = sd.Fq;
        w.c2 = a.c2;
        w.cp = tc;
        w.cq = dc;
        double before = 0.0;
        auto segw = [&](int q) -> double {
            const int c = q >> 6;
            double v = 0.0;
#pragma unroll
            for (int cc = 0; cc < kResidRegs; ++cc) v = c == cc ? rv[cc] : v;
            return c < kResidRegs ? v : rs[q];
        };
        const double target = u * tot;
        const int sj = find_segment(a.nseg, target, segw, lane, before);
        if (sj < 0) {
            tok = 0;
        } else {
            bool uniform = false;
            ThrCut tp, tq;
            if constexpr (CUT)
                uniform = w.cp.seg_uniform(sj * kSeg, kSeg, tp) && w.cq.seg_uniform(sj * kSeg, kSeg, tq);
            tok = uniform ? draw_in_segment(sj, a.V, target - before, with_cuts(w, tp, tq), lane)
                          : draw_in_segment(sj, a.V, target - before, w, lane);
        }
    } else {
        tok = draw_softmax_row(zpr, a.V, a.seg_m + rowj * a.nseg, a.seg_s + rowj * a.nseg, a.nseg, a.c2, sd.Mj,
                               sd.Sj, u, lane, tc);
    }
    if (lane == 0) a.out_tokens[rowj] = tok;
}

// ------------------------------------------------------------- planning
struct VerifyLayout {
    int nseg;
    size_t seg_m, seg_s, row_M, row_S, row_arg, resid, seq, bytes;
};

VerifyLayout verify_layout(int batch, int gamma, int vocab) {
    VerifyLayout L{};
    const size_t rows = (size_t)batch * gamma;
    L.nseg = (vocab + kSeg - 1) / kSeg;
    Carve c;
    L.seg_m = c.take<float>(2 * rows * L.nseg);
    L.seg_s = c.take<double>(2 * rows * L.nseg);
    L.row_M = c.take<float>(2 * rows);
    L.row_S = c.take<double>(2 * rows);
    L.row_arg = c.take<int>(rows);
    L.resid = c.take<double>((size_t)batch * L.nseg);
    L.seq = c.take<SeqDraw>((size_t)batch);
    L.bytes = c.total();
    return L;
}

bool ws_ok(const void* ws, size_t have, size_t need) {
    return ws && !(reinterpret_cast<uintptr_t>(ws) & 255) && have >= need;
}

// Shape part of spec_verify's checks: DFLASH_ERR_SHAPE, DFLASH_ERR_UNSUPPORTED
// or OK.  The row cap keeps batch * gamma (and twice it) inside the 32-bit
// counts of the launches.
int verify_shape(int batch, int gamma, int vocab) {
    if (batch < 0 || gamma < 1 || vocab < 1) return DFLASH_ERR_SHAPE;
    if (gamma > 32 || vocab % 4 != 0 || vocab > kMaxVocab ||
        capped_product(kMaxRowsPerCall, {batch, gamma}) < 0)
        return DFLASH_ERR_UNSUPPORTED;
    return DFLASH_OK;
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" size_t dflash_topk_workspace_size(int batch, int gamma, int vocab, int k) {
    (void)batch;
    (void)gamma;
    (void)vocab;
    (void)k;
    return 0;  // everything lives in the row workgroup's LDS
}

extern "C" int dflash_topk(const float* logits, const dflash_nucleus_cut* cut, int batch, int gamma,
                           int vocab, int k,
                           float temperature, const uint64_t* seeds, uint64_t step,
                           int32_t* topk_idx, float* topk_val, double* lse, int32_t* draft,
                           void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    if (batch < 0 || gamma < 1 || vocab < 1 || k < 1 || k > vocab) return DFLASH_ERR_SHAPE;
    if (!(temperature >= 0.f) || !std::isfinite(temperature)) return DFLASH_ERR_SHAPE;
    if (batch == 0) return DFLASH_OK;
    if (!logits || !topk_idx || !topk_val) return DFLASH_ERR_NULL;
    if (temperature > 0.f && draft && !seeds) return DFLASH_ERR_NULL;
    if (k > 64 || gamma > 32 || vocab % 4 != 0 || vocab > kMaxTopkVocab ||
        capped_product(kMaxRowsPerCall, {batch, gamma}) < 0)
        return DFLASH_ERR_UNSUPPORTED;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    TopKArgs f{};
    f.z = logits;
    f.cut = cut;
    f.B = batch;
    f.G = gamma;
    f.V = vocab;
    f.nseg = (vocab + kSeg - 1) / kSeg;
    f.k = k;
    f.T = temperature;
    f.c2 = temperature > 0.f ? (float)(1.4426950408889634 / (double)temperature) : 0.f;
    f.seeds = seeds;
    f.step = step;
    f.topk_idx = topk_idx;
    f.topk_val = topk_val;
    f.lse = lse;
    f.draft = draft;
    const dim3 grid((unsigned)(batch * gamma)), block(kRowThreads);
    if (temperature > 0.f) {
        if (cut) hipLaunchKernelGGL((topk_row_kernel<kSumExp, true>), grid, block, 0, st, f);
        else hipLaunchKernelGGL((topk_row_kernel<kSumExp, false>), grid, block, 0, st, f);
    } else {
        if (cut) hipLaunchKernelGGL((topk_row_kernel<kSegMax, true>), grid, block, 0, st, f);
        else hipLaunchKernelGGL((topk_row_kernel<kSegMax, false>), grid, block, 0, st, f);
    }
    return launch_status();
}

extern "C" size_t spec_verify_workspace_size(int batch, int gamma, int vocab) {
    if (verify_shape(batch, gamma, vocab) != DFLASH_OK) return 0;
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
    return verify_shape(batch, gamma, vocab);
}

size_t verify_scratch_bytes(int batch, int gamma, int vocab) {
    return verify_layout(batch, gamma, vocab).bytes;
}

int verify_enqueue(const float* target_logits, const float* draft_logits,
                   const int32_t* draft_tokens, const double* draft_lse,
                   const dflash_nucleus_cut* target_cut, const dflash_nucleus_cut* draft_cut,
                   float temperature, const uint64_t* seeds, uint64_t step, int32_t* accept_len,
                   int32_t* out_tokens, uint8_t* accepted, int batch, int gamma, int vocab,
                   void* scratch_ws, hipStream_t st) {
    // the argmax is always in the nucleus: cuts only matter when sampling
    if (temperature == 0.f) target_cut = draft_cut = nullptr;
    const VerifyLayout L = verify_layout(batch, gamma, vocab);
    char* ws = static_cast<char*>(scratch_ws);
    const float c2 = temperature > 0.f ? (float)(1.4426950408889634 / (double)temperature) : 0.f;
    const int rows = batch * gamma;
    RowArgs ra{};
    ra.zp = target_logits;
    ra.zq = draft_logits;
    ra.tcut = target_cut;
    ra.dcut = draft_cut;
    ra.rows = rows;
    ra.V = vocab;
    ra.nseg = L.nseg;
    ra.B = batch;
    ra.c2 = c2;
    ra.seg_m = reinterpret_cast<float*>(ws + L.seg_m);
    ra.seg_s = reinterpret_cast<double*>(ws + L.seg_s);
    ra.row_M = reinterpret_cast<float*>(ws + L.row_M);
    ra.row_S = reinterpret_cast<double*>(ws + L.row_S);
    ra.row_arg = reinterpret_cast<int*>(ws + L.row_arg);
    if (temperature == 0.f) {
        hipLaunchKernelGGL((verify_row_kernel<kArgmax, false>), dim3((unsigned)rows), dim3(kRowThreads), 0, st,
                           ra);
    } else {
        // the drafter rows' log-normalisers come from the same launch when
        // they are not given
        const bool both = !draft_lse && draft_logits;
        const int launch_rows = both ? 2 * rows : rows;
        if (target_cut || (both && draft_cut))
            hipLaunchKernelGGL((verify_row_kernel<kSumExp, true>), dim3((unsigned)launch_rows), dim3(kRowThreads),
                               0, st, ra);
        else
            hipLaunchKernelGGL((verify_row_kernel<kSumExp, false>), dim3((unsigned)launch_rows),
                               dim3(kRowThreads), 0, st, ra);
    }
    int rc = launch_status();
    if (rc) return rc;
    TailArgs t{};
    t.zp = target_logits;
    t.zq = draft_logits;
    t.drafts = draft_tokens;
    t.draft_lse = draft_lse;
    t.tcut = target_cut;
    t.dcut = draft_logits ? draft_cut : nullptr;
    t.B = batch;
    t.G = gamma;
    t.V = vocab;
    t.nseg = L.nseg;
    t.nr = temperature > 0.f ? (L.nseg + kTailWaves - 1) / kTailWaves : 1;
    t.T = temperature;
    t.c2 = c2;
    t.seeds = seeds;
    t.step = step;
    t.seg_m = ra.seg_m;
    t.seg_s = ra.seg_s;
    t.row_M = ra.row_M;
    t.row_S = ra.row_S;
    t.row_arg = ra.row_arg;
    t.resid_s = reinterpret_cast<double*>(ws + L.resid);
    t.seq = reinterpret_cast<SeqDraw*>(ws + L.seq);
    t.accept_len = accept_len;
    t.out_tokens = out_tokens;
    t.accepted = accepted;
    const bool cut = t.tcut || t.dcut;
    if (cut)
        hipLaunchKernelGGL(verify_tail_kernel<true>, dim3((unsigned)(batch * t.nr)), dim3(64 * kTailWaves), 0, st, t);
    else
        hipLaunchKernelGGL(verify_tail_kernel<false>, dim3((unsigned)(batch * t.nr)), dim3(64 * kTailWaves), 0, st, t);
    rc = launch_status();
    if (rc || temperature == 0.f) return rc;
    if (cut)
        hipLaunchKernelGGL(verify_draw_kernel<true>, dim3((unsigned)batch), dim3(64), 0, st, t);
    else
        hipLaunchKernelGGL(verify_draw_kernel<false>, dim3((unsigned)batch), dim3(64), 0, st, t);
    return launch_status();
}

}  // namespace dfl

extern "C" int spec_verify(const float* target_logits, const float* draft_logits,
                           const int32_t* draft_tokens, const double* draft_lse,
                           const dflash_nucleus_cut* target_cut, const dflash_nucleus_cut* draft_cut,
                           float temperature, const uint64_t* seeds, uint64_t step,
                           int32_t* accept_len, int32_t* out_tokens, uint8_t* accepted,
                           int batch, int gamma, int vocab, void* workspace,
                           size_t workspace_bytes, void* stream) {
    const int rc = verify_check(target_logits, draft_tokens, temperature, seeds, accept_len,
                                out_tokens, batch, gamma, vocab);
    if (rc || batch == 0) return rc;
    if (!ws_ok(workspace, workspace_bytes, verify_scratch_bytes(batch, gamma, vocab)))
        return DFLASH_ERR_WORKSPACE;
    return verify_enqueue(target_logits, draft_logits, draft_tokens, draft_lse, target_cut, draft_cut,
                          temperature, seeds, step, accept_len, out_tokens, accepted, batch, gamma,
                          vocab, workspace, reinterpret_cast<hipStream_t>(stream));
}
