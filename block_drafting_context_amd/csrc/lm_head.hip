// lm_head.hip -- the drafter's LM head with top-k, the row log-normaliser and
// the draft draw fused into the GEMM epilogue, for gfx950.
//
// "Beam 1.0 DFlash2" model card, "Model": the drafter reuses the target's LM
// head (151,936-entry vocabulary, hidden size 5,120).  "DFlash vs DFlash 2",
// "The candidate selector": top-k candidates of every block position, and the
// full-vocabulary LM-head pass is the costly part; "The problem: one
// expensive token at a time": the drafter proposes y ~ q = softmax(z / T).
//
// The logits z = h W^T never reach HBM.  One persistent workgroup per CU owns
// a run of consecutive 128-entry vocabulary segments and streams them as
// tiles of 256 entries x (up to) 256 hidden rows, so every weight byte is read
// once per pass.  K advances in stages of 64 through LDS (weights in a 3-slot
// ring, two stages ahead; hidden rows in a 2-slot ring, one ahead; both
// by buffer_load_dwordx4 ... lds with the 16-byte chunks of each row
// XOR-swizzled).  Eight waves each accumulate one segment (128 entries)
// x 64 rows with v_mfma_f32_16x16x32_bf16, the vocabulary as the MFMA row
// operand: lane (g, i) of a 16 x 16 tile then holds entries 4g..4g+3 of
// hidden row i, i.e. every lane ends with 32 logits of one row and the four
// lanes i, i+16, i+32, i+48 share that row's segment.  The epilogue reduces
// each (row, segment) in registers across those four lanes:
//   * m = max z and s = sum 2^((z - m) log2(e)/T), with the sums of its eight
//     16-entry groups (kept for the draw);
//   * top-k candidates: theta = a lower bound of the k-th largest of the
//     segment's 32 quad maxima (quad: 4 consecutive entries in one lane's
//     registers), taken from the four lanes' TT largest quad maxima (TT =
//     min(4, ceil(k/2)), 4 TT >= k), hence of the segment's k-th largest
//     entry; every quad whose maximum is >= theta is written whole to the
//     segment's record slots, in order, with a 32-bit mask of which quads they
//     are (ties need no special case: all of them are written).
// A finalize kernel per row takes tau = the k-th largest segment maximum
// (every top-k entry is >= tau, so only segments with m >= tau are read),
// merges their records and adds the segment masses in fp64 for the
// log-normaliser.  The draft is one inverse-CDF draw over the whole row in
// increasing vocabulary order at the row's purpose-0 uniform u: the running
// mass first exceeds u S inside the segment J found from the segment masses,
// inside the 16-entry group of J found from its group sums, and at the entry
// of that group found from its 16 logits, which the finalize recomputes from
// the hidden row and 16 weight rows (32 KB per row at d = 5,120, instead of
// keeping any logit in memory).
#include <climits>
#include <cmath>

#include "common.hpp"

namespace dfl {
namespace {

constexpr int kSegW = 128;            // vocabulary segment: candidate slot and statistics record
constexpr int kGrpW = 16;             // entries per group of a segment (eight group sums)
constexpr int kHeadRows = 256;        // hidden rows per pass over the weights
constexpr int kTileV = 2 * kSegW;     // vocabulary entries per workgroup tile
#ifndef DFL_HEAD_BK
#define DFL_HEAD_BK 64
#endif
#ifndef DFL_HEAD_WSLOTS
#define DFL_HEAD_WSLOTS 3
#endif
#ifndef DFL_HEAD_HSLOTS
#define DFL_HEAD_HSLOTS 2
#endif
constexpr int kHBK = DFL_HEAD_BK;     // K stage
constexpr int kHRowB = kHBK * 2;      // bytes per staged row
constexpr int kChunks = kHRowB / 16;  // 16-byte chunks per staged row
constexpr int kRowsPerIns = 1024 / kHRowB;  // rows per 1 KB DMA instruction
constexpr int kWSlots = DFL_HEAD_WSLOTS;    // weight ring: kWSlots - 1 stages in flight
constexpr int kHSlots = DFL_HEAD_HSLOTS;    // hidden-row ring: kHSlots - 1 stages in flight
constexpr int kLeadW = kWSlots - 1, kLeadH = kHSlots - 1;
static_assert(kLeadW >= kLeadH && kLeadH >= 1, "the weights are issued at least as far ahead");
static_assert(kWSlots * kTileV * kHRowB + kHSlots * 256 * kHRowB <= 160 * 1024, "LDS");
constexpr int kHWaves = 8;            // 2 segments x 4 row quarters
constexpr int kLoadsPerWave = kTileV * kHRowB / 1024 / kHWaves;  // 1 KB DMA instructions per ring
// loads a wave may still have in flight when it needs stage j: those issued
// after h(j), i.e. W(j - kLeadH + kLeadW) and the kLeadH - 1 later batches
constexpr int kWaitLoads = kLoadsPerWave + (kLeadH - 1) * 2 * kLoadsPerWave;
constexpr int kQuads = kSegW / 4;     // quads of 4 entries per segment: candidate record slots
constexpr int kHeadMaxK = 16;
constexpr int kHeadMaxD = 65536;     // keeps a tile's byte offsets (256 rows x d x 2 B) in 32 bits
constexpr int kHeadCUs = 256;
constexpr int kFinThreads = 256;
constexpr int kNone = INT_MAX;
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource word 3 for raw byte buffers on gfx9 parts

static_assert(kLoadsPerWave == kHeadRows * kHRowB / 1024 / kHWaves, "both rings load alike");

// 16-byte chunk c of staged row r is stored at chunk c ^ swz(r): with the
// row's 128 (or 64) bytes, eight consecutive rows read at one logical chunk
// hit eight distinct 16-byte bank groups
__device__ __forceinline__ int chunk_swz(int r) { return kChunks == 8 ? (r & 7) : ((r >> 1) & 3); }

template <int N>
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void bare_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct SegStat {
    float m;     // segment maximum
    float s;     // sum 2^((z - m) log2(e)/T) (0 when greedy)
    int mask;    // bit vb*4 + g: candidate quad (vb, g) was written (in bit order)
    int pad;
};

struct HeadArgs {
    const uint16_t* h;     // [rows, d] bf16
    const uint16_t* hs;    // the same rows in K slabs: [pass][d / kHBK][256][kHBK], zero past rows
    const uint16_t* w;     // [V, d] bf16
    SegStat* stats;        // [rows][nseg]
    u32x4* cand;           // [rows][nseg][kQuads]: candidate quads (4 logits each), in mask order
    u32x2* gsum;           // [rows][nseg][4]: the segment's eight 16-entry group sums (fp32 pairs)
    int M, row0, d, V, nseg, groups, k;
    float c2;              // log2(e) / T (0 when greedy)
    int want_exp, want_draw;
};

// {value of the lane with bit W of its index clear, value of the lane with it
// set}, for the pair (lane, lane ^ W), W = 16 or 32 (v_permlane16/32_swap; the
// layout was measured on gfx950).  Used where the order within a pair matters.
template <int W>
__device__ __forceinline__ void lo_hi(float v, float& lo, float& hi) {
    unsigned r0, r1;
    swap_pair<W>(__float_as_uint(v), r0, r1);
    lo = __uint_as_float(r0);
    hi = __uint_as_float(r1);
}
template <int W>
__device__ __forceinline__ void lo_hi(int v, int& lo, int& hi) {
    unsigned r0, r1;
    swap_pair<W>((unsigned)v, r0, r1);
    lo = (int)r0;
    hi = (int)r1;
}

// Over the four lanes (grp = 0..3) sharing a row: the exclusive prefix of v in
// grp order, and the total.  Every lane adds the same operands in the same
// order, so the total is bit-identical across the four lanes.
__device__ __forceinline__ float quad_scan(float v, int grp, float& total) {
    float lo, hi;
    lo_hi<16>(v, lo, hi);
    const float pair = lo + hi;
    const float in_pair = (grp & 1) ? lo : 0.f;
    float plo, phi;
    lo_hi<32>(pair, plo, phi);
    total = plo + phi;
    return in_pair + ((grp & 2) ? plo : 0.f);
}
__device__ __forceinline__ int quad_scan(int v, int grp, int& total) {
    int lo, hi;
    lo_hi<16>(v, lo, hi);
    const int pair = lo + hi;
    int plo, phi;
    lo_hi<32>(pair, plo, phi);
    total = plo + phi;
    return ((grp & 1) ? lo : 0) + ((grp & 2) ? plo : 0);
}
__device__ __forceinline__ float quad_min(float v) {
    float lo, hi;
    lo_hi<16>(v, lo, hi);
    v = fminf(lo, hi);
    lo_hi<32>(v, lo, hi);
    return fminf(lo, hi);
}
__device__ __forceinline__ float quad_max(float v) {
    float lo, hi;
    lo_hi<16>(v, lo, hi);
    v = fmaxf(lo, hi);
    lo_hi<32>(v, lo, hi);
    return fmaxf(lo, hi);
}
__device__ __forceinline__ int quad_min(int v) {
    int lo, hi;
    lo_hi<16>(v, lo, hi);
    v = min(lo, hi);
    lo_hi<32>(v, lo, hi);
    return min(lo, hi);
}
__device__ __forceinline__ int quad_max(int v) {
    int lo, hi;
    lo_hi<16>(v, lo, hi);
    v = max(lo, hi);
    lo_hi<32>(v, lo, hi);
    return max(lo, hi);
}

// 16 bytes per lane from a raw buffer straight into LDS at m0 + 16 * lane
// (buffer_load_dwordx4 ... lds).  Written as inline assembly so that the
// compiler, which cannot see which ring slot a DMA targets, does not guard the
// operand fetches from the other slots with waits for every load in flight;
// the kernel waits for its own loads explicitly.  NT: non-temporal.  m0 (the
// LDS destination) is declared clobbered, so the compiler keeps nothing there,
// and the s_nop is the one wait state an LDS DMA needs after a scalar write of
// m0 (the compiler puts the same s_nop between the two when it emits the DMA).
// The backend warns that m0 is a reserved register whose value it will not
// preserve around the statement; nothing needs it preserved (no other code
// of this file reads or writes m0, which the codegen tests check), the
// clobber only tells the compiler that the statement overwrites it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, i32x4 rsrc, uint32_t soff) {
    if (NT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// raw byte buffer over [base, base + bytes)
__device__ __forceinline__ i32x4 byte_buffer(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = (int)(uint32_t)p;
    r[1] = (int)((uint32_t)(p >> 32) & 0xFFFFu);  // stride 0
    r[2] = (int)bytes;
    r[3] = kRsrcWord3;
    return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);  // low half of the flat address = LDS offset
}

// TT = min(4, ceil(k / 2)): per-lane depth of the top-k threshold (4 TT >= k).
template <int TT>
__global__ void __launch_bounds__(64 * kHWaves) lm_head_kernel(HeadArgs a) {
    __shared__ __attribute__((aligned(1024))) unsigned char sw[kWSlots][kTileV * kHRowB];
    __shared__ __attribute__((aligned(1024))) unsigned char sh[kHSlots][kHeadRows * kHRowB];

    const int gidx = blockIdx.x;
    const int s0 = (int)((long)gidx * a.nseg / a.groups);
    const int s1 = (int)((long)(gidx + 1) * a.nseg / a.groups);
    const int ntile = (s1 - s0 + 1) / 2;
    const int nk = a.d / kHBK;
    const int total = ntile * nk;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wv = wave >> 2, wr = wave & 3;   // segment of the tile, row quarter
    const int i16 = lane & 15, grp = lane >> 4;
    const int rl = lane / kChunks, pc = lane % kChunks;  // DMA: row within an instruction, physical chunk

    // DMA: a buffer resource over exactly the tile's weight rows or the pass's
    // hidden rows, a per-lane byte offset (row, swizzled chunk) and the stage's
    // K offset as the scalar offset.  Rows beyond the tile or the pass fall
    // outside the resource, so the hardware skips their reads (they still
    // count as issued loads, which keeps every wave's wait counts the same);
    // what their LDS rows hold only reaches outputs that are never stored
    // (rows >= M) or entries the epilogue replaces by -inf (>= V).
    // hidden rows from their K slabs: a stage's 256 rows are one contiguous
    // 32 KB block (read in row pieces 2 d bytes apart, the rows' chunks at one
    // K step all fall on the same few memory channels)
    uint32_t h_off[kLoadsPerWave];
#pragma unroll
    for (int ins = 0; ins < kLoadsPerWave; ++ins) {
        const int r = (wave * kLoadsPerWave + ins) * kRowsPerIns + rl;
        h_off[ins] = (uint32_t)r * (uint32_t)kHRowB + (uint32_t)((pc ^ chunk_swz(r)) * 16);
    }
    const i32x4 h_rsrc = byte_buffer(a.hs + (size_t)a.row0 * a.d, (uint32_t)(kHeadRows * a.d * 2));
    // K step kk of a tile is read at byte offset kbyte(kk): each workgroup
    // starts its K sweep at its own step, so the CUs' concurrent loads are
    // spread over the memory channels instead of all touching one K column of
    // the hidden rows and of their weight rows (measured: 470 -> 446 us at
    // 256 x 5120 x 151,936)
    const int krot = gidx % nk;
    auto kstep = [&](int kk) { int x = kk + krot; x -= x >= nk ? nk : 0; return (uint32_t)x; };
    auto kbyte = [&](int kk) { return kstep(kk) * (uint32_t)kHRowB; };                 // weight rows
    auto kslab = [&](int kk) { return kstep(kk) * (uint32_t)(kHeadRows * kHRowB); };  // hidden slabs
    auto issue_w = [&](int j) {
        const int t = j / nk, kk = j - t * nk;
        const int v0 = (s0 + 2 * t) * kSegW;
        const int nv = min(min(s1 * kSegW, a.V), v0 + kTileV) - v0;  // valid rows of the tile
        const i32x4 rsrc = byte_buffer(a.w + (size_t)v0 * a.d, (uint32_t)(nv * a.d * 2));
        const uint32_t lds = lds_addr(sw[j % kWSlots]) + (uint32_t)(wave * kLoadsPerWave * 1024);
#pragma unroll
        for (int ins = 0; ins < kLoadsPerWave; ++ins) {
            const int r = (wave * kLoadsPerWave + ins) * kRowsPerIns + rl;
            const uint32_t voff = (uint32_t)r * (uint32_t)(a.d * 2) + (uint32_t)((pc ^ chunk_swz(r)) * 16);
            dma16<true>(lds + ins * 1024, voff, rsrc, kbyte(kk));
        }
    };
    auto issue_h = [&](int j) {
        const int kk = j % nk;
        const uint32_t lds = lds_addr(sh[j % kHSlots]) + (uint32_t)(wave * kLoadsPerWave * 1024);
#pragma unroll
        for (int ins = 0; ins < kLoadsPerWave; ++ins)
            dma16<false>(lds + ins * 1024, h_off[ins], h_rsrc, kslab(kk));
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bool rows_live = wr * 64 < a.M;

    auto compute = [&](int j) {
        const unsigned char* Ws = sw[j % kWSlots];
        const unsigned char* Hs = sh[j % kHSlots];
#pragma unroll
        for (int s = 0; s < kHBK / 32; ++s) {
            const int c = s * 4 + grp;
            bf16x8 fa[8], fb[4];
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
                const int r = wv * kSegW + vb * 16 + i16;
                fa[vb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                        Ws + r * kHRowB + ((c ^ chunk_swz(r)) * 16)));
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int r = wr * 64 + rb * 16 + i16;
                fb[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                        Hs + r * kHRowB + ((c ^ chunk_swz(r)) * 16)));
            }
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int vb = 0; vb < 8; ++vb)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    acc[vb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[vb], fb[rb],
                                                                          acc[vb][rb], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        }
    };

    // Pass-relative offsets of the lane's rows in the outputs, fixed before
    // the loop so that no 64-bit address is carried through it.
    SegStat* const stats_p = a.stats + (size_t)a.row0 * a.nseg;
    u32x2* const gsum_p = a.gsum + (size_t)a.row0 * a.nseg * 4;
    u32x4* const cand_p = a.cand + (size_t)a.row0 * a.nseg * kQuads;
    const uint32_t lane_row_off = (uint32_t)(wr * 64 + i16) * (uint32_t)a.nseg;

    // candidate records through a raw buffer over this pass's record slots:
    // a record that is not a candidate is stored at an offset past the end,
    // which the hardware drops (no branch per quad)
    const __amdgpu_buffer_rsrc_t rec_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        cand_p, (short)0, (int)((size_t)a.M * a.nseg * kQuads * 16), kRsrcWord3);

    // acc[vb][rb][e]: entry seg*128 + vb*16 + 4*grp + e, row wr*64 + rb*16 + i16
    auto epilogue = [&](int t) {
        const int seg = s0 + 2 * t + wv;
        const int vseg = seg * kSegW;
        const int nvalid = min(kSegW, a.V - vseg);
        // Opaque copies: everything derived from them is computed here, per
        // tile, instead of being hoisted out of the tile loop into registers
        // that would then live through the whole K loop.
        int g4 = grp << 2, li16 = i16, gq = grp;
        uint32_t lro = lane_row_off;
        asm volatile("" : "+v"(g4), "+v"(li16), "+v"(gq), "+v"(lro));
        const float c2 = a.c2;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
#define Z(i) acc[(i) >> 2][rb][(i) & 3]
            const bool live = wr * 64 + rb * 16 + li16 < a.M;
            const uint32_t so = lro + (uint32_t)(rb * 16) * (uint32_t)a.nseg + (uint32_t)seg;
            if (nvalid < kSegW) {
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    if ((i >> 2) * 16 + g4 + (i & 3) >= nvalid) Z(i) = -INFINITY;
            }
            // quad maxima: the largest of the 4 consecutive entries a lane holds
            float qm[8];
#pragma unroll
            for (int vb = 0; vb < 8; ++vb)
                qm[vb] = fmaxf(fmaxf(Z(vb * 4), Z(vb * 4 + 1)), fmaxf(Z(vb * 4 + 2), Z(vb * 4 + 3)));
            float mx = fmaxf(fmaxf(fmaxf(qm[0], qm[1]), fmaxf(qm[2], qm[3])),
                             fmaxf(fmaxf(qm[4], qm[5]), fmaxf(qm[6], qm[7])));
            mx = quad_max(mx);

            // theta: a lower bound of the k-th largest of the segment's 32 quad
            // maxima, hence of its k-th largest entry.  Each lane keeps its TT
            // largest quad maxima (sorted); a value x of that list has at least
            // (its rank + 1) entries >= x in its own list, and the three other
            // lanes' lists are counted exactly; theta is the largest list value
            // with at least k counted (4 TT >= k, so the smallest qualifies).
            float top[TT];
#pragma unroll
            for (int q = 0; q < TT; ++q) top[q] = -INFINITY;
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
#pragma unroll
                for (int q = TT - 1; q > 0; --q) top[q] = __builtin_amdgcn_fmed3f(top[q - 1], top[q], qm[vb]);
                top[0] = fmaxf(top[0], qm[vb]);
            }
            float th = -INFINITY;
            {
                float o16[TT], o32[TT], o48[TT];  // the lists of lanes grp^1, grp^2, grp^3
#pragma unroll
                for (int q = 0; q < TT; ++q) {
                    float lo, hi;
                    lo_hi<32>(top[q], lo, hi);
                    o32[q] = (gq & 2) ? lo : hi;
                    lo_hi<16>(top[q], lo, hi);
                    o16[q] = (gq & 1) ? lo : hi;
                    lo_hi<16>(o32[q], lo, hi);
                    o48[q] = (gq & 1) ? lo : hi;
                }
#pragma unroll
                for (int q = 0; q < TT; ++q) {
                    int c = q + 1;
#pragma unroll
                    for (int r = 0; r < TT; ++r)
                        c += (o16[r] >= top[q]) + (o32[r] >= top[q]) + (o48[r] >= top[q]);
                    th = c >= a.k ? fmaxf(th, top[q]) : th;
                }
                th = quad_max(th);  // the lanes' bounds may differ: all take the largest
            }

            // candidate quads (4 consecutive entries held by one lane): those
            // whose maximum is >= theta, stored in (vb, grp) order
            int qb = 0;
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) qb |= (qm[vb] >= th && qm[vb] > -INFINITY) ? (1 << vb) : 0;
            uint32_t mask = 0;
            {
                int lo, hi;
                lo_hi<16>(qb, lo, hi);
                const int b16 = (gq & 1) ? lo : hi;
                lo_hi<32>(qb, lo, hi);
                const int b32 = (gq & 2) ? lo : hi;
                lo_hi<16>(b32, lo, hi);
                const int b48 = (gq & 1) ? lo : hi;
                // spread each lane's 8 bits to bit vb*4 + its grp
                auto spread = [](uint32_t x) {
                    x = (x | (x << 12)) & 0x000F000Fu;
                    x = (x | (x << 6)) & 0x03030303u;
                    x = (x | (x << 3)) & 0x11111111u;
                    return x;
                };
                mask = (spread((uint32_t)qb) << gq) | (spread((uint32_t)b16) << (gq ^ 1)) |
                       (spread((uint32_t)b32) << (gq ^ 2)) | (spread((uint32_t)b48) << (gq ^ 3));
            }
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
                const int bit = vb * 4 + gq;
                const uint32_t at = so * kQuads + (uint32_t)__builtin_popcount(mask & ((1u << bit) - 1u));
                const bool st_ok = live && ((qb >> vb) & 1);
                u32x4 v;
                v[0] = __float_as_uint(Z(vb * 4));
                v[1] = __float_as_uint(Z(vb * 4 + 1));
                v[2] = __float_as_uint(Z(vb * 4 + 2));
                v[3] = __float_as_uint(Z(vb * 4 + 3));
                __builtin_amdgcn_raw_buffer_store_b128(v, rec_rsrc, st_ok ? (int)(at * 16u) : (int)0x7FFFFFF0, 0, 0);
            }

            // segment mass and its 16-entry group sums (Z becomes the weights):
            // group vb holds quad vb of each of the four lanes; every lane adds
            // the same operands in the same order, so all four hold
            // bit-identical sums, and the segment mass is their sum in group order
            float ssum = 0.f;
            if (a.want_exp) {
                const float mc = mx * c2;
#pragma unroll
                for (int i = 0; i < 32; ++i) Z(i) = fast_exp2(__builtin_fmaf(Z(i), c2, -mc));
                float gs[8];
#pragma unroll
                for (int vb = 0; vb < 8; ++vb) {
                    const float qs = ((Z(vb * 4) + Z(vb * 4 + 1)) + Z(vb * 4 + 2)) + Z(vb * 4 + 3);
                    float lo, hi;
                    lo_hi<16>(qs, lo, hi);
                    const float pair = lo + hi;
                    lo_hi<32>(pair, lo, hi);
                    gs[vb] = lo + hi;
                    ssum += gs[vb];
                }
                if (a.want_draw && live) {
                    // lane gq stores groups 2 gq and 2 gq + 1
                    float e0 = gs[0], e1 = gs[1];
#pragma unroll
                    for (int q = 1; q < 4; ++q) {
                        e0 = gq == q ? gs[2 * q] : e0;
                        e1 = gq == q ? gs[2 * q + 1] : e1;
                    }
                    gsum_p[(size_t)so * 4 + gq] = u32x2{__float_as_uint(e0), __float_as_uint(e1)};
                }
            }
            if (live && gq == 0) stats_p[so] = SegStat{mx, ssum, (int)mask, 0};
#undef Z
        }
    };

    // One continuous stream of stages over all tiles (stage j: tile j / nk,
    // K step j % nk), so the next tile's first stages load during an epilogue.
    // Issue order: W(0 .. kLeadW - kLeadH - 1), then batches [h(i), W(i + kLeadW
    // - kLeadH)]; stage j issues the batch [h(j + kLeadH), W(j + kLeadW)] into
    // the slots that stage j - 1 used.
    for (int i = 0; i < kLeadW - kLeadH && i < total; ++i) issue_w(i);
    for (int i = 0; i < kLeadH; ++i) {
        if (i < total) issue_h(i);
        if (i + kLeadW - kLeadH < total) issue_w(i + kLeadW - kLeadH);
    }
    for (int j = 0; j < total; ++j) {
        const int t = j / nk, kk = j - t * nk;
        // the first stage of a tile also waits for the previous epilogue's stores
        if ((kk == 0 && j > 0) || j + kLeadW - 1 >= total) wait_vmem<0>();
        else wait_vmem<kWaitLoads>();
        bare_barrier();  // stage j landed for every wave; stage j - 1's slots are free
        if (j + kLeadH < total) issue_h(j + kLeadH);
        if (j + kLeadW < total) issue_w(j + kLeadW);
        const bool live = rows_live && (s0 + 2 * t + wv < s1);
        if (live) compute(j);
        if (kk == nk - 1) {
            if (live) epilogue(t);
#pragma unroll
            for (int x = 0; x < 8; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
}

// Hidden rows -> K slabs [pass][d / kHBK][256][kHBK] (rows past the last one
// zero): 16 bytes per thread.
__global__ void __launch_bounds__(256) head_slabs_kernel(const uint16_t* h, int rows, int d, uint16_t* hs) {
    const int chunks = d / 8;  // 16-byte pieces of a row
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t npass_rows = (int64_t)((rows + kHeadRows - 1) / kHeadRows) * kHeadRows;
    if (e >= npass_rows * chunks) return;
    const int r = (int)(e / chunks), c8 = (int)(e % chunks);
    const u32x4 v = r < rows ? *reinterpret_cast<const u32x4*>(h + (size_t)r * d + c8 * 8) : u32x4{0u, 0u, 0u, 0u};
    const int pass = r / kHeadRows, rr = r % kHeadRows;
    const int kt = (c8 * 8) / kHBK, cc = (c8 * 8) % kHBK;
    const size_t at = (((size_t)pass * (d / kHBK) + kt) * kHeadRows + rr) * kHBK + cc;
    *reinterpret_cast<u32x4*>(hs + at) = v;
}

// ------------------------------------------------------------------ finalize
constexpr int kFinMaxSeg = 8192;  // segments per row the finalize stages in LDS

struct FinArgs {
    const SegStat* stats;
    const u32x4* cand;
    const u32x2* gsum;
    const uint16_t* h;     // [rows, d] bf16: recomputes the logits of the drawn group
    const uint16_t* w;     // [V, d] bf16
    int d;
    const uint64_t* seeds;
    uint64_t step;
    int nseg, gamma, k, V;
    double c2;       // log2(e) / T as used by the segment sums
    int want_exp, want_draw;
    int32_t* idx;
    float* val;
    double* lse;
    int32_t* draft;
};

// A workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight across it (a full barrier waits for every one of them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void block_best(float& v, int& i, float* sv, int* si) {
    wave_best(v, i);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { sv[wave] = v; si[wave] = i; }
    __syncthreads();
    v = sv[0];
    i = si[0];
#pragma unroll
    for (int w = 1; w < kFinThreads / 64; ++w) best_of(v, i, sv[w], si[w]);
    __syncthreads();
}

__device__ __forceinline__ int block_min(int v, int* si) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = min(v, __shfl_xor(v, 1));
    v = min(v, __shfl_xor(v, 2));
    v = min(v, __shfl_xor(v, 4));
    v = min(v, __shfl_xor(v, 8));
    v = min(v, __shfl_xor(v, 16));
    v = min(v, __shfl_xor(v, 32));
    if (lane == 0) si[wave] = v;
    __syncthreads();
    int r = si[0];
#pragma unroll
    for (int w = 1; w < kFinThreads / 64; ++w) r = min(r, si[w]);
    __syncthreads();
    return r;
}

// segment j's mass relative to the row maximum mx
__device__ __forceinline__ double seg_mass(float s, float m, float mx, double c2) {
    return (double)s * exp2(((double)m - (double)mx) * c2);
}

// position of the r-th (0-based) set bit of m (r < popcount(m))
__device__ __forceinline__ int nth_set_bit(uint32_t m, int r) {
    int pos = 0;
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1) {
        const int c = __builtin_popcount(m & ((1u << w) - 1u));
        if (r >= c) { r -= c; m >>= w; pos += w; }
    }
    return pos;
}

constexpr int kFinBatch = 8;                         // segment records per thread per preload batch
constexpr int kFinChunk = 8;                         // candidate segments per selection chunk
constexpr int kFinCand = kFinChunk * kQuads * 4;     // candidate entries per chunk

// One workgroup per row.
__global__ void __launch_bounds__(kFinThreads) lm_head_finalize_kernel(FinArgs a) {
    __shared__ float s_m[kFinMaxSeg];
    __shared__ float c_v[kFinCand + kHeadMaxK];
    __shared__ int c_i[kFinCand + kHeadMaxK];
    __shared__ int q_seg[kFinMaxSeg];
    __shared__ float w_v[kHeadMaxK];
    __shared__ int w_i[kHeadMaxK];
    __shared__ int n_q, n_s;
    __shared__ float s_s[kFinMaxSeg];
    __shared__ float s_tm[kFinThreads];
    __shared__ float sv[kFinThreads / 64];
    __shared__ int si[kFinThreads / 64];
    __shared__ double sd[kFinThreads / 64];
    __shared__ float s_z[kGrpW];
    __shared__ double s_tg;
    __shared__ int s_v0;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t R = blockIdx.x;
    const SegStat* st = a.stats + R * a.nseg;
    const u32x4* cd = a.cand + R * a.nseg * kQuads;

    if (tid == 0) n_q = 0;
    // segment statistics into LDS, kFinBatch records per thread in flight
    // (addresses clamped into the row, so no load waits behind a branch); each
    // thread also keeps the largest maximum of the segments it loaded
    float tmax = -INFINITY;
    for (int j0 = 0; j0 < a.nseg; j0 += kFinBatch * kFinThreads) {
        SegStat t[kFinBatch];
#pragma unroll
        for (int q = 0; q < kFinBatch; ++q) {
            const int j = j0 + q * kFinThreads + tid;
            t[q] = st[j < a.nseg ? j : a.nseg - 1];
        }
#pragma unroll
        for (int q = 0; q < kFinBatch; ++q) {
            const int j = j0 + q * kFinThreads + tid;
            if (j < a.nseg) {
                s_m[j] = t[q].m;
                s_s[j] = t[q].s;
                tmax = fmaxf(tmax, t[q].m);
            }
        }
    }
    s_tm[tid] = tmax;
    __syncthreads();

    // tau: the k-th largest of the threads' maxima, counting repeats (-inf
    // when fewer than k are above -inf).  Those k maxima are k distinct
    // entries of the row, so tau bounds the row's k-th largest entry from
    // below and every top-k entry lies in a segment whose maximum is >= tau.
    // Every wave computes it (and the row maximum mx) from the same 256
    // values, with wave-level reductions only: no barrier per round.
    constexpr int kTm = kFinThreads / 64;
    float cm[kTm];
    float lm = -INFINITY;
#pragma unroll
    for (int q = 0; q < kTm; ++q) {
        cm[q] = s_tm[q * 64 + lane];
        lm = fmaxf(lm, cm[q]);
    }
    const float mx = wave_max(lm);
    float tau = -INFINITY;
    {
        float t = INFINITY;
        int counted = 0;
        for (;;) {
            float m = -INFINITY;
#pragma unroll
            for (int q = 0; q < kTm; ++q)
                if (cm[q] < t) m = fmaxf(m, cm[q]);
            m = wave_max(m);
            if (m == -INFINITY) break;
#pragma unroll
            for (int q = 0; q < kTm; ++q) counted += __popcll(__ballot(cm[q] == m));
            if (counted >= a.k) { tau = m; break; }
            t = m;
        }
    }

    // ---- log-normaliser and the draw's location (before the top-k, so the
    // loads of the drawn group's weight rows are in flight while it runs)
    const int j0 = (int)((long)tid * a.nseg / kFinThreads);
    const int j1 = (int)((long)(tid + 1) * a.nseg / kFinThreads);
    int J = 0;
    // the group's 16 logits are recomputed: wave w takes entries 4w .. 4w+3,
    // each lane a strided set of 16-byte chunks of the hidden row and weight
    // rows (entries past the vocabulary read its last row and weigh nothing);
    // the first kRecHold chunks per lane are loaded before the top-k runs
    constexpr int kRecHold = 10;
    const int nch = a.d / 8;
    const size_t hoff = R * (size_t)a.d;
    size_t woff[4] = {0, 0, 0, 0};  // element offsets of the 4 weight rows of this wave
    u32x4 hv[kRecHold], wv[kRecHold][4];
    int v0 = 0;
    if (a.want_exp) {
        // segment masses in vocabulary order: contiguous runs per thread, fp64
        double run = 0.0;
        for (int j = j0; j < j1; ++j) run += seg_mass(s_s[j], s_m[j], mx, a.c2);
        const double incl = wave_inclusive_scan(run);
        double excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0;
        if (lane == 63) sd[wave] = incl;
        __syncthreads();
        double before = 0.0, total = 0.0;
#pragma unroll
        for (int w = 0; w < kFinThreads / 64; ++w) {
            if (w < wave) before += sd[w];
            total += sd[w];
        }
        excl += before;
        if (tid == 0 && a.lse) a.lse[R] = (double)mx * a.c2 * kLn2 + log(total);
        if (a.want_draw) {
            const int b = (int)(R / a.gamma), g = (int)(R % a.gamma);
            const double u = philox_uniform(a.seeds[b], a.step, (uint64_t)b, (uint64_t)g, kDraftDraw);
            const double tgt = u * total;
            // the segment J where the running mass (vocabulary order) first
            // exceeds u S, or the last segment with mass when rounding leaves no
            // crossing; each thread notes the mass before its own candidates
            int first = kNone, last = -1;
            double before_first = 0.0, before_last = 0.0;
            double cum = excl;
            for (int j = j0; j < j1; ++j) {
                const double sj = seg_mass(s_s[j], s_m[j], mx, a.c2);
                if (sj > 0.0) {
                    if (cum + sj > tgt && first == kNone) { first = j; before_first = cum; }
                    last = j;
                    before_last = cum;
                }
                cum += sj;
            }
            const int my_first = first, my_last = last;
            first = block_min(first, si);
            last = -block_min(-last, si);
            J = first != kNone ? first : last;
            if (J < 0) J = 0;  // no positive mass (non-finite logits): any segment, never out of range
            if (j0 <= J && J < j1) {
                // the thread whose run holds J: the group inside J, from J's eight
                // group sums (in units of J's weights 2^((z - m_J) c2))
                const double before_J = J == my_first ? before_first : (J == my_last ? before_last : 0.0);
                const double t = (tgt - before_J) / exp2(((double)s_m[J] - (double)mx) * a.c2);
                const u32x2* gp = a.gsum + ((size_t)R * a.nseg + J) * 4;
                float gs[8];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x2 x = gp[q];
                    gs[2 * q] = __uint_as_float(x[0]);
                    gs[2 * q + 1] = __uint_as_float(x[1]);
                }
                int G = -1, Gl = -1;
                double bG = 0.0, bGl = 0.0, c = 0.0;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (gs[q] > 0.f) {
                        if (G < 0 && c + (double)gs[q] > t) { G = q; bG = c; }
                        Gl = q;
                        bGl = c;
                    }
                    c += (double)gs[q];
                }
                if (G < 0) { G = Gl < 0 ? 0 : Gl; bG = Gl < 0 ? 0.0 : bGl; }
                s_v0 = J * kSegW + G * kGrpW;
                s_tg = t - bG;
            }
            __syncthreads();
            v0 = s_v0;
#pragma unroll
            for (int e = 0; e < 4; ++e) woff[e] = (size_t)min(v0 + wave * 4 + e, a.V - 1) * a.d;
#pragma unroll
            for (int u = 0; u < kRecHold; ++u) {
                const int c = min(lane + 64 * u, nch - 1);  // clamped: not added
                hv[u] = *reinterpret_cast<const u32x4*>(a.h + hoff + c * 8);
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[u][e] = *reinterpret_cast<const u32x4*>(a.w + woff[e] + c * 8);
            }
        }
    }

    // the segments that can hold a top-k entry (m >= tau), in any order
    for (int j = tid; j < a.nseg; j += kFinThreads)
        if (s_m[j] >= tau) q_seg[atomicAdd(&n_q, 1)] = j;
    lds_barrier();
    const int nq = n_q;

    // Only entries >= tau can rank (tau is at most the row's k-th largest
    // value), and every top-k entry's quad was recorded by its segment.  The
    // records of the candidate segments are unpacked keeping just those
    // entries; when at most kFinThreads survive (the usual case), each thread
    // ranks one by counting the survivors ranked ahead of it (every index
    // appears once, so the ranks are 0, 1, ... without repeats).
    const int k = a.k;
    if (tid == 0) n_s = 0;
    lds_barrier();
    for (int slot = tid; slot < nq * kQuads; slot += kFinThreads) {
        const int j = q_seg[slot / kQuads], r = slot % kQuads;
        // the record slot is read with the mask (slots past the mask's count
        // hold stale data and are ignored)
        const uint32_t mask = (uint32_t)st[j].mask;
        const u32x4 q = cd[(size_t)j * kQuads + r];
        if (r < __builtin_popcount(mask)) {
            const int bit = nth_set_bit(mask, r);
            const int i0 = j * kSegW + (bit >> 2) * 16 + (bit & 3) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = __uint_as_float(q[e]);
                if (i0 + e < a.V && v >= tau) {
                    const int at = atomicAdd(&n_s, 1);
                    if (at < kFinCand) { c_v[at] = v; c_i[at] = i0 + e; }
                }
            }
        }
    }
    lds_barrier();
    const int ns = n_s;
    int top1;
    if (ns <= kFinThreads) {
        const bool mine = tid < ns;
        const float v = mine ? c_v[tid] : -INFINITY;
        const int i = mine ? c_i[tid] : -1;
        int rank = 0;
        for (int e = 0; e < ns; ++e) rank += ranks_ahead(c_v[e], c_i[e], v, i) ? 1 : 0;
        if (mine && rank < k) {
            a.idx[R * k + rank] = i;
            a.val[R * k + rank] = v;
            if (rank == 0) w_i[0] = i;
        }
        lds_barrier();
        top1 = w_i[0];
    } else {
        // many entries >= tau (long runs of equal logits): chunks of kFinChunk
        // segments, every record unpacked into LDS, then k rounds of a
        // block-wide (value desc, index asc) selection over the chunk and the
        // running top k (kept in the last kHeadMaxK entries)
        if (tid < kHeadMaxK) { c_v[kFinCand + tid] = -INFINITY; c_i[kFinCand + tid] = -1; }
        for (int c0 = 0; c0 < nq; c0 += kFinChunk) {
            for (int slot = tid; slot < kFinChunk * kQuads; slot += kFinThreads) {
                const int qi = c0 + slot / kQuads, r = slot % kQuads;
                float v4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                int i0 = -1;
                if (qi < nq) {
                    const int j = q_seg[qi];
                    const uint32_t mask = (uint32_t)st[j].mask;
                    if (r < __builtin_popcount(mask)) {
                        const u32x4 q = cd[(size_t)j * kQuads + r];
                        const int bit = nth_set_bit(mask, r);
                        i0 = j * kSegW + (bit >> 2) * 16 + (bit & 3) * 4;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            v4[e] = i0 + e < a.V ? __uint_as_float(q[e]) : -INFINITY;
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    c_v[slot * 4 + e] = v4[e];
                    c_i[slot * 4 + e] = v4[e] > -INFINITY ? i0 + e : -1;
                }
            }
            __syncthreads();
            float qv = INFINITY;
            int qi_ = -1;
            for (int r = 0; r < k; ++r) {
                float bv = -INFINITY;
                int bi = -1;
                for (int e = tid; e < kFinCand + k; e += kFinThreads) {  // chunk, then running top k
                    const float v = c_v[e];
                    const int i = c_i[e];
                    if (i >= 0 && ranks_ahead(qv, qi_, v, i) && ranks_ahead(v, i, bv, bi)) { bv = v; bi = i; }
                }
                block_best(bv, bi, sv, si);
                if (tid == 0) { w_v[r] = bv; w_i[r] = bi; }
                qv = bv;
                qi_ = bi;
            }
            __syncthreads();
            if (tid < k) { c_v[kFinCand + tid] = w_v[tid]; c_i[kFinCand + tid] = w_i[tid]; }
            __syncthreads();
        }
        if (tid < k) {
            a.idx[R * k + tid] = c_i[kFinCand + tid];
            a.val[R * k + tid] = c_v[kFinCand + tid];
        }
        top1 = c_i[kFinCand];
    }


    if (!a.want_exp) {
        if (tid == 0) {
            if (a.lse) a.lse[R] = NAN;
            if (a.draft) a.draft[R] = top1;
        }
        return;
    }
    if (!a.want_draw) return;
    auto dot8 = [](const u32x4& h, const u32x4& w, float acc) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = __builtin_fmaf(__uint_as_float(h[q] << 16), __uint_as_float(w[q] << 16), acc);
            acc = __builtin_fmaf(__uint_as_float(h[q] & 0xFFFF0000u), __uint_as_float(w[q] & 0xFFFF0000u), acc);
        }
        return acc;
    };
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kRecHold; ++u) {
        if (lane + 64 * u >= nch) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) part[e] = dot8(hv[u], wv[u][e], part[e]);
    }
    // chunks past the first kRecHold per lane (d_model > 5,120)
    for (int c = lane + 64 * kRecHold; c < nch; c += 64) {
        const u32x4 h1 = *reinterpret_cast<const u32x4*>(a.h + hoff + c * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            part[e] = dot8(h1, *reinterpret_cast<const u32x4*>(a.w + woff[e] + c * 8), part[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) part[e] = wave_sum(part[e]);
    if (lane == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s_z[wave * 4 + e] = part[e];
    }
    lds_barrier();
    if (tid == 0) {
        // the entry of the group where the running weight first passes the
        // rest of the target (weights by the epilogue's own formula)
        const float c2f = (float)a.c2;
        const float mc = s_m[J] * c2f;
        const double tg = s_tg;
        double acc = 0.0;
        int pick = -1, lastp = -1;
        for (int e = 0; e < kGrpW; ++e) {
            const int v = v0 + e;
            const float wgt = v < a.V ? fast_exp2(__builtin_fmaf(s_z[e], c2f, -mc)) : 0.f;
            if (wgt > 0.f) {
                acc += (double)wgt;
                lastp = v;
                if (pick < 0 && acc > tg) pick = v;
            }
        }
        a.draft[R] = pick >= 0 ? pick : (lastp >= 0 ? lastp : min(v0, a.V - 1));
    }
}

struct HeadLayout {
    size_t stats, cand, gsum, hs, bytes;
};

HeadLayout head_layout(int rows, int vocab, int d) {
    const size_t nseg = ((size_t)vocab + kSegW - 1) / kSegW;
    const size_t npass = ((size_t)rows + kHeadRows - 1) / kHeadRows;
    HeadLayout L{};
    Carve c;
    L.stats = c.take<SegStat>((size_t)rows * nseg);
    L.cand = c.take<u32x4>((size_t)rows * nseg * kQuads);
    L.gsum = c.take<u32x2>((size_t)rows * nseg * 4);
    L.hs = c.take<uint16_t>(npass * kHeadRows * (size_t)d);
    L.bytes = c.total();
    return L;
}

void launch_head(int tt, dim3 grid, const HeadArgs& a, hipStream_t st) {
    const dim3 block(64 * kHWaves);
    switch (tt) {
        case 1: hipLaunchKernelGGL(lm_head_kernel<1>, grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL(lm_head_kernel<2>, grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL(lm_head_kernel<3>, grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL(lm_head_kernel<4>, grid, block, 0, st, a); break;
    }
}

}  // namespace
}  // namespace dfl

using namespace dfl;

namespace dfl {
namespace {

// Size part of the checks (every size already >= 1): true when the kernels run
// this shape.  The row cap keeps the finalize's one workgroup per row within a
// launch's 32-bit count of work-items and the 256-row passes within int.
bool head_shape_ok(int rows, int d_model, int vocab, int k) {
    return k <= kHeadMaxK && k <= vocab && d_model % kHBK == 0 && d_model <= kHeadMaxD &&
           vocab <= kFinMaxSeg * kSegW && rows <= kMaxRowsPerCall;
}

}  // namespace
}  // namespace dfl

extern "C" size_t dflash_lm_head_topk_workspace_size(int rows, int d_model, int vocab, int k) {
    if (rows < 1 || d_model < 1 || vocab < 1 || k < 1 || !head_shape_ok(rows, d_model, vocab, k))
        return 0;
    return head_layout(rows, vocab, d_model).bytes;
}

extern "C" int dflash_lm_head_topk(const uint16_t* hidden, const uint16_t* w_head, int rows,
                                   int gamma, int d_model, int vocab, int k, float temperature,
                                   const uint64_t* seeds, uint64_t step, int32_t* topk_idx,
                                   float* topk_val, double* lse, int32_t* draft, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (rows < 0 || gamma < 1 || d_model < 1 || vocab < 1 || k < 1 || k > vocab)
        return DFLASH_ERR_SHAPE;
    if (!(temperature >= 0.f) || !std::isfinite(temperature)) return DFLASH_ERR_SHAPE;
    if (rows == 0) return DFLASH_OK;
    if (!hidden || !w_head || !topk_idx || !topk_val) return DFLASH_ERR_NULL;
    const bool sample = temperature > 0.f;
    if (sample && draft && !seeds) return DFLASH_ERR_NULL;
    if (!head_shape_ok(rows, d_model, vocab, k) || (reinterpret_cast<uintptr_t>(hidden) & 15) ||
        (reinterpret_cast<uintptr_t>(w_head) & 15))
        return DFLASH_ERR_UNSUPPORTED;
    const HeadLayout L = head_layout(rows, vocab, d_model);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) || workspace_bytes < L.bytes)
        return DFLASH_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);

    const int nseg = (vocab + kSegW - 1) / kSegW;
    HeadArgs ha{};
    ha.h = hidden;
    ha.hs = reinterpret_cast<uint16_t*>(ws + L.hs);
    {
        const int64_t pieces = ((int64_t)(rows + kHeadRows - 1) / kHeadRows) * kHeadRows * (d_model / 8);
        hipLaunchKernelGGL(head_slabs_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, st, hidden, rows,
                           d_model, const_cast<uint16_t*>(ha.hs));
        const int rc = launch_status();
        if (rc) return rc;
    }
    ha.w = w_head;
    ha.stats = reinterpret_cast<SegStat*>(ws + L.stats);
    ha.cand = reinterpret_cast<u32x4*>(ws + L.cand);
    ha.gsum = reinterpret_cast<u32x2*>(ws + L.gsum);
    ha.d = d_model;
    ha.V = vocab;
    ha.nseg = nseg;
    ha.groups = min(kHeadCUs, (nseg + 1) / 2);
    ha.k = k;
    ha.c2 = sample ? (float)(1.4426950408889634 / (double)temperature) : 0.f;
    ha.want_exp = sample && (lse || draft);
    ha.want_draw = sample && draft;
    for (int row0 = 0; row0 < rows; row0 += kHeadRows) {
        ha.row0 = row0;
        ha.M = min(kHeadRows, rows - row0);
        launch_head(min(4, (k + 1) / 2), dim3(ha.groups), ha, st);
        const int rc = launch_status();
        if (rc) return rc;
    }
    FinArgs fa{};
    fa.stats = ha.stats;
    fa.cand = ha.cand;
    fa.gsum = ha.gsum;
    fa.h = hidden;
    fa.w = w_head;
    fa.d = d_model;
    fa.seeds = seeds;
    fa.step = step;
    fa.nseg = nseg;
    fa.gamma = gamma;
    fa.k = k;
    fa.V = vocab;
    fa.c2 = (double)ha.c2;
    fa.want_exp = ha.want_exp;
    fa.want_draw = ha.want_draw;
    fa.idx = topk_idx;
    fa.val = topk_val;
    fa.lse = lse;
    fa.draft = draft;
    hipLaunchKernelGGL(lm_head_finalize_kernel, dim3(rows), dim3(kFinThreads), 0, st, fa);
    return launch_status();
}
