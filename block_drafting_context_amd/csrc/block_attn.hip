// block_attn.hip -- block-draft attention for gfx950.
//
// "DFlash vs DFlash 2", "DFlash: generate the block all at once" and
// "Conditioning on the target model" (Q_i, K_i, V_i equation): the block's
// queries attend without a causal mask to the context window and to the
// block's own keys.  "Beam 1.0 DFlash2", "Model": 40 query heads share 8 KV
// heads of dimension 128; the window holds the last 4,096 context tokens.
//
// bf16 path.  One workgroup owns one (sequence, KV head, key split, group of
// query tiles).  The key sequence of a (sequence, KV head) is virtual: index
// t < n_b reads ring slot t, t >= n_b reads block row t - n_b, so the block
// keys are streamed like the window keys.  Every query row of the GQA group
// (group * gamma rows, padded to 16) is a column of one MFMA tile, so each
// K/V byte is fetched from HBM once and used by all query heads of its group.
//
// Four waves per workgroup, one per SIMD, split the keys: each wave streams
// its own 32-key K and V tiles into two private LDS stages with non-temporal
// global_load_lds (HBM to LDS, no registers), so loads and compute overlap
// without any barrier between waves.  A wave computes all query tiles of its
// group (up to three 16-column MFMA tiles), so every K/V operand it reads
// from LDS serves all of them: S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_16x16x32_bf16, V^T read with LDS transpose loads, online softmax
// in base 2 with a lazily raised reference max.  The waves' partial softmax
// states are merged through LDS; key splits (only when the grid would not
// fill the GPU) are merged by a second kernel.
//
// fp32 path (small shapes): one wave per query, scores in LDS, exact expf.
#include <cmath>

#include "common.hpp"

namespace dfl {
DFL_VIOLATION_WORD(violations_attn)
namespace {

constexpr int TK = 32;             // keys per tile
constexpr int kWaves = 4;          // waves per workgroup, one per SIMD
constexpr int kMaxNCT = 3;         // 16-column query tiles per wave
constexpr int kCUs = 256;          // MI355X compute units
constexpr int kLdsPerCU = 160 * 1024;
constexpr int kMinKeysPerSplit = 512;  // at least 4 tiles per wave in every key split
constexpr int kMaxWindow = 1 << 28;        // ring slots per (sequence, KV head)
constexpr int64_t kMaxQueryRows = 1 << 28;  // batch * gamma * n_q
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may trail the true max

struct AttnArgs {
    const uint16_t* q;
    const uint16_t* kb;
    const uint16_t* vb;
    const uint16_t* kr;
    const uint16_t* vr;
    const int64_t* ctx_len;
    float scale_log2;  // softmax scale * log2(e)
    uint16_t* out;
    float* lse;
    float* part_o;   // [B*HKV][n_splits][n_qt*16][D]
    float* part_ml;  // [B*HKV][n_splits][n_qt*16][2]  (reference max, sum), base 2
    int B, G, HQ, HKV, W, group, nrows, n_qt, n_splits;
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define DFL_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define DFL_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))

// Wait until every LDS operation of this wave has completed.
__device__ __forceinline__ void wait_lds() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    // s_waitcnt encoding on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Block-draft attention, bf16.
//
// Workgroup = 4 waves (one per SIMD) for one (sequence, KV head, key split,
// group of up to NCT query tiles).  Wave w takes the 32-key tiles w, w+4,
// w+8, ... of the split and streams each into its own two LDS stages with
// non-temporal global_load_lds_dwordx4 (HBM to LDS, no registers): the next
// tile is in flight while the current one is computed, and no wave ever
// waits for another inside the key loop.  K rows are stored with 16-byte
// chunk c of row r at chunk c ^ (r % 16) (conflict-free ds_read_b128 of the
// S^T = K Q^T operand); V rows with 32-byte double chunk d of row r at
// d ^ (r % 8), which ds_read_b64_tr_b16 turns into the dims-by-keys operand
// of O^T += V^T P^T.  Every K/V operand read from LDS serves all NCT query
// tiles of the wave.  The four waves' softmax states (max, sum, O) are merged
// through LDS at the end.
template <int D, int NCT>
__global__ void __launch_bounds__(256) block_attn_bf16_kernel(AttnArgs a) {
    constexpr int ROWB = D * 2;               // bytes per key row
    constexpr int CHR = ROWB / 16;            // 16-byte chunks per row
    constexpr int TILEB = TK * ROWB;          // bytes of one K (or V) tile
    constexpr int NI = TILEB / 1024;          // 1 KB load instructions per K (or V) tile
    constexpr int RPI = 1024 / ROWB;          // rows per load instruction
    constexpr int DT = D / 16;                // 16-dim tiles of O^T
    constexpr int KS = D / 32;                // k-steps of S^T
    constexpr int OSTR = 17;                  // padded row stride of the merge buffer
    static_assert(4 * NI <= 63, "vmcnt");
    static_assert(kWaves * 2 * 2 * TILEB >= (kWaves * NCT * D * OSTR + 2 * kWaves * NCT * 16) * 4,
                  "merge buffer fits in the ring");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kWaves][2][2][TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char sq[NCT * 16 * ROWB];

    const int split = blockIdx.x;
    const int bk = blockIdx.y;
    const int b = bk / a.HKV, kvh = bk % a.HKV;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int g = lane >> 4, i16 = lane & 15;

    const int64_t cl = a.ctx_len[b];
    if (DFLASH_DEVICE_CHECKS && cl < 0 && tid == 0) DFL_VIOLATION(DFLASH_VIOLATION_CTX_LEN);
    const int n = (int)(cl < (int64_t)a.W ? (cl < 0 ? 0 : cl) : (int64_t)a.W);
    const int total = n + a.G;
    int per = (total + a.n_splits - 1) / a.n_splits;
    per = (per + TK - 1) / TK * TK;
    const int t0 = split * per;
    const int t1 = min(t0 + per, total);
    const int ntiles = t1 > t0 ? (t1 - t0 + TK - 1) / TK : 0;
    const int mine = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;  // tiles of this wave

    // ---- loads of this wave's j-th tile (tile wave + 4 j of the split) into stage j % 2
    const uint16_t* kring = a.kr + (size_t)bk * a.W * D;
    const uint16_t* vring = a.vr + (size_t)bk * a.W * D;
    const size_t blk_off = ((size_t)b * a.G * a.HKV + kvh) * D;
    const size_t blk_stride = (size_t)a.HKV * D;
    const int rl = lane / CHR, p = lane % CHR;  // row within an instruction, physical chunk
    // The swizzle of instruction ins depends on (ins * RPI + rl) % CHR, which repeats
    // every NPAT instructions: per-lane byte offsets of the first NPAT instructions.
    constexpr int NPAT = CHR > RPI ? CHR / RPI : 1;
    uint32_t koff[NPAT], voff[NPAT];
#pragma unroll
    for (int q = 0; q < NPAT; ++q) {
        const int r = q * RPI + rl;
        const int ck = p ^ (r % CHR);
        const int cv = ((((p >> 1) ^ (r % (CHR / 2)))) << 1) | (p & 1);
        koff[q] = (uint32_t)((r * D + ck * 8) * 2);
        voff[q] = (uint32_t)((r * D + cv * 8) * 2);
    }
    // loads of this wave's j-th tile (tile wave + 4 j of the split), K (kv = 0) or V (kv = 1)
    // half, into stage j % 2
    auto issue = [&](int j, int kv) {
        const int tb = t0 + (wave + kWaves * j) * TK;
        unsigned char* dst = smem[wave][j & 1][kv];
        const uint16_t* ring = kv ? vring : kring;
        if (tb + TK <= min(n, t1)) {
            // whole tile inside the ring: wave-uniform base + per-lane offset
            const unsigned char* base = reinterpret_cast<const unsigned char*>(ring + (size_t)tb * D);
#pragma unroll
            for (int ins = 0; ins < NI; ++ins) {
                const int q = ins % NPAT, hi = (ins / NPAT) * NPAT * 1024;
                __builtin_amdgcn_global_load_lds(DFL_GLOBAL(base + hi + (kv ? voff[q] : koff[q])),
                                                 DFL_LDS(dst + ins * 1024), 16, 0, kLoadStream);
            }
            return;
        }
        // tile with block rows or past the end of the split: row by row
        const uint16_t* blk = kv ? a.vb : a.kb;
#pragma unroll
        for (int ins = 0; ins < NI; ++ins) {
            const int r = ins * RPI + rl;
            int t = tb + r;
            if (t >= t1) t = t1 - 1;  // masked key: any valid row
            const uint16_t* row = t < n ? ring + (size_t)t * D : blk + blk_off + (size_t)(t - n) * blk_stride;
            const int c = kv ? ((((p >> 1) ^ (r % (CHR / 2)))) << 1) | (p & 1) : p ^ (r % CHR);
            __builtin_amdgcn_global_load_lds(DFL_GLOBAL(row + c * 8), DFL_LDS(dst + ins * 1024), 16, 0,
                                             kLoadStream);
        }
    };
    // two tiles in flight per wave: K and V of tiles 0 and 1
    for (int j = 0; j < 2 && j < mine; ++j) {
        issue(j, 0);
        issue(j, 1);
    }

    // ---- the workgroup's query rows (columns of S^T: (block row, head) pairs) in LDS,
    // 16-byte chunk c of row q at chunk c ^ (q % CHR); rows past the group are zero
    for (int idx = tid; idx < NCT * 16 * CHR; idx += 64 * kWaves) {
        const int qr = idx / CHR, c = idx % CHR;
        const int j = blockIdx.z * NCT * 16 + qr;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < a.nrows) {
            const int r = j / a.group, hl = j % a.group;
            v = *reinterpret_cast<const u32x4*>(
                a.q + ((size_t)((size_t)b * a.G + r) * a.HQ + kvh * a.group + hl) * D + c * 8);
        }
        *reinterpret_cast<u32x4*>(sq + qr * ROWB + ((c ^ (qr % CHR)) * 16)) = v;
    }
    __syncthreads();

    f32x4 o[NCT][DT];
    float m_run[NCT], l_run[NCT];  // running reference max (base 2) and this lane's share of the sum
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[ct] = -INFINITY;
        l_run[ct] = 0.f;
    }

    // S^T of this wave's tile j (waits for it, starts the loads of tile j + 1);
    // sx = raw scores with keys past the split masked, tmax = column max in base 2
    f32x4 sx[NCT][2];
    float tmax[NCT];
    auto scores = [&](int j) {
        // loads are issued in the order K(j) V(j) K(j+1) V(j+1): wait for the first two
        if (j + 1 < mine) wait_vmem<2 * NI>();
        else wait_vmem<0>();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const int tb = t0 + (wave + kWaves * j) * TK;
        const unsigned char* kt = smem[wave][j & 1][0];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int st = 0; st < 2; ++st) sx[ct][st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 qv[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const int qr = ct * 16 + i16;
                qv[ct] = *reinterpret_cast<const u32x4*>(sq + qr * ROWB + (((s * 4 + g) ^ (qr % CHR)) * 16));
            }
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const int r = st * 16 + i16;
                const u32x4 kvv = *reinterpret_cast<const u32x4*>(
                    kt + r * ROWB + (((s * 4 + g) ^ (r % CHR)) * 16));
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    sx[ct][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, kvv), __builtin_bit_cast(bf16x8, qv[ct]), sx[ct][st],
                        0, 0, 0);
            }
        }
        // K(j) has been read: refill its stage with K(j + 2)
        wait_lds();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (j + 2 < mine) issue(j + 2, 0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (tb + TK > t1) {  // the split's last, partial tile
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (tb + st * 16 + g * 4 + e >= t1) sx[ct][st][e] = -INFINITY;
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float mx = sx[ct][0][0];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sx[ct][st][e]);
            tmax[ct] = xor32_max(xor16_max(mx)) * a.scale_log2;
        }
    };
    // P^T = 2^(S^T scale - m_run) packed to bf16 in the B-operand layout (k position
    // 8g + e holds key 4g + e, 8g + 4 + e holds key 16 + 4g + e), then O^T += V^T P^T
    auto accumulate = [&](int j) {
        const unsigned char* vt = smem[wave][j & 1][1];
        bf16x8 pb[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float pv[8];
            float psum = 0.f;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pv[st * 4 + e] = fast_exp2(fmaf(sx[ct][st][e], a.scale_log2, -m_run[ct]));
                    psum += pv[st * 4 + e];
                }
            u32x4 pk;
            pk[0] = pack_bf16x2(pv[0], pv[1]);
            pk[1] = pack_bf16x2(pv[2], pv[3]);
            pk[2] = pack_bf16x2(pv[4], pv[5]);
            pk[3] = pack_bf16x2(pv[6], pv[7]);
            pb[ct] = __builtin_bit_cast(bf16x8, pk);
            l_run[ct] += psum;
        }
        // the V^T operand (16 dims x 8 keys per lane) comes from two transposing
        // reads, keys 4g + {0..3} and 16 + 4g + {0..3}
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            v4i16 h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int r = hh * 16 + g * 4 + (i16 >> 2);
                const unsigned char* src = vt + r * ROWB + ((dt ^ (r % (CHR / 2))) * 32) + (i16 & 3) * 8;
                h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16*)(DFL_LDS(src)));
            }
            u32x4 av;
            av[0] = __builtin_bit_cast(u32x2, h[0])[0];
            av[1] = __builtin_bit_cast(u32x2, h[0])[1];
            av[2] = __builtin_bit_cast(u32x2, h[1])[0];
            av[3] = __builtin_bit_cast(u32x2, h[1])[1];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                o[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb[ct],
                                                                    o[ct][dt], 0, 0, 0);
        }
        // V(j) has been read: refill its stage with V(j + 2)
        wait_lds();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (j + 2 < mine) issue(j + 2, 1);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // The reference max m_run is raised only when a tile's max exceeds it by more
    // than kRescaleSlack (then O and the sum are rescaled).  That rare step sits
    // outside the key loop, so the loop touches O only through the matrix cores.
    int j = 0;
    while (j < mine) {
        bool raise = false;
        for (; j < mine; ++j) {
            scores(j);
            bool r = false;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) r = r || (tmax[ct] > m_run[ct] + kRescaleSlack);
            raise = __ballot(r) != 0;  // wave-uniform
            if (raise) break;
            accumulate(j);
        }
        if (!raise) break;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const float mnew = fmaxf(m_run[ct], tmax[ct]);
            const float alpha = fast_exp2(m_run[ct] - mnew);
            l_run[ct] *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[ct][dt] *= alpha;
            m_run[ct] = mnew;
        }
        accumulate(j);
        ++j;
    }

    // ---- merge the four waves: M = max m_w, O = sum O_w 2^(m_w - M), L likewise
    // the 4 lane groups of a column hold disjoint keys: column sums
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) l_run[ct] = xor32_sum(xor16_sum(l_run[ct]));
    __syncthreads();  // every wave is done with its stages
    float* mb = reinterpret_cast<float*>(&smem[0][0][0][0]);  // [wave][ct][16]
    float* lb = mb + kWaves * NCT * 16;                        // [wave][ct][16]
    float* ob = lb + kWaves * NCT * 16;                        // [wave][ct][D][OSTR]
    if (g == 0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) mb[(wave * NCT + ct) * 16 + i16] = m_run[ct];
    }
    __syncthreads();
    float M[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        M[ct] = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M[ct] = fmaxf(M[ct], mb[(w * NCT + ct) * 16 + i16]);
        const float f = m_run[ct] == -INFINITY ? 0.f : fast_exp2(m_run[ct] - M[ct]);
        if (g == 0) lb[(wave * NCT + ct) * 16 + i16] = l_run[ct] * f;
        float* od = ob + (size_t)(wave * NCT + ct) * D * OSTR;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) od[(dt * 16 + g * 4 + e) * OSTR + i16] = o[ct][dt][e] * f;
    }
    __syncthreads();
    // wave w finishes the 16-dim tiles dt = w, w + 4, ...
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        const int j = (blockIdx.z * NCT + ct) * 16 + i16;
        if (j >= a.nrows) continue;
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) L += lb[(w * NCT + ct) * 16 + i16];
        const int r = j / a.group, h = kvh * a.group + j % a.group;
        const size_t row = ((size_t)b * a.G + r) * a.HQ + h;
        const size_t prow = ((size_t)bk * a.n_splits + split) * (a.n_qt * 16) + j;
        for (int dt = wave; dt < DT; dt += kWaves) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float* od = ob + (size_t)(w * NCT + ct) * D * OSTR;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += od[(dt * 16 + g * 4 + e) * OSTR + i16];
            }
            if (a.n_splits == 1) {
                const float inv = 1.f / L;
                u32x2 w2;
                w2[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
                w2[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
                *reinterpret_cast<u32x2*>(a.out + row * D + dt * 16 + g * 4) = w2;
            } else {
                *reinterpret_cast<f32x4*>(a.part_o + prow * D + dt * 16 + g * 4) = acc;
            }
        }
        if (wave == 0 && g == 0) {
            if (a.n_splits == 1) {
                if (a.lse) a.lse[row] = (M[ct] + __log2f(L)) * (float)kLn2;
            } else {
                a.part_ml[prow * 2 + 0] = M[ct];
                a.part_ml[prow * 2 + 1] = L;
            }
        }
    }
}

// Merge key splits: O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// One workgroup per (sequence, KV head, query tile); 16 threads per row.
template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(AttnArgs a) {
    const int bk = blockIdx.x, qt = blockIdx.y;
    const int b = bk / a.HKV, kvh = bk % a.HKV;
    const int jl = threadIdx.x >> 4, part = threadIdx.x & 15;
    const int j = qt * 16 + jl;
    if (j >= a.nrows) return;
    const int S = a.n_splits;
    const size_t base = (size_t)bk * S * (a.n_qt * 16) + j;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[(base + (size_t)s * a.n_qt * 16) * 2]);
    const float muse = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    constexpr int PER = D / 16;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int s = 0; s < S; ++s) {
        const size_t prow = base + (size_t)s * a.n_qt * 16;
        const float f = fast_exp2(a.part_ml[prow * 2] - muse);
        L += a.part_ml[prow * 2 + 1] * f;
        if (f == 0.f) continue;
        const f32x4* src = reinterpret_cast<const f32x4*>(a.part_o + prow * D + part * PER);
#pragma unroll
        for (int e = 0; e < PER / 4; ++e) {
            const f32x4 v = src[e];
            acc[4 * e + 0] += v[0] * f;
            acc[4 * e + 1] += v[1] * f;
            acc[4 * e + 2] += v[2] * f;
            acc[4 * e + 3] += v[3] * f;
        }
    }
    const float inv = 1.f / L;
    const int r = j / a.group, h = kvh * a.group + j % a.group;
    const size_t row = ((size_t)b * a.G + r) * a.HQ + h;
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.out + row * D + part * PER);
#pragma unroll
    for (int e = 0; e < PER / 2; ++e) dst[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    if (a.lse && part == 0) a.lse[row] = (M + __log2f(L)) * (float)kLn2;
}

// ------------------------------------------------------------- fp32 path
struct Attn32Args {
    const float* q;
    const float* kb;
    const float* vb;
    const float* kr;
    const float* vr;
    const int64_t* ctx_len;
    float scale;
    float* out;
    float* lse;
    int B, G, HQ, HKV, W, D;
    int vec;  // d_head % 4 == 0 and every tensor 16-byte aligned: whole-float4 loads and stores
};

constexpr int kQR32 = 16;   // query rows per workgroup, all of one (sequence, KV head) group
constexpr int kKC32 = 64;   // keys per chunk staged in LDS
constexpr float kSlack32 = 8.f * 0.6931471805599453f;  // natural-log units the reference may trail the max

// Columns 4 c4 .. 4 c4 + 3 of a row of d floats, zero past d.
__device__ __forceinline__ f32x4 load_cols(const float* row, int c4, int d, bool vec) {
    const int c = 4 * c4;
    if (c >= d) return f32x4{0.f, 0.f, 0.f, 0.f};
    if (vec) return *reinterpret_cast<const f32x4*>(row + c);
    f32x4 v = {row[c], 0.f, 0.f, 0.f};
    if (c + 1 < d) v[1] = row[c + 1];
    if (c + 2 < d) v[2] = row[c + 2];
    if (c + 3 < d) v[3] = row[c + 3];
    return v;
}

// fp32 attention of up to 16 query rows of one (sequence, KV head) group
// against that group's keys: the min(len, W) ring rows, then the block's.
// Key chunks of 64 rows are staged in LDS (the next chunk loaded into
// registers while the current one is used); a staged row holds C4 float4
// columns (C4 = the power of two >= d/4, zero past d) plus one, so that
// consecutive rows start 4 banks apart.  Each of the 16 waves owns one query
// row: lane k scores key k of the chunk against it (a sequential fma chain
// over d), the row's maximum and sum are wave reductions, and the row keeps a
// reference that trails its running maximum by at most 8 ln 2 (exp(s - ref)
// stays below 256; output and sum carry the same factor, so their ratio is
// unaffected), rescaled only when a chunk exceeds it.  For O = sum p v, lane
// (q, c) accumulates column c over the chunk's keys q, q + 64/C4, ...; the key
// subsets are summed across lanes at the end.  Four waves per SIMD keep the
// LDS latency of the small per-row chains covered.
constexpr int kRPW32 = 2;                        // query rows per wave
constexpr int kThreads32 = 64 * kQR32 / kRPW32;  // 512
template <int C4>
__global__ void __launch_bounds__(kThreads32) block_attn_f32_kernel(Attn32Args a) {
    constexpr int KQ = 64 / C4;                 // key subsets of the output lanes
    constexpr int RPW = kRPW32;
    constexpr int NW = 64 * C4 / kThreads32 >= 1 ? 64 * C4 / kThreads32 : 1;  // staged rows per thread and chunk
    constexpr int LG = C4 == 1 ? 0 : C4 == 2 ? 1 : C4 == 4 ? 2 : C4 == 8 ? 3 : C4 == 16 ? 4 : 5;
    static_assert((1 << LG) == C4 && C4 <= 32, "C4: a power of two up to 32");
    __shared__ f32x4 qs[kQR32][C4 + 1];
    __shared__ f32x4 ks[kKC32][C4 + 1];
    __shared__ f32x4 vs[kKC32][C4 + 1];
    __shared__ float ps[kQR32][kKC32 + 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int group = a.HQ / a.HKV, nrows = a.G * group;
    const int nrb = (nrows + kQR32 - 1) / kQR32;
    const int rb = blockIdx.x % nrb;
    const int kvh = (blockIdx.x / nrb) % a.HKV, b = blockIdx.x / (nrb * a.HKV);
    const int D = a.D;
    const bool vec = a.vec != 0;

    const int64_t cl = a.ctx_len[b];
    if (DFLASH_DEVICE_CHECKS && cl < 0 && tid == 0) DFL_VIOLATION(DFLASH_VIOLATION_CTX_LEN);
    const int n = (int)(cl < (int64_t)a.W ? (cl < 0 ? 0 : cl) : (int64_t)a.W);
    const int total = n + a.G;
    const int nch = (total + kKC32 - 1) / kKC32;

    // query row jr of the group block -> its flattened (sequence, block row, head)
    auto q_index = [&](int jr) {
        return ((size_t)b * a.G + jr / group) * a.HQ + (size_t)kvh * group + jr % group;
    };
    for (int e = tid; e < kQR32 * C4; e += kThreads32) {
        const int r = e >> LG, c4 = e & (C4 - 1);
        const int jr = rb * kQR32 + r;
        qs[r][c4] = jr < nrows ? load_cols(a.q + q_index(jr) * D, c4, D, vec) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // chunk loads: thread tid stages column tid % C4 of rows tid / C4 + (256 / C4) w
    const int lc4 = tid & (C4 - 1), lrow = tid >> LG;
    const float* kring = a.kr + ((size_t)b * a.HKV + kvh) * a.W * D;
    const float* vring = a.vr + ((size_t)b * a.HKV + kvh) * a.W * D;
    auto key_row = [&](const float* ring, const float* blk, int t) {
        return t < n ? ring + (size_t)t * D : blk + (((size_t)b * a.G + (t - n)) * a.HKV + kvh) * D;
    };
    f32x4 kreg[NW], vreg[NW];
    auto fetch = [&](int c) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int key = lrow + (kThreads32 >> LG) * w, t = c * kKC32 + key;
            const bool ok = key < kKC32 && t < total;
            kreg[w] = ok ? load_cols(key_row(kring, a.kb, t), lc4, D, vec) : f32x4{0.f, 0.f, 0.f, 0.f};
            vreg[w] = ok ? load_cols(key_row(vring, a.vb, t), lc4, D, vec) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };

    float ref[RPW], l[RPW];
    f32x4 acc[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        ref[r] = -INFINITY;
        l[r] = 0.f;
        acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int pc4 = lane & (C4 - 1), kq = lane >> LG;
    fetch(0);
    for (int c = 0; c < nch; ++c) {
        __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int key = lrow + (kThreads32 >> LG) * w;
            if (key < kKC32) {
                ks[key][lc4] = kreg[w];
                vs[key][lc4] = vreg[w];
            }
        }
        __syncthreads();
        if (c + 1 < nch) fetch(c + 1);
        // lane: key c * 64 + lane against rows RPW wave + r
        float sc[RPW];
#pragma unroll
        for (int r = 0; r < RPW; ++r) sc[r] = 0.f;
#pragma unroll 4
        for (int c4 = 0; c4 < C4; ++c4) {
            const f32x4 kv = ks[lane][c4];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const f32x4 qv = qs[RPW * wave + r][c4];
                sc[r] = fmaf(qv[0], kv[0], sc[r]);
                sc[r] = fmaf(qv[1], kv[1], sc[r]);
                sc[r] = fmaf(qv[2], kv[2], sc[r]);
                sc[r] = fmaf(qv[3], kv[3], sc[r]);
            }
        }
        const bool valid = c * kKC32 + lane < total;
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const float x = valid ? sc[r] * a.scale : -INFINITY;
            const float cm = wave_max(x);
            if (cm > ref[r] + kSlack32) {  // wave-uniform; always on the first chunk
                const float f = expf(ref[r] - cm);
                l[r] *= f;
                acc[r] *= f;
                ref[r] = cm;
            }
            const float pv = valid ? expf(x - ref[r]) : 0.f;
            ps[RPW * wave + r][lane] = pv;
            l[r] += pv;
        }
        wave_lds_sync();  // this wave's weights are in LDS
#pragma unroll 4
        for (int st = 0; st < C4; ++st) {
            const int k = kq + KQ * st;
            const f32x4 v = vs[k][pc4];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const float pv = ps[RPW * wave + r][k];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[r][e] = fmaf(pv, v[e], acc[r][e]);
            }
        }
    }
    // sum the key subsets (lanes pc4 + C4 q) and the lanes' weight sums
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
        for (int o = C4; o < 64; o <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r][e] += __shfl_xor(acc[r][e], o);
        l[r] = wave_sum(l[r]);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const int jr = rb * kQR32 + RPW * wave + r;
        if (jr >= nrows) break;  // wave-uniform
        const size_t qi = q_index(jr);
        const int col = 4 * pc4;
        if (kq == 0 && col < D) {
            const f32x4 o = acc[r] * (1.f / l[r]);
            float* orow = a.out + qi * D;
            if (vec) {
                *reinterpret_cast<f32x4*>(orow + col) = o;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (col + e < D) orow[col + e] = o[e];
            }
        }
        if (a.lse && lane == 0) a.lse[qi] = ref[r] + logf(l[r]);
    }
}

// --------------------------------------------------------------- planning
struct AttnPlan {
    int n_qt, nct, n_qgroups, n_splits;
    size_t off_o, off_ml, bytes;
};

AttnPlan plan_attn(int batch, int gamma, int n_q, int n_kv, int d_head, int window, int dtype) {
    AttnPlan p{};
    const int group = n_q / n_kv;
    const int nrows = group * gamma;
    p.n_qt = (nrows + 15) / 16;
    p.n_qgroups = (p.n_qt + kMaxNCT - 1) / kMaxNCT;
    p.nct = (p.n_qt + p.n_qgroups - 1) / p.n_qgroups;
    if (dtype != DFLASH_DTYPE_BF16) {
        p.n_splits = 1;
        p.bytes = 0;
        return p;
    }
    // split the keys only as far as needed to give every CU a workgroup
    const int wg_lds = kWaves * 2 * 2 * TK * d_head * 2;
    const long per_cu = kLdsPerCU / wg_lds;
    const long units = (long)batch * n_kv * p.n_qgroups;
    const long want = (long)kCUs * per_cu;
    int splits = (int)((want + units - 1) / units);
    const int max_splits = (window + gamma + kMinKeysPerSplit - 1) / kMinKeysPerSplit;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    p.n_splits = splits;
    Carve c;
    if (splits > 1) {
        const size_t rows = (size_t)batch * n_kv * splits * p.n_qt * 16;
        p.off_o = c.take<float>(rows * d_head);
        p.off_ml = c.take<float>(rows * 2);
    }
    p.bytes = c.total();
    return p;
}

template <int D, int NCT>
void launch_bf16(const AttnArgs& a, int n_qgroups, hipStream_t st) {
    dim3 grid(a.n_splits, a.B * a.HKV, n_qgroups);
    hipLaunchKernelGGL((block_attn_bf16_kernel<D, NCT>), grid, dim3(64 * kWaves), 0, st, a);
}

template <int D>
void launch_bf16_nct(const AttnArgs& a, int nct, int n_qgroups, hipStream_t st) {
    switch (nct) {
        case 1: launch_bf16<D, 1>(a, n_qgroups, st); break;
        case 2: launch_bf16<D, 2>(a, n_qgroups, st); break;
        default: launch_bf16<D, 3>(a, n_qgroups, st); break;
    }
}

}  // namespace
}  // namespace dfl

using namespace dfl;

namespace dfl {
namespace {

// Shape part of the checks: DFLASH_ERR_SHAPE, DFLASH_ERR_UNSUPPORTED or OK.
// The caps keep every count the host forms (query rows, window + gamma, grid
// extents) far inside 32 bits.
int attn_shape(int batch, int gamma, int n_q, int n_kv, int d_head, int window, int dtype) {
    if (batch < 0 || gamma < 1 || n_q < 1 || n_kv < 1 || d_head < 1 || window < 1)
        return DFLASH_ERR_SHAPE;
    if (n_q % n_kv != 0) return DFLASH_ERR_SHAPE;
    if (dtype != DFLASH_DTYPE_BF16 && dtype != DFLASH_DTYPE_FP32) return DFLASH_ERR_SHAPE;
    if (gamma > 32 || window % 64 != 0 || window > kMaxWindow ||
        capped_product(kMaxQueryRows, {batch, gamma, n_q}) < 0)
        return DFLASH_ERR_UNSUPPORTED;
    if (dtype == DFLASH_DTYPE_BF16 && d_head != 64 && d_head != 128) return DFLASH_ERR_UNSUPPORTED;
    if (dtype == DFLASH_DTYPE_FP32 && d_head > 128)
        return DFLASH_ERR_UNSUPPORTED;
    return DFLASH_OK;
}

}  // namespace
}  // namespace dfl

extern "C" size_t dflash_block_attn_workspace_size(int batch, int gamma, int n_q, int n_kv,
                                                   int d_head, int window, int dtype) {
    if (batch == 0 || attn_shape(batch, gamma, n_q, n_kv, d_head, window, dtype) != DFLASH_OK)
        return 0;
    return plan_attn(batch, gamma, n_q, n_kv, d_head, window, dtype).bytes;
}

extern "C" int dflash_block_attn(const void* q, const void* k_blk, const void* v_blk,
                                 const void* k_ring, const void* v_ring, const int64_t* ctx_len,
                                 float scale, void* out, float* lse, int dtype, int batch,
                                 int gamma, int n_q, int n_kv, int d_head, int window,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    const int shape = attn_shape(batch, gamma, n_q, n_kv, d_head, window, dtype);
    if (shape == DFLASH_ERR_SHAPE || !(scale > 0.f) || !std::isfinite(scale)) return DFLASH_ERR_SHAPE;
    if (batch == 0) return DFLASH_OK;
    if (!q || !k_blk || !v_blk || !k_ring || !v_ring || !ctx_len || !out) return DFLASH_ERR_NULL;
    if (shape != DFLASH_OK) return shape;
    const AttnPlan p = plan_attn(batch, gamma, n_q, n_kv, d_head, window, dtype);
    if (p.bytes > 0) {
        if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) || workspace_bytes < p.bytes)
            return DFLASH_ERR_WORKSPACE;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == DFLASH_DTYPE_FP32) {
        auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
        const int vec = d_head % 4 == 0 && al16(q) && al16(k_blk) && al16(v_blk) && al16(k_ring) &&
                        al16(v_ring) && al16(out);
        Attn32Args a{static_cast<const float*>(q), static_cast<const float*>(k_blk),
                     static_cast<const float*>(v_blk), static_cast<const float*>(k_ring),
                     static_cast<const float*>(v_ring), ctx_len, scale,
                     static_cast<float*>(out), lse, batch, gamma, n_q, n_kv, window, d_head, vec};
        // one workgroup per (sequence, KV head, block of 16 of its gamma * n_q / n_kv query rows)
        const int64_t nrb = ((int64_t)gamma * (n_q / n_kv) + kQR32 - 1) / kQR32;
        const dim3 grid((unsigned)((int64_t)batch * n_kv * nrb)), block(kThreads32);
        const int c4 = (d_head + 3) / 4;
        if (c4 <= 1) hipLaunchKernelGGL(block_attn_f32_kernel<1>, grid, block, 0, st, a);
        else if (c4 <= 2) hipLaunchKernelGGL(block_attn_f32_kernel<2>, grid, block, 0, st, a);
        else if (c4 <= 4) hipLaunchKernelGGL(block_attn_f32_kernel<4>, grid, block, 0, st, a);
        else if (c4 <= 8) hipLaunchKernelGGL(block_attn_f32_kernel<8>, grid, block, 0, st, a);
        else if (c4 <= 16) hipLaunchKernelGGL(block_attn_f32_kernel<16>, grid, block, 0, st, a);
        else hipLaunchKernelGGL(block_attn_f32_kernel<32>, grid, block, 0, st, a);
        return launch_status();
    }
    AttnArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.kb = static_cast<const uint16_t*>(k_blk);
    a.vb = static_cast<const uint16_t*>(v_blk);
    a.kr = static_cast<const uint16_t*>(k_ring);
    a.vr = static_cast<const uint16_t*>(v_ring);
    a.ctx_len = ctx_len;
    a.scale_log2 = scale * kLog2e;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    char* ws = static_cast<char*>(workspace);
    a.part_o = p.n_splits > 1 ? reinterpret_cast<float*>(ws + p.off_o) : nullptr;
    a.part_ml = p.n_splits > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
    a.B = batch; a.G = gamma; a.HQ = n_q; a.HKV = n_kv; a.W = window;
    a.group = n_q / n_kv;
    a.nrows = a.group * gamma;
    a.n_qt = p.n_qt;
    a.n_splits = p.n_splits;
    if (d_head == 128) launch_bf16_nct<128>(a, p.nct, p.n_qgroups, st);
    else launch_bf16_nct<64>(a, p.nct, p.n_qgroups, st);
    int rc = launch_status();
    if (rc != DFLASH_OK || p.n_splits == 1) return rc;
    dim3 grid(batch * n_kv, p.n_qt);
    if (d_head == 128) hipLaunchKernelGGL(attn_combine_kernel<128>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, st, a);
    return launch_status();
}
