// block_attn.hip -- block-draft attention for gfx950.
//
// "DFlash vs DFlash 2", "DFlash: generate the block all at once" and
// "Conditioning on the target model" (Q_i, K_i, V_i equation): the block's
// queries attend without a causal mask to the context window and to the
// block's own keys.  "Beam 1.0 DFlash2", "Model": 40 query heads share 8 KV
// heads of dimension 128; the window holds the last 4,096 context tokens.
//
// bf16 path.  One workgroup (4 waves) owns one (sequence, KV head, key split,
// query-tile group).  The key sequence of a (sequence, KV head) is virtual:
// index t < n_b reads ring slot t, t >= n_b reads block row t - n_b, so the
// block keys are streamed like the window keys.  Every query row of the GQA
// group (group * gamma rows, padded to 16) is a column of one MFMA tile, so
// each K/V byte is fetched once and used by all query heads of its group.
//
// Per 32-key tile a wave
//   1. has the tile's K rows in registers, already in the A-operand layout of
//      v_mfma_f32_16x16x32_bf16 (each lane reads 64 contiguous bytes of rows),
//      and the tile's V rows in registers (4 tokens x 8 dims per lane);
//   2. issues the loads of its next tile (register double buffer);
//   3. writes V transposed into its private LDS tile (8-byte stores);
//   4. computes S^T = K Q^T (keys x query rows) with MFMA, fp32;
//   5. runs the online softmax in base 2 (column max across the 4 lane
//      groups, rescale of the running sum and of O^T);
//   6. packs P^T to bf16 straight from the S^T accumulator layout and
//      accumulates O^T += V^T P^T with MFMA, reading V^T from LDS.
// The four waves of a workgroup take interleaved tiles and are merged
// through LDS at the end; key splits are merged by a second kernel.
//
// fp32 path (small shapes): one wave per query, scores in LDS, exact expf.
#include <cmath>

#include "common.hpp"

namespace dfl {
namespace {

constexpr int TK = 64;             // keys per tile
constexpr int kStages = 4;         // LDS ring depth (tiles)
constexpr int kMaxNC = 8;          // consumer waves (16-row query tiles) per workgroup
constexpr int kCUs = 256;          // MI355X compute units
constexpr int kWGsPerCU = 1;       // resident attention workgroups per CU (LDS-limited)
constexpr int kMinTilesPerSplit = 2;
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
    int B, G, HQ, HKV, W, group, nrows, n_qt, n_splits, nw;
};

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define DFL_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define DFL_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    // s_waitcnt encoding on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Block-draft attention, bf16.
//
// Workgroup = NC consumer waves + 2 producer waves.  Consumer wave w owns
// query tile blockIdx.z * NC + w (16 rows of the GQA group: (block row, head)
// pairs) for every key of the workgroup's split.  The two producer waves
// stream the split's keys in 64-key tiles straight from HBM into a
// kStages-deep LDS ring with global_load_lds_dwordx4 (no registers, no LDS
// store instructions): the K producer places each 16-byte chunk c of key row
// r at chunk c ^ (r % 16) (conflict-free ds_read_b128 of the S^T = K Q^T
// operand), the V producer places each 32-byte double chunk d of row r at
// d ^ (r % 8), which ds_read_b64_tr_b16 turns into the keys-by-dims operand of
// O^T += V^T P^T.  Every K/V byte is read from HBM once per (sequence, KV head)
// and used by all query heads of the group.
template <int D, int NC>
__global__ void __launch_bounds__(64 * (NC + 2)) block_attn_bf16_kernel(AttnArgs a) {
    constexpr int ROWB = D * 2;               // bytes per key row
    constexpr int CHR = ROWB / 16;            // 16-byte chunks per row
    constexpr int TILEB = TK * ROWB;          // bytes of one K (or V) tile
    constexpr int NI = TILEB / 1024;          // 1 KB load instructions per K (or V) tile
    constexpr int RPI = 1024 / ROWB;          // rows per load instruction
    constexpr int DT = D / 16;                // 16-dim tiles of O^T
    constexpr int KS = D / 32;                // k-steps of S^T
    __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages][2][TILEB];

    const int split = blockIdx.x;
    const int bk = blockIdx.y;
    const int b = bk / a.HKV, kvh = bk % a.HKV;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, i16 = lane & 15;

    const int64_t cl = a.ctx_len[b];
    const int n = (int)(cl < (int64_t)a.W ? (cl < 0 ? 0 : cl) : (int64_t)a.W);
    const int total = n + a.G;
    int per = (total + a.n_splits - 1) / a.n_splits;
    per = (per + TK - 1) / TK * TK;
    const int t0 = split * per;
    const int t1 = min(t0 + per, total);
    const int ntiles = t1 > t0 ? (t1 - t0 + TK - 1) / TK : 0;

    if (wave >= NC) {
        // ------------------------------------------------------ producers
        const int kv = wave - NC;  // 0: K, 1: V
        const uint16_t* ring = (kv == 0 ? a.kr : a.vr) + (size_t)bk * a.W * D;
        const uint16_t* blk = (kv == 0 ? a.kb : a.vb) + ((size_t)b * a.G * a.HKV + kvh) * D;
        const size_t blk_stride = (size_t)a.HKV * D;
        const int rl = lane / CHR, p = lane % CHR;  // row within an instruction, physical chunk
        auto issue = [&](int tile) {
            const int tb = t0 + tile * TK;
            unsigned char* dst = smem[tile % kStages][kv];
#pragma unroll
            for (int ins = 0; ins < NI; ++ins) {
                const int r = ins * RPI + rl;
                int t = tb + r;
                if (t >= t1) t = t1 - 1;  // masked key: any valid row
                int c;
                if (kv == 0) c = p ^ (r % CHR);
                else c = ((((p >> 1) ^ (r % (CHR / 2)))) << 1) | (p & 1);
                const uint16_t* row = t < n ? ring + (size_t)t * D : blk + (size_t)(t - n) * blk_stride;
                __builtin_amdgcn_global_load_lds(DFL_GLOBAL(row + c * 8), DFL_LDS(dst + ins * 1024),
                                                 16, 0, 0);
            }
        };
        const int pre = ntiles < kStages - 1 ? ntiles : kStages - 1;
        for (int i = 0; i < pre; ++i) issue(i);
        for (int i = 0; i < ntiles; ++i) {
            const int ahead = min(kStages - 2, ntiles - 1 - i);  // tiles issued beyond tile i
            if (ahead >= 2) wait_vmem<2 * NI>();
            else if (ahead == 1) wait_vmem<NI>();
            else wait_vmem<0>();
            // tile i is in LDS; a bare barrier (a release fence here would also
            // wait for the tiles still in flight)
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (i + kStages - 1 < ntiles) issue(i + kStages - 1);
        }
        return;
    }

    // ---------------------------------------------------------- consumers
    const int qt = blockIdx.z * NC + wave;
    u32x4 qreg[KS];
    {
        const int j = qt * 16 + i16;
        const bool ok = qt < a.n_qt && j < a.nrows;
        const int r = ok ? j / a.group : 0, hl = ok ? j % a.group : 0;
        const uint16_t* qrow = a.q + ((size_t)((size_t)b * a.G + r) * a.HQ + kvh * a.group + hl) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qreg[s] = ok ? *reinterpret_cast<const u32x4*>(qrow + s * 32 + g * 8) : z;
        }
    }

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running reference max of this lane's query column (base 2)
    float l_run = 0.f;        // this lane's share of sum 2^(x - m_run)

    for (int i = 0; i < ntiles; ++i) {
        __syncthreads();
        const int tb = t0 + i * TK;
        const unsigned char* kt = smem[i % kStages][0];
        const unsigned char* vt = smem[i % kStages][1];

        // S^T = K Q^T for 4 subtiles of 16 keys
        f32x4 sacc[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int r = st * 16 + i16;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 kvv = *reinterpret_cast<const u32x4*>(
                    kt + r * ROWB + (((s * 4 + g) ^ (r % CHR)) * 16));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kvv),
                                                              __builtin_bit_cast(bf16x8, qreg[s]),
                                                              acc, 0, 0, 0);
            }
            sacc[st] = acc;
        }
        // online softmax with a lazily raised reference max
        float x[16];
        const bool tail = tb + TK > t1;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = sacc[st][e] * a.scale_log2;
                x[st * 4 + e] = (tail && tb + st * 16 + g * 4 + e >= t1) ? -INFINITY : v;
            }
        float tmax = x[0];
#pragma unroll
        for (int k = 1; k < 16; ++k) tmax = fmaxf(tmax, x[k]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        if (__ballot(tmax > m_run + kRescaleSlack)) {
            const float mnew = fmaxf(m_run, tmax);
            const float alpha = fast_exp2(m_run - mnew);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
            m_run = mnew;
        }
        float psum = 0.f;
        bf16x8 pb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pv[e] = fast_exp2(x[(2 * ks) * 4 + e] - m_run);
                pv[4 + e] = fast_exp2(x[(2 * ks + 1) * 4 + e] - m_run);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) psum += pv[e];
            u32x4 pk;
            pk[0] = pack_bf16x2(pv[0], pv[1]);
            pk[1] = pack_bf16x2(pv[2], pv[3]);
            pk[2] = pack_bf16x2(pv[4], pv[5]);
            pk[3] = pack_bf16x2(pv[6], pv[7]);
            pb[ks] = __builtin_bit_cast(bf16x8, pk);
        }
        l_run += psum;
        // O^T += V^T P^T: the A operand (16 dims x 8 keys per lane) comes from two
        // transposing reads, keys 32ks+4g+{0..3} and 32ks+16+4g+{0..3}
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                v4i16 h[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int r = ks * 32 + hh * 16 + g * 4 + (i16 >> 2);
                    const unsigned char* src =
                        vt + r * ROWB + ((dt ^ (r % (CHR / 2))) * 32) + (i16 & 3) * 8;
                    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16*)(DFL_LDS(src)));
                }
                u32x4 av;
                av[0] = __builtin_bit_cast(u32x2, h[0])[0];
                av[1] = __builtin_bit_cast(u32x2, h[0])[1];
                av[2] = __builtin_bit_cast(u32x2, h[1])[0];
                av[3] = __builtin_bit_cast(u32x2, h[1])[1];
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                pb[ks], o[dt], 0, 0, 0);
            }
        }
    }
    // the last tile's buffer is not reused, so no trailing barrier is needed

    // the 4 lane groups of a column hold disjoint keys: column sum
    l_run += __shfl_xor(l_run, 16, kWave);
    l_run += __shfl_xor(l_run, 32, kWave);

    const int j = qt * 16 + i16;
    if (qt >= a.n_qt || j >= a.nrows) return;
    if (a.n_splits == 1) {
        const int r = j / a.group, h = kvh * a.group + j % a.group;
        const size_t row = ((size_t)b * a.G + r) * a.HQ + h;
        const float inv = 1.f / l_run;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            u32x2 w2;
            w2[0] = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
            w2[1] = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
            *reinterpret_cast<u32x2*>(a.out + row * D + dt * 16 + g * 4) = w2;
        }
        if (a.lse && g == 0) a.lse[row] = (m_run + __log2f(l_run)) * (float)kLn2;
    } else {
        const size_t prow = ((size_t)bk * a.n_splits + split) * (a.n_qt * 16) + j;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<f32x4*>(a.part_o + prow * D + dt * 16 + g * 4) = o[dt];
        if (g == 0) {
            a.part_ml[prow * 2 + 0] = m_run;
            a.part_ml[prow * 2 + 1] = l_run;
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
};

constexpr int kMaxKeys32 = 4096 + 32;
constexpr int kWaves32 = 4;

__global__ void __launch_bounds__(256) block_attn_f32_kernel(Attn32Args a) {
    __shared__ float sc[kWaves32][kMaxKeys32];
    __shared__ float qs[kWaves32][128];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int qi = blockIdx.x * kWaves32 + wave;  // (b, r, h) flattened
    if (qi >= a.B * a.G * a.HQ) return;
    const int h = qi % a.HQ, b = qi / (a.HQ * a.G);
    const int kvh = h / (a.HQ / a.HKV);
    const int64_t cl = a.ctx_len[b];
    const int n = (int)(cl < (int64_t)a.W ? (cl < 0 ? 0 : cl) : (int64_t)a.W);
    const int total = n + a.G;
    const int D = a.D;
    const float* qrow = a.q + (size_t)qi * D;
    for (int d = lane; d < D; d += kWave) qs[wave][d] = qrow[d];
    __builtin_amdgcn_wave_barrier();
    float mx = -INFINITY;
    for (int t = lane; t < total; t += kWave) {
        const float* krow = t < n ? a.kr + ((size_t)((size_t)b * a.HKV + kvh) * a.W + t) * D
                                  : a.kb + ((size_t)((size_t)b * a.G + (t - n)) * a.HKV + kvh) * D;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(qs[wave][d], krow[d], s);
        s *= a.scale;
        sc[wave][t] = s;
        mx = fmaxf(mx, s);
    }
    mx = wave_max(mx);
    float sum = 0.f;
    for (int t = lane; t < total; t += kWave) {
        const float p = expf(sc[wave][t] - mx);
        sc[wave][t] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    wave_lds_sync();
    const float inv = 1.f / sum;
    for (int d = lane; d < D; d += kWave) {
        float acc = 0.f;
        for (int t = 0; t < total; ++t) {
            const float* vrow = t < n ? a.vr + ((size_t)((size_t)b * a.HKV + kvh) * a.W + t) * D
                                      : a.vb + ((size_t)((size_t)b * a.G + (t - n)) * a.HKV + kvh) * D;
            acc = fmaf(sc[wave][t], vrow[d], acc);
        }
        a.out[(size_t)qi * D + d] = acc * inv;
    }
    if (a.lse && lane == 0) a.lse[qi] = mx + logf(sum);
}

// --------------------------------------------------------------- planning
struct AttnPlan {
    int n_qt, nw, n_qgroups, n_splits;
    size_t off_o, off_ml, bytes;
};

AttnPlan plan_attn(int batch, int gamma, int n_q, int n_kv, int d_head, int window, int dtype) {
    AttnPlan p{};
    const int group = n_q / n_kv;
    const int nrows = group * gamma;
    p.n_qt = (nrows + 15) / 16;
    p.n_qgroups = (p.n_qt + kMaxNC - 1) / kMaxNC;
    p.nw = (p.n_qt + p.n_qgroups - 1) / p.n_qgroups;
    if (dtype != DFLASH_DTYPE_BF16) {
        p.n_splits = 1;
        p.bytes = 0;
        return p;
    }
    const long units = (long)batch * n_kv * p.n_qgroups;
    const long want = (long)kCUs * kWGsPerCU;
    int splits = (int)((want + units - 1) / units);
    const int max_splits = (window + gamma + TK * kMinTilesPerSplit - 1) / (TK * kMinTilesPerSplit);
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

template <int D, int NC>
void launch_bf16(const AttnArgs& a, int n_qgroups, hipStream_t st) {
    dim3 grid(a.n_splits, a.B * a.HKV, n_qgroups);
    hipLaunchKernelGGL((block_attn_bf16_kernel<D, NC>), grid, dim3(64 * (NC + 2)), 0, st, a);
}

template <int D>
void launch_bf16_nw(const AttnArgs& a, int nw, int n_qgroups, hipStream_t st) {
    switch (nw) {
        case 1: launch_bf16<D, 1>(a, n_qgroups, st); break;
        case 2: launch_bf16<D, 2>(a, n_qgroups, st); break;
        case 3: launch_bf16<D, 3>(a, n_qgroups, st); break;
        case 4: launch_bf16<D, 4>(a, n_qgroups, st); break;
        case 5: launch_bf16<D, 5>(a, n_qgroups, st); break;
        case 6: launch_bf16<D, 6>(a, n_qgroups, st); break;
        case 7: launch_bf16<D, 7>(a, n_qgroups, st); break;
        default: launch_bf16<D, 8>(a, n_qgroups, st); break;
    }
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" size_t dflash_block_attn_workspace_size(int batch, int gamma, int n_q, int n_kv,
                                                   int d_head, int window, int dtype) {
    if (batch < 0 || gamma < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv || window < 1) return 0;
    return plan_attn(batch, gamma, n_q, n_kv, d_head, window, dtype).bytes;
}

extern "C" int dflash_block_attn(const void* q, const void* k_blk, const void* v_blk,
                                 const void* k_ring, const void* v_ring, const int64_t* ctx_len,
                                 float scale, void* out, float* lse, int dtype, int batch,
                                 int gamma, int n_q, int n_kv, int d_head, int window,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    if (batch < 0 || gamma < 1 || n_q < 1 || n_kv < 1 || d_head < 1 || window < 1)
        return DFLASH_ERR_SHAPE;
    if (n_q % n_kv != 0 || !(scale > 0.f) || !std::isfinite(scale)) return DFLASH_ERR_SHAPE;
    if (dtype != DFLASH_DTYPE_BF16 && dtype != DFLASH_DTYPE_FP32) return DFLASH_ERR_SHAPE;
    if (batch == 0) return DFLASH_OK;
    if (!q || !k_blk || !v_blk || !k_ring || !v_ring || !ctx_len || !out) return DFLASH_ERR_NULL;
    if (gamma > 32 || window % 64 != 0) return DFLASH_ERR_UNSUPPORTED;
    if (dtype == DFLASH_DTYPE_BF16 && d_head != 64 && d_head != 128) return DFLASH_ERR_UNSUPPORTED;
    if (dtype == DFLASH_DTYPE_FP32 && (d_head > 128 || window + gamma > kMaxKeys32))
        return DFLASH_ERR_UNSUPPORTED;
    const AttnPlan p = plan_attn(batch, gamma, n_q, n_kv, d_head, window, dtype);
    if (p.bytes > 0) {
        if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) || workspace_bytes < p.bytes)
            return DFLASH_ERR_WORKSPACE;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dtype == DFLASH_DTYPE_FP32) {
        Attn32Args a{static_cast<const float*>(q), static_cast<const float*>(k_blk),
                     static_cast<const float*>(v_blk), static_cast<const float*>(k_ring),
                     static_cast<const float*>(v_ring), ctx_len, scale,
                     static_cast<float*>(out), lse, batch, gamma, n_q, n_kv, window, d_head};
        const int nq = batch * gamma * n_q;
        hipLaunchKernelGGL(block_attn_f32_kernel, dim3((nq + kWaves32 - 1) / kWaves32),
                           dim3(64 * kWaves32), 0, st, a);
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
    a.nw = p.nw;
    if (d_head == 128) launch_bf16_nw<128>(a, p.nw, p.n_qgroups, st);
    else launch_bf16_nw<64>(a, p.nw, p.n_qgroups, st);
    int rc = launch_status();
    if (rc != DFLASH_OK || p.n_splits == 1) return rc;
    dim3 grid(batch * n_kv, p.n_qt);
    if (d_head == 128) hipLaunchKernelGGL(attn_combine_kernel<128>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(attn_combine_kernel<64>, grid, dim3(256), 0, st, a);
    return launch_status();
}
