// context_fuse.hip -- context fusion and context K/V append, for gfx950.
//
// "DFlash vs DFlash 2", "Conditioning on the target model", equation for H_t:
// the tapped target states of each new token are concatenated, projected by
// W_c and RMS-normalised; equation for K_i, V_i: the context half of every
// draft layer's keys and values is W_i^K H_t, W_i^V H_t.
//
//   1. gemm  : P1[s] = X[:, Ks] W_c[:, Ks]^T      (bf16 MFMA, fp32 partials)
//   2. norm  : H_t = RMSNorm(sum_s P1[s]) * g   -> bf16
//   3. gemm  : P2[s] = H_t[:, Ks] W_kv[:, Ks]^T
//   4. append: kv_ring[slot(row)] = bf16(sum_s P2[s])
//
// The GEMM is "NT": both operands are K-contiguous (weights stored one row
// per output feature), so global loads and the MFMA operand layout agree.
// Workgroup tile 256 x 160, K-tile 64, eight waves of 64 x 80 built from
// v_mfma_f32_16x16x32_bf16, fed by three producer waves through a 3-stage LDS
// ring (XOR swizzle of the 16-byte chunks of each 128-byte row, so the
// ds_read_b128 operand fetches are conflict-free); split-K across workgroups
// to fill the 256 CUs when M is only a few hundred rows.
#include <cmath>

#include "common.hpp"

namespace dfl {
DFL_VIOLATION_WORD(violations_fuse)
namespace {

constexpr int BM = 256, BN = 160, BK = 64;   // workgroup tile and K stage
constexpr int WN = BN / 2 / 16;              // 16-column MFMA tiles per consumer wave
constexpr int kGStages = 3;                  // LDS ring depth (2 stages in flight)
constexpr int kGConsumers = 8;               // 4 x 2 waves of 64 x 80, two per SIMD
constexpr int kGProducers = 3;               // A rows 0-127, A rows 128-255, B rows
constexpr int kCUs = 256;
constexpr int kXCDs = 8;
constexpr int64_t kMaxFuseWidth = 1 << 30;  // n_taps * d_tgt and n_layers * 2 * n_kv * d_head
constexpr int kMaxFuseRows = 65535;        // the K/V append spans the rows in its grid's y extent

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define DFL_LDS(p) ((__attribute__((address_space(3))) void*)(p))
#define DFL_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))

template <int N>
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

struct GemmArgs {
    const uint16_t* A;  // [M, K], or in K slabs [K / 64][M][64] (A_SLABS)
    const uint16_t* B;  // [N, K]
    float* C;           // [S, M, N]
    int M, N, K, S, n_mt, n_nt;
};

// Split-K "NT" GEMM, C[s] = A[:, Ks] B[:, Ks]^T, bf16 in, fp32 partials.
// Three producer waves stream 64-wide K stages of the 256 x 160 workgroup tile
// straight into a kGStages-deep LDS ring with global_load_lds_dwordx4 (each
// 16-byte chunk c of a 128-byte row r placed at chunk c ^ (r % 8)); eight
// consumer waves (two per SIMD, so one's MFMAs cover the other's LDS waits)
// each accumulate a 64 x 80 block with 16 x 16 x 32 MFMAs.
//
// Tile order: workgroup L runs on XCD L % 8.  The split count S divides 8 and
// split s is computed only on the XCDs x with x % S == s, so each XCD's L2
// holds a single K slice of A (re-read by every column block of that XCD),
// and the M tiles of one column block run on one XCD, sharing its B slice.
template <bool A_SLABS>
__global__ void __launch_bounds__(64 * (kGConsumers + kGProducers)) gemm_nt_bf16_kernel(GemmArgs g) {
    constexpr int ROWB = BK * 2;  // 128 bytes per tile row and stage
    constexpr int NIB = BN / 8;   // 1 KB load instructions per B stage
    __shared__ __attribute__((aligned(1024))) unsigned char sa[kGStages][BM * ROWB];
    __shared__ __attribute__((aligned(1024))) unsigned char sb[kGStages][BN * ROWB];

    const int L = blockIdx.x;
    const int xcd = L % kXCDs, q = L / kXCDs;
    const int mt = q % g.n_mt, r8 = q / g.n_mt;
    const int split = xcd % g.S;
    const int nt = r8 * (kXCDs / g.S) + xcd / g.S;
    if (nt >= g.n_nt) return;
    const int m0 = mt * BM, n0 = nt * BN;
    const int ktiles = g.K / BK;
    const int kt0 = (int)((long)split * ktiles / g.S), kt1 = (int)((long)(split + 1) * ktiles / g.S);
    const int nst = kt1 - kt0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    if (wave >= kGConsumers) {
        const int pw = wave - kGConsumers;  // 0, 1: A halves; 2: B
        const int rl = lane >> 3, p = lane & 7;  // row within an instruction, physical chunk
        auto issue = [&](int st) {
            const int k0 = (kt0 + st) * BK;
            if (pw < 2) {
                // activations: re-read by every column block, keep them cached
                unsigned char* dst = sa[st % kGStages] + pw * 128 * ROWB;
#pragma unroll
                for (int ins = 0; ins < 16; ++ins) {
                    const int r = ins * 8 + rl;  // row within this producer's 128
                    const int c = p ^ (r % 8);
                    int m = m0 + pw * 128 + r;
                    if (m >= g.M) m = g.M - 1;  // rows beyond M: any valid row, never stored
                    // in K slabs, a stage's 256 rows are one contiguous 32 KB block
                    const uint16_t* src = A_SLABS ? g.A + ((size_t)(k0 / BK) * g.M + m) * BK + c * 8
                                                  : g.A + (size_t)m * g.K + k0 + c * 8;
                    __builtin_amdgcn_global_load_lds(DFL_GLOBAL(src), DFL_LDS(dst + ins * 1024), 16, 0,
                                                     kLoadDefault);
                }
            } else {
                // weights: streamed once, non-temporal so they do not evict the A slice
                unsigned char* dst = sb[st % kGStages];
#pragma unroll
                for (int ins = 0; ins < NIB; ++ins) {
                    const int r = ins * 8 + rl;
                    const int c = p ^ (r % 8);
                    int n = n0 + r;
                    if (n >= g.N) n = g.N - 1;  // columns beyond N: any valid row, never stored
                    const uint16_t* src = g.B + (size_t)n * g.K + k0 + c * 8;
                    __builtin_amdgcn_global_load_lds(DFL_GLOBAL(src), DFL_LDS(dst + ins * 1024), 16, 0,
                                                     kLoadStream);
                }
            }
        };
        const int pre = nst < kGStages - 1 ? nst : kGStages - 1;
        for (int i = 0; i < pre; ++i) issue(i);
        for (int i = 0; i < nst; ++i) {
            const int ahead = min(kGStages - 2, nst - 1 - i);
            if (ahead >= 1) {
                if (pw < 2) wait_vmem<16>();
                else wait_vmem<NIB>();
            } else {
                wait_vmem<0>();
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (i + kGStages - 1 < nst) issue(i + kGStages - 1);
        }
        return;
    }

    const int wm = wave >> 1, wn = wave & 1;
    const int i16 = lane & 15, grp = lane >> 4;
    f32x4 acc[4][WN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int i = 0; i < nst; ++i) {
        __syncthreads();
        const unsigned char* A = sa[i % kGStages];
        const unsigned char* Bt = sb[i % kGStages];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = s * 4 + grp;
            bf16x8 fa[4], fb[WN];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int ra = wm * 64 + t * 16 + i16;
                fa[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(A + ra * ROWB + ((c ^ (ra % 8)) * 16)));
            }
#pragma unroll
            for (int t = 0; t < WN; ++t) {
                const int rb = wn * (WN * 16) + t * 16 + i16;
                fb[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bt + rb * ROWB + ((c ^ (rb % 8)) * 16)));
            }
            // the wave issuing MFMAs goes first on its SIMD (measured: 121 -> 117 us at 512 rows)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti)
#pragma unroll
                for (int tj = 0; tj < WN; ++tj)
                    acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ti], fb[tj], acc[ti][tj], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
        }
    }
    // acc[i][j]: rows m0 + wm*64 + i*16 + 4*grp + e, column n0 + wn*80 + j*16 + i16
    float* C = g.C + (size_t)split * g.M * g.N;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = m0 + wm * 64 + ti * 16 + 4 * grp + e;
            if (m >= g.M) continue;
#pragma unroll
            for (int tj = 0; tj < WN; ++tj) {
                const int n = n0 + wn * (WN * 16) + tj * 16 + i16;
                if (n < g.N) C[(size_t)m * g.N + n] = acc[ti][tj][e];
            }
        }
}


// H_t row r = RMSNorm(sum_s P[s][r]) * g, one 1,024-thread workgroup per row.  The
// S split-K partials of a thread's (at most two) float4 columns are loaded together
// (S is a template argument, so every load is issued before the first add).
// H_t goes to the workspace in K slabs of 64 columns, [N / 64][M][64], the layout
// in which the K/V projection reads its activation tiles: each stage's 256 rows
// are one contiguous block instead of 256 pieces 2 N bytes apart (measured on
// the K/V GEMM at 256 x 5,120 -> 10,240: 43 -> 38 us); h_out, if given, gets
// the row-major copy.
constexpr int kNormThreads = 1024;
constexpr int kNormChunks = 2;  // float4 columns per thread: d_model <= 8192
template <int S>
__global__ void __launch_bounds__(kNormThreads) rmsnorm_kernel(const float* P, int M, int N,
                                                             const float* gain, float eps,
                                                             uint16_t* H, uint16_t* h_out) {
    extern __shared__ f32x4 y4[];
    __shared__ float red[kNormThreads / 64];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int N4 = N / 4;
    f32x4 v[kNormChunks][S];
#pragma unroll
    for (int c = 0; c < kNormChunks; ++c) {
        const int n4 = tid + c * kNormThreads;
#pragma unroll
        for (int s = 0; s < S; ++s)
            v[c][s] = n4 < N4 ? *reinterpret_cast<const f32x4*>(P + ((size_t)s * M + r) * N + 4 * n4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < kNormChunks; ++c) {
        const int n4 = tid + c * kNormThreads;
        f32x4 y = v[c][0];
#pragma unroll
        for (int s = 1; s < S; ++s) y += v[c][s];
        if (n4 < N4) y4[n4] = y;
        ss += (y[0] * y[0] + y[1] * y[1]) + (y[2] * y[2] + y[3] * y[3]);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kNormThreads / 64; ++w) tot += red[w];
    const float inv = 1.f / sqrtf(tot / (float)N + eps);
#pragma unroll
    for (int c = 0; c < kNormChunks; ++c) {
        const int n4 = tid + c * kNormThreads;
        if (n4 >= N4) continue;
        const f32x4 y = y4[n4];
        const f32x4 gg = *reinterpret_cast<const f32x4*>(gain + 4 * n4);
        u32x2 w;
        w[0] = pack_bf16x2(y[0] * inv * gg[0], y[1] * inv * gg[1]);
        w[1] = pack_bf16x2(y[2] * inv * gg[2], y[3] * inv * gg[3]);
        *reinterpret_cast<u32x2*>(H + ((size_t)(n4 >> 4) * M + r) * 64 + 4 * (n4 & 15)) = w;
        if (h_out) *reinterpret_cast<u32x2*>(h_out + (size_t)r * N + 4 * n4) = w;
    }
}

template <int S>
__global__ void __launch_bounds__(256) kv_append_kernel(const float* P, int M, int NC,
                                                        const int32_t* row_seq,
                                                        const int64_t* row_pos, uint16_t* ring,
                                                        int B, int NKV, int DH, int W) {
    const int r = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= NC) return;
    f32x4 p[S];
#pragma unroll
    for (int s = 0; s < S; ++s) p[s] = *reinterpret_cast<const f32x4*>(P + ((size_t)s * M + r) * NC + c);
    f32x4 v = p[0];
#pragma unroll
    for (int s = 1; s < S; ++s) v += p[s];
    const int seq = row_seq[r];
    const int64_t pos = row_pos[r];
    if (seq < 0 || seq >= B || pos < 0) {  // violated precondition: row skipped
        if (DFLASH_DEVICE_CHECKS && c == 0) DFL_VIOLATION(DFLASH_VIOLATION_ROW);
        return;
    }
    const int64_t slot = pos % W;
    const int d = c % DH, h = (c / DH) % NKV, lt = c / (DH * NKV);  // lt = layer*2 + t
    const size_t at = ((((size_t)lt * B + seq) * NKV + h) * W + (size_t)slot) * DH + d;
    u32x2 w;
    w[0] = pack_bf16x2(v[0], v[1]);
    w[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(ring + at) = w;
}

#if DFLASH_DEVICE_CHECKS
// Rows of one call that address the same (sequence, slot): each row compares
// itself with every later row (builds with device checks only: rows^2 work).
__global__ void __launch_bounds__(256) fuse_slot_check_kernel(const int32_t* row_seq, const int64_t* row_pos,
                                                             int rows, int B, int W) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= rows) return;
    const int s = row_seq[r];
    const int64_t p = row_pos[r];
    if (s < 0 || s >= B || p < 0) return;  // recorded by the append
    const int64_t slot = p % W;
    bool dup = false;
    for (int q = r + 1; q < rows; ++q) {
        const int64_t p2 = row_pos[q];
        dup |= row_seq[q] == s && p2 >= 0 && p2 % W == slot;
    }
    if (dup) DFL_VIOLATION(DFLASH_VIOLATION_SLOT);
}
#endif

// Split-K count from a two-term time model: workgroup waves of one CU each
// times one workgroup's MFMA time, plus writing and re-reading the fp32
// partials at HBM speed (at most 16 splits).  (Rates are round planning figures for one MI355X
// CU and for HBM; only their ratio matters.)
// Split-K factor S in {1, 2, 4, 8} (so that splits map onto whole XCDs): the
// smallest modelled time, with each workgroup bounded by the slower of its
// MFMA work and its share of the weight stream, plus the fp32 partial sums
// written and read back once.
int pick_splits(int M, int N, int K) {
    const long tiles = (long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int kt = K / BK;
    const double cu_rate = 1.25e15 / kCUs;  // sustained bf16 MFMA flop/s of one CU
    const double hbm = 5.0e12;              // sustained HBM bytes/s
    int best = 1;
    double best_t = 1e30;
    for (int s = 1; s <= kXCDs && s <= kt; s *= 2) {
        const long wgs = tiles * s;
        const long waves = (wgs + kCUs - 1) / kCUs;
        const long active = wgs < kCUs ? wgs : kCUs;
        const double mfma_t = 2.0 * BM * BN * ((double)K / s) / cu_rate;
        const double load_t = 2.0 * BN * ((double)K / s) / (hbm / active);
        const double t = waves * (mfma_t > load_t ? mfma_t : load_t) +
                         (s > 1 ? 2.0 * s * (double)M * N * 4 / hbm : 0.0);
        if (t < best_t * (1.0 - 1e-9)) { best_t = t; best = s; }
    }
    return best;
}

struct FuseLayout {
    int s1, s2;
    size_t p1, h, p2, bytes;
};

FuseLayout fuse_layout(int rows, int kx, int d_model, int nkvc) {
    FuseLayout L{};
    L.s1 = pick_splits(rows, d_model, kx);
    L.s2 = pick_splits(rows, nkvc, d_model);
    Carve c;
    L.p1 = c.take<float>((size_t)L.s1 * rows * d_model);
    L.h = c.take<uint16_t>((size_t)rows * d_model);
    L.p2 = c.take<float>((size_t)L.s2 * rows * nkvc);
    L.bytes = c.total();
    return L;
}

void launch_rmsnorm(int S, const float* P, int M, int N, const float* gain, float eps, uint16_t* H,
                    uint16_t* h_out, hipStream_t st) {
    const size_t lds = (size_t)N * sizeof(float);
    switch (S) {
        case 1: hipLaunchKernelGGL(rmsnorm_kernel<1>, dim3(M), dim3(kNormThreads), lds, st, P, M, N, gain, eps, H, h_out); break;
        case 2: hipLaunchKernelGGL(rmsnorm_kernel<2>, dim3(M), dim3(kNormThreads), lds, st, P, M, N, gain, eps, H, h_out); break;
        case 4: hipLaunchKernelGGL(rmsnorm_kernel<4>, dim3(M), dim3(kNormThreads), lds, st, P, M, N, gain, eps, H, h_out); break;
        default: hipLaunchKernelGGL(rmsnorm_kernel<8>, dim3(M), dim3(kNormThreads), lds, st, P, M, N, gain, eps, H, h_out); break;
    }
}

void launch_append(int S, dim3 grid, const float* P, int M, int NC, const int32_t* row_seq,
                   const int64_t* row_pos, uint16_t* ring, int B, int NKV, int DH, int W, hipStream_t st) {
    switch (S) {
        case 1: hipLaunchKernelGGL(kv_append_kernel<1>, grid, dim3(256), 0, st, P, M, NC, row_seq, row_pos, ring, B, NKV, DH, W); break;
        case 2: hipLaunchKernelGGL(kv_append_kernel<2>, grid, dim3(256), 0, st, P, M, NC, row_seq, row_pos, ring, B, NKV, DH, W); break;
        case 4: hipLaunchKernelGGL(kv_append_kernel<4>, grid, dim3(256), 0, st, P, M, NC, row_seq, row_pos, ring, B, NKV, DH, W); break;
        default: hipLaunchKernelGGL(kv_append_kernel<8>, grid, dim3(256), 0, st, P, M, NC, row_seq, row_pos, ring, B, NKV, DH, W); break;
    }
}

void launch_gemm(const uint16_t* A, bool a_slabs, const uint16_t* B, float* C, int M, int N, int K, int S,
                 hipStream_t st) {
    GemmArgs g{A, B, C, M, N, K, S, (M + BM - 1) / BM, (N + BN - 1) / BN};
    const int per_round = kXCDs / S;  // column blocks per round of 8 workgroups
    const int rounds = (g.n_nt + per_round - 1) / per_round;
    const dim3 grid(kXCDs * rounds * g.n_mt), block(64 * (kGConsumers + kGProducers));
    if (a_slabs) hipLaunchKernelGGL(gemm_nt_bf16_kernel<true>, grid, block, 0, st, g);
    else hipLaunchKernelGGL(gemm_nt_bf16_kernel<false>, grid, block, 0, st, g);
}

}  // namespace
}  // namespace dfl

using namespace dfl;

namespace dfl {
namespace {

// Shape part of the checks (every size already >= 1): DFLASH_ERR_UNSUPPORTED
// or OK, with the GEMMs' reduction and output widths in kx and nkvc.
int fuse_shape(int rows, int n_taps, int d_tgt, int d_model, int n_layers, int n_kv, int d_head,
               int64_t& kx, int64_t& nkvc) {
    kx = capped_product(kMaxFuseWidth, {n_taps, d_tgt});
    nkvc = capped_product(kMaxFuseWidth, {n_layers, 2, n_kv, d_head});
    if (kx < 0 || nkvc < 0 || rows > kMaxFuseRows) return DFLASH_ERR_UNSUPPORTED;
    if (kx % 64 || d_model % 128 || nkvc % 128 || d_model > 8192 || d_head % 4)
        return DFLASH_ERR_UNSUPPORTED;
    return DFLASH_OK;
}

}  // namespace
}  // namespace dfl

extern "C" size_t dflash_context_fuse_workspace_size(int rows, int n_taps, int d_tgt, int d_model,
                                                     int n_layers, int n_kv, int d_head) {
    if (rows < 1 || n_taps < 1 || d_tgt < 1 || d_model < 1 || n_layers < 1 || n_kv < 1 ||
        d_head < 1)
        return 0;
    int64_t kx, nkvc;
    if (fuse_shape(rows, n_taps, d_tgt, d_model, n_layers, n_kv, d_head, kx, nkvc) != DFLASH_OK)
        return 0;
    return fuse_layout(rows, (int)kx, d_model, (int)nkvc).bytes;
}

extern "C" int dflash_context_fuse(const uint16_t* taps, const uint16_t* w_c, const float* rms_gain,
                                   float eps, const uint16_t* w_kv, const int32_t* row_seq,
                                   const int64_t* row_pos, uint16_t* kv_ring, uint16_t* h_t_out,
                                   int rows, int n_taps, int d_tgt, int d_model, int n_layers,
                                   int n_kv, int d_head, int window, int batch, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (rows < 1 || n_taps < 1 || d_tgt < 1 || d_model < 1 || n_layers < 1 || n_kv < 1 ||
        d_head < 1 || window < 1 || batch < 1)
        return DFLASH_ERR_SHAPE;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return DFLASH_ERR_SHAPE;
    if (!taps || !w_c || !rms_gain || !w_kv || !row_seq || !row_pos || !kv_ring)
        return DFLASH_ERR_NULL;
    int64_t kx, nkvc;
    const int shape = fuse_shape(rows, n_taps, d_tgt, d_model, n_layers, n_kv, d_head, kx, nkvc);
    if (shape != DFLASH_OK) return shape;
    const FuseLayout L = fuse_layout(rows, (int)kx, d_model, (int)nkvc);
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255) || workspace_bytes < L.bytes)
        return DFLASH_ERR_WORKSPACE;
    char* ws = static_cast<char*>(workspace);
    float* P1 = reinterpret_cast<float*>(ws + L.p1);
    uint16_t* H = reinterpret_cast<uint16_t*>(ws + L.h);
    float* P2 = reinterpret_cast<float*>(ws + L.p2);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    launch_gemm(taps, false, w_c, P1, rows, d_model, (int)kx, L.s1, st);
    int rc = launch_status();
    if (rc) return rc;
    launch_rmsnorm(L.s1, P1, rows, d_model, rms_gain, eps, H, h_t_out, st);
    rc = launch_status();
    if (rc) return rc;
    launch_gemm(H, true, w_kv, P2, rows, (int)nkvc, d_model, L.s2, st);
    rc = launch_status();
    if (rc) return rc;
#if DFLASH_DEVICE_CHECKS
    hipLaunchKernelGGL(fuse_slot_check_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, row_seq,
                       row_pos, rows, batch, window);
    rc = launch_status();
    if (rc) return rc;
#endif
    dim3 grid((unsigned)((nkvc / 4 + 255) / 256), rows);
    launch_append(L.s2, grid, P2, rows, (int)nkvc, row_seq, row_pos, kv_ring, batch, n_kv, d_head,
                  window, st);
    return launch_status();
}
