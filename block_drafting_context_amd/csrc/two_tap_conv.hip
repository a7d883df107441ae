// two_tap_conv.hip -- the DFlash 2 two-tap dynamic convolution, for gfx950.
//
// "DFlash vs DFlash 2", "The two-tap dynamic convolution": every block position
// mixes its representation with its immediate predecessor,
//     y_t = k_{t,0} * x_t + k_{t,1} * x_{t-1},
// depthwise, with content-dependent kernel values shared by a group of
// channels, never across a block boundary.  Block row 0 is the anchor's
// position; row t >= 1 reads row t - 1 (so the first drafted position reads
// the anchor) and row 0 has no predecessor.
//
// Memory-bound and elementwise: one thread per 8 channels of one (sequence,
// position), 16-byte loads of x_t and x_{t-1}, fp32 arithmetic, bf16 output
// rounded to nearest even.
#include "common.hpp"

namespace dfl {
namespace {

// batch * gamma * d: one thread per 8 channels keeps the launch below 2^32 work-items
constexpr int64_t kMaxConvElems = int64_t(1) << 34;

struct ConvArgs {
    const uint16_t* x;  // [B, G, D] bf16
    const float* kern;  // [B, G, 2, n_groups]
    uint16_t* y;        // [B, G, D] bf16
    int B, G, D, n_groups, gs;
    long n8;            // B * G * D / 8
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ void __launch_bounds__(256) two_tap_conv_kernel(ConvArgs a) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n8) return;
    const int d8 = a.D / 8;
    const long bt = i / d8;         // b * G + t
    const int c = (int)(i % d8) * 8;  // first channel
    const int t = (int)(bt % a.G);
    const int grp = c / a.gs;
    const float* kt = a.kern + bt * 2 * a.n_groups;
    const float k0 = kt[grp], k1 = kt[a.n_groups + grp];
    const u32x4 xt = *reinterpret_cast<const u32x4*>(a.x + bt * a.D + c);
    u32x4 xp = {0u, 0u, 0u, 0u};
    if (t > 0) xp = *reinterpret_cast<const u32x4*>(a.x + (bt - 1) * a.D + c);
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float lo = fmaf(k0, bf16_lo(xt[q]), k1 * bf16_lo(xp[q]));
        const float hi = fmaf(k0, bf16_hi(xt[q]), k1 * bf16_hi(xp[q]));
        out[q] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<u32x4*>(a.y + bt * a.D + c) = out;
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" int dflash_two_tap_conv(const uint16_t* x, const float* kern, uint16_t* y, int batch,
                                   int gamma, int d, int n_groups, void* stream) {
    if (batch < 0 || gamma < 1 || d < 1 || n_groups < 1 || d % n_groups) return DFLASH_ERR_SHAPE;
    if (batch == 0) return DFLASH_OK;
    if (!x || !kern || !y) return DFLASH_ERR_NULL;
    if (x == y) return DFLASH_ERR_SHAPE;
    if ((d / n_groups) % 8 || ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15))
        return DFLASH_ERR_UNSUPPORTED;
    // one thread per 8 channels: the launch's work-item count stays in 32 bits
    if (capped_product(kMaxConvElems, {batch, gamma, d}) < 0) return DFLASH_ERR_UNSUPPORTED;
    ConvArgs a{x, kern, y, batch, gamma, d, n_groups, d / n_groups, (long)batch * gamma * (d / 8)};
    const long blocks = (a.n8 + 255) / 256;
    hipLaunchKernelGGL(two_tap_conv_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), a);
    return launch_status();
}
