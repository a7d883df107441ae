// noalloc.hip -- spec_verify without a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// The verification's scratch lives in a fixed array in device memory: one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (in host code it names a host-side
// stand-in, not device memory): its device address on each device is looked
// up once, on the first call with that device current, by hipGetSymbolAddress,
// and that address is what the kernels receive.  Every call on one GPU shares
// the array, so calls that overlap on one GPU race; the kernels write every
// scratch entry they later read, so nothing has to start at zero.
#include <atomic>

#include "common.hpp"
#include "verify_run.hpp"

namespace dfl {
namespace {

constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up once per device).
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH_ERR_HIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return DFLASH_OK;
}

}  // namespace
}  // namespace dfl

using namespace dfl;

extern "C" size_t spec_verify_noalloc_max_scratch(void) { return kScratchBytes; }

extern "C" int spec_verify_noalloc(const float* target_logits, const float* draft_logits,
                                   const int32_t* draft_tokens, const double* draft_lse,
                                   const dflash_nucleus_cut* target_cut,
                                   const dflash_nucleus_cut* draft_cut, float temperature, const uint64_t* seeds, uint64_t step,
                                   int32_t* accept_len, int32_t* out_tokens, uint8_t* accepted,
                                   int batch, int gamma, int vocab, void* stream) {
    int rc = verify_check(target_logits, draft_tokens, temperature, seeds, accept_len, out_tokens,
                          batch, gamma, vocab);
    if (rc || batch == 0) return rc;
    if (verify_scratch_bytes(batch, gamma, vocab) > kScratchBytes) return DFLASH_ERR_TOO_LARGE;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return verify_enqueue(target_logits, draft_logits, draft_tokens, draft_lse, target_cut, draft_cut,
                          temperature, seeds, step, accept_len, out_tokens, accepted, batch, gamma,
                          vocab, ws, reinterpret_cast<hipStream_t>(stream));
}
