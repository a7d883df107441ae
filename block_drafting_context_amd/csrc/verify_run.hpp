// verify_run.hpp -- spec_verify's host-side checks and kernel sequence, for the
// entry points of libdflash.so that run a verification (internal; not part of
// the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dflash.h"

namespace dfl {

// Checks every host-checkable argument of spec_verify (no HIP call); returns
// a DFLASH_* status (DFLASH_OK also when batch == 0: nothing to do).
int verify_check(const float* target_logits, const int32_t* draft_tokens, float temperature,
                 const uint64_t* seeds, const int32_t* accept_len, const int32_t* out_tokens,
                 int batch, int gamma, int vocab);

// Bytes of device scratch one verification of this shape uses.
size_t verify_scratch_bytes(int batch, int gamma, int vocab);

// Enqueues the verification kernels on st, with their scratch at `scratch_ws`
// (256-byte aligned, verify_scratch_bytes bytes).  Arguments already checked.
int verify_enqueue(const float* target_logits, const float* draft_logits,
                   const int32_t* draft_tokens, const double* draft_lse,
                   const dflash_nucleus_cut* target_cut, const dflash_nucleus_cut* draft_cut,
                   float temperature, const uint64_t* seeds, uint64_t step, int32_t* accept_len,
                   int32_t* out_tokens, uint8_t* accepted, int batch, int gamma, int vocab,
                   void* scratch_ws, hipStream_t st);

}  // namespace dfl
