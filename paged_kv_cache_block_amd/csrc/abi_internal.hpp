// Internal interface between the C ABI's source files: the fused append +
// store + attention step with its workspace given by the caller of this
// function (abi.cpp passes the caller's buffer, noalloc.hip the library's
// static scratch).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "pagedattn.h"

namespace pa {

struct StepWorkspace {
  void* ptr;
  size_t bytes;
  // The library's fixed scratch array: nothing in the call may allocate
  // device or pinned host memory (a plan larger than the pool's reserved
  // staging buffers is an error instead of a reason to grow them).
  bool static_scratch;
};

// Append n_tokens[b] (1 each when NULL) tokens to every sequence, store
// their K/V rows and run attention for those rows (pa_decode_step when
// n_tokens is NULL, pa_verify_step otherwise).
pa_status fused_step(pa_pool* pool, const int64_t* seqs, const int32_t* n_tokens, int32_t B,
                     int32_t num_heads, const void* k_new, const void* v_new, const void* q, void* out,
                     const StepWorkspace& ws, int64_t* slots_out, void* stream);

// Record `msg` as the calling thread's last error and return `status`.
pa_status fail_status(pa_status status, const std::string& msg);

}  // namespace pa
