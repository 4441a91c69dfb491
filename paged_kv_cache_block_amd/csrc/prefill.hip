// Chunked causal prefill over the paged pool.
//
// What is computed (docs.rs ferrum-kv 0.4.0 src/attention.rs,
// paged_attention with q_tokens > 1): the q_len query rows of a sequence are
// its last q_len positions; row t sees keys j <= kv_len - q_len + t.
#include "device.hpp"
#include "kernels.hpp"

namespace pa {

hipError_t launch_prefill_generic(const PoolGeom& geom, const PrefillArgs& a, hipStream_t stream);

bool prefill_uses_mfma(const PoolGeom&, int32_t) { return false; }

int32_t prefill_rows_per_tile(const PoolGeom&, int32_t) { return 64; }

hipError_t launch_prefill(const PoolGeom& geom, const PrefillArgs& a, hipStream_t stream) {
  return launch_prefill_generic(geom, a, stream);
}

}  // namespace pa
