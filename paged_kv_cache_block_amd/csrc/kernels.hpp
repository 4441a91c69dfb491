// Host launchers of the gfx950 kernels (defined in the .hip files).
#pragma once

#include <hip/hip_runtime_api.h>

#include "plan.hpp"

namespace pa {

constexpr int kMaxCopiesPerLaunch = 64;

// Timing events of one launch (either may be null): set from the kernel's
// dispatch, with nothing added to the stream between kernels.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Whole-block copies src[i] -> dst[i] (K and V, all heads), i < n <= 64, in
// one launch.  The caller splits dependent copies into separate launches.
hipError_t launch_copy_blocks(const PoolGeom& geom, void* k_pool, void* v_pool,
                              const int32_t* src, const int32_t* dst, int n, hipStream_t stream,
                              const KernelEvents& ev = KernelEvents{});

// Copy `bytes` (a multiple of 16) from device-visible pinned host memory to
// device memory with a kernel on `stream`, so the copy is ordered with the
// stream's kernels without a hand-off to a DMA engine.
hipError_t launch_upload(const void* host_src, void* dst, size_t bytes, hipStream_t stream);

// One kernel: upload `bytes` of plan (pinned -> device) and store n new K/V
// rows at `slots` (a device-visible pinned array).
hipError_t launch_step_prep(const PoolGeom& geom, const void* plan_src, void* plan_dst, size_t bytes,
                            const int64_t* slots, void* k_pool, void* v_pool, const void* k_new,
                            const void* v_new, int32_t n, hipStream_t stream,
                            const KernelEvents& ev = KernelEvents{});

// Kpool[slot/bs][h][slot%bs][:] = k_new[i][h][:], Vpool[slot/bs][h][:][slot%bs] = v_new[i][h][:].
hipError_t launch_reshape_and_cache(const PoolGeom& geom, void* k_pool, void* v_pool,
                                    const void* k_new, const void* v_new, const int64_t* slots,
                                    int32_t n, hipStream_t stream,
                                    const KernelEvents& ev = KernelEvents{});

// Debug slot check of n rows' slots (device int64 [n]): result (device
// int32 [2]) receives the smallest row whose slot is outside the pool and the
// smallest row that found its slot already taken by another row of the call
// (-1 = none; which row of a repeated pair reports it depends on timing).
// marks (device uint32 [num_blocks * block_size]) keeps per slot the stamp of
// the last check that saw it; stamps must differ between calls.
hipError_t launch_check_slots(const PoolGeom& geom, const int64_t* slots, int32_t n, uint32_t* marks,
                              uint32_t stamp, int32_t* result, hipStream_t stream);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t stream);

// Which decode kernel serves a geometry (for timing labels and tests).
enum class DecodeKernel { kGqaMfma, kQ8Mfma, kGeneric };
DecodeKernel pick_decode_kernel(const PoolGeom& geom, int32_t group);

// Query-row columns (q_len * group) one decode workgroup covers.
constexpr int32_t kDecodeMaxCols = 32;
// Whether the split-K decode kernels serve query rows of up to max_q_len
// positions per sequence (the MFMA kernels, q_len * group <= 32).
bool decode_handles_rows(const PoolGeom& geom, int32_t group, int32_t max_q_len);

// Decode: partial kernel, then (if any sequence was split) the merge.
hipError_t launch_decode_partial(const PoolGeom& geom, const DecodeArgs& args, hipStream_t stream,
                                 const KernelEvents& ev = KernelEvents{});
hipError_t launch_decode_merge(const PoolGeom& geom, const DecodeArgs& args, hipStream_t stream,
                               const KernelEvents& ev = KernelEvents{});
// Whether split sequences need the separate merge kernel (false when the
// partial kernel merges in its last workgroup, or never splits).
bool decode_needs_merge_kernel(const PoolGeom& geom, int32_t group);

// Prefill (chunked, causal).
hipError_t launch_prefill(const PoolGeom& geom, const PrefillArgs& args, hipStream_t stream,
                          const KernelEvents& ev = KernelEvents{});
bool prefill_uses_mfma(const PoolGeom& geom, int32_t group);
int32_t prefill_rows_per_tile(const PoolGeom& geom, int32_t group);

}  // namespace pa
