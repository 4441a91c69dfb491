// pa_decode_step_noalloc: the fused decode step for callers that cannot
// allocate memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Its workspace -- the uploaded plan and
// the split-K partial results -- is `scratch` below instead of a caller
// buffer; the kernels are the ones pa_decode_step launches.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "abi_internal.hpp"
#include "pagedattn.h"

namespace {

// One copy per GPU, held by that GPU until the process ends.  In host code
// this name is only a handle for hipGetSymbolAddress: the device address of
// each GPU's copy comes from that call (scratch_address) and is what the
// kernels receive.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the NULL stream), looked up once per device with that device
// current.
pa_status scratch_address(hipStream_t stream, void** addr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess)
    return pa::fail_status(PA_ERR_DEVICE, std::string("device of the stream: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return pa::fail_status(PA_ERR_DEVICE, "device ordinal " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_addr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    if (e != hipSuccess)
      return pa::fail_status(PA_ERR_DEVICE, std::string("select device: ") + hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || p == nullptr)
      return pa::fail_status(PA_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") +
                                                hipGetErrorString(e));
    if (back != hipSuccess)
      return pa::fail_status(PA_ERR_DEVICE, std::string("restore device: ") + hipGetErrorString(back));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_step_noalloc(pa_pool* pool, const int64_t* seqs, int32_t B,
                                            int32_t num_heads, const void* k_new, const void* v_new,
                                            const void* q, void* out, int64_t* slots_out, void* stream) {
  if (!pool) return pa::fail_status(PA_ERR_INVALID_ARG, "NULL pool");
  void* ws = nullptr;
  const pa_status r = scratch_address(static_cast<hipStream_t>(stream), &ws);
  if (r != PA_OK) return r;
  return pa::fused_step(pool, seqs, nullptr, B, num_heads, k_new, v_new, q, out,
                        {ws, PA_NOALLOC_SCRATCH_BYTES, true}, slots_out, stream);
}
