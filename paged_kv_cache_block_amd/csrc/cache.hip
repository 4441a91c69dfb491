// Cache writes: reshape_and_cache (new K/V rows into their slots) and the
// whole-block copies a copy-on-write needs.
//
// Slot semantics follow abhik.ai "examples/pagedattention.py" (region
// append_or_allocate stores token p at (table[p / block_size], p % block_size);
// region copy_on_write copies the whole shared block before the private
// append).  Both kernels are plain HBM streams: 16-byte accesses where the
// layout allows, no LDS.
#include "device.hpp"
#include "kernels.hpp"

namespace pa {

namespace {

struct CopyList {
  int32_t src[kMaxCopiesPerLaunch];
  int32_t dst[kMaxCopiesPerLaunch];
};

// grid.y = copy index, grid.z = 0 (K) / 1 (V); each thread moves 16 bytes.
__global__ __launch_bounds__(256) void copy_blocks_16(uint4* __restrict__ k_pool,
                                                      uint4* __restrict__ v_pool,
                                                      CopyList list, int64_t words_per_block) {
  uint4* pool = blockIdx.z ? v_pool : k_pool;
  const int64_t src = list.src[blockIdx.y], dst = list.dst[blockIdx.y];
  for (int64_t w = blockIdx.x * 256ll + threadIdx.x; w < words_per_block; w += gridDim.x * 256ll)
    pool[dst * words_per_block + w] = pool[src * words_per_block + w];
}

// Same with 2-byte words, for block sizes that are not a multiple of 16 bytes.
__global__ __launch_bounds__(256) void copy_blocks_2(uint16_t* __restrict__ k_pool,
                                                     uint16_t* __restrict__ v_pool,
                                                     CopyList list, int64_t words_per_block) {
  uint16_t* pool = blockIdx.z ? v_pool : k_pool;
  const int64_t src = list.src[blockIdx.y], dst = list.dst[blockIdx.y];
  for (int64_t w = blockIdx.x * 256ll + threadIdx.x; w < words_per_block; w += gridDim.x * 256ll)
    pool[dst * words_per_block + w] = pool[src * words_per_block + w];
}

// One thread per (row i, head h, element d).  K rows are contiguous in d; the
// V page is stored transposed ([head_dim][block_size]), so V writes stride
// by block_size.
template <typename T>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    T* __restrict__ k_pool, T* __restrict__ v_pool, const T* __restrict__ k_new,
    const T* __restrict__ v_new, const int64_t* __restrict__ slots, int64_t n, int32_t hkv,
    int32_t bs, int32_t dim, int64_t num_slots) {
  const int64_t per_row = static_cast<int64_t>(hkv) * dim;
  const int64_t total = n * per_row;
  for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < total; e += gridDim.x * 256ll) {
    const int64_t i = e / per_row;
    const int64_t rem = e - i * per_row;
    const int64_t h = rem / dim;
    const int64_t d = rem - h * dim;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / bs, off = slot - blk * bs;
    const int64_t page = (blk * hkv + h) * bs * dim;
    k_pool[page + off * dim + d] = k_new[e];
    v_pool[page + d * bs + off] = v_new[e];
  }
}

__global__ __launch_bounds__(256) void upload_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                     int64_t n16) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n16; i += gridDim.x * 256ll) dst[i] = src[i];
}

// Prologue of a decode step: blocks [0, nu) copy the plan (n16 16-byte
// words) from pinned host memory into the workspace; the other blocks store
// the batch's new K/V rows at the slots the plan carries (read from the same
// pinned buffer, since the workspace copy is being written concurrently).
template <typename T>
__global__ __launch_bounds__(256) void step_prep_kernel(
    const uint4* __restrict__ plan_src, uint4* __restrict__ plan_dst, int64_t n16, int nu,
    const int64_t* __restrict__ slots, T* __restrict__ k_pool, T* __restrict__ v_pool,
    const T* __restrict__ k_new, const T* __restrict__ v_new, int64_t n, int32_t hkv, int32_t bs,
    int32_t dim, int64_t num_slots) {
  if (static_cast<int>(blockIdx.x) < nu) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n16; i += nu * 256ll) plan_dst[i] = plan_src[i];
    return;
  }
  const int64_t per_row = static_cast<int64_t>(hkv) * dim;
  const int64_t total = n * per_row;
  const int64_t stride = (gridDim.x - nu) * 256ll;
  for (int64_t e = (blockIdx.x - nu) * 256ll + threadIdx.x; e < total; e += stride) {
    const int64_t i = e / per_row;
    const int64_t rem = e - i * per_row;
    const int64_t h = rem / dim;
    const int64_t d = rem - h * dim;
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / bs, off = slot - blk * bs;
    const int64_t page = (blk * hkv + h) * bs * dim;
    k_pool[page + off * dim + d] = k_new[e];
    v_pool[page + d * bs + off] = v_new[e];
  }
}

int grid_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_copy_blocks(const PoolGeom& geom, void* k_pool, void* v_pool,
                              const int32_t* src, const int32_t* dst, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  CopyList list{};
  for (int i = 0; i < n; ++i) {
    list.src[i] = src[i];
    list.dst[i] = dst[i];
  }
  const size_t bytes = geom.block_bytes();
  if (bytes % 16 == 0) {
    const int64_t words = static_cast<int64_t>(bytes / 16);
    dim3 grid(grid_for(words, 256, 1024), n, 2);
    hipLaunchKernelGGL(copy_blocks_16, grid, dim3(256), 0, stream, static_cast<uint4*>(k_pool),
                       static_cast<uint4*>(v_pool), list, words);
  } else {
    const int64_t words = static_cast<int64_t>(bytes / 2);
    dim3 grid(grid_for(words, 256, 1024), n, 2);
    hipLaunchKernelGGL(copy_blocks_2, grid, dim3(256), 0, stream, static_cast<uint16_t*>(k_pool),
                       static_cast<uint16_t*>(v_pool), list, words);
  }
  return hipGetLastError();
}

hipError_t launch_upload(const void* host_src, void* dst, size_t bytes, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(upload_kernel, dim3(grid_for(n16, 256, 64)), dim3(256), 0, stream,
                     static_cast<const uint4*>(host_src), static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

hipError_t launch_step_prep(const PoolGeom& geom, const void* plan_src, void* plan_dst, size_t bytes,
                            const int64_t* slots, void* k_pool, void* v_pool, const void* k_new,
                            const void* v_new, int32_t n, hipStream_t stream) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const int nu = grid_for(n16, 256, 32);
  const int64_t total = static_cast<int64_t>(n) * geom.num_kv_heads * geom.head_dim;
  const int nc = grid_for(total, 256, 4096);
  const int64_t num_slots = static_cast<int64_t>(geom.num_blocks) * geom.block_size;
  const dim3 grid(nu + nc);
  if (geom.dtype == 1)
    hipLaunchKernelGGL(step_prep_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(plan_src), static_cast<uint4*>(plan_dst), n16, nu, slots,
                       static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim, num_slots);
  else
    hipLaunchKernelGGL(step_prep_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(plan_src), static_cast<uint4*>(plan_dst), n16, nu, slots,
                       static_cast<float*>(k_pool), static_cast<float*>(v_pool),
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim, num_slots);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const PoolGeom& geom, void* k_pool, void* v_pool,
                                    const void* k_new, const void* v_new, const int64_t* slots,
                                    int32_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(n) * geom.num_kv_heads * geom.head_dim;
  const int64_t num_slots = static_cast<int64_t>(geom.num_blocks) * geom.block_size;
  const int grid = grid_for(total, 256, 65536);
  if (geom.dtype == 1) {
    hipLaunchKernelGGL(reshape_and_cache_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slots, static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size,
                       geom.head_dim, num_slots);
  } else {
    hipLaunchKernelGGL(reshape_and_cache_kernel<float>, dim3(grid), dim3(256), 0, stream,
                       static_cast<float*>(k_pool), static_cast<float*>(v_pool),
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new), slots,
                       static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim,
                       num_slots);
  }
  return hipGetLastError();
}

}  // namespace pa
