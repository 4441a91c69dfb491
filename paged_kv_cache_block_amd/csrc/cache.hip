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
