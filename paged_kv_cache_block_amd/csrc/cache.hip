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
#include "launch.hpp"

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

// Element offset of K (token t of the page, dim d): bf16 pages in the
// decode kernel's operand order where the shape allows it, fp32 row-major.
template <typename T>
__device__ __forceinline__ int64_t k_offset(int t, int d, int dim, int bs) {
  if constexpr (sizeof(T) == 2) return k16_offset(t, d, dim, bs);
  else return static_cast<int64_t>(t) * dim + d;
}

// One thread per (row i, head h, element d).  K elements go to their place
// in the page order above; the V page is stored transposed ([head_dim]
// [block_size]), so V writes stride by block_size.
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
    k_pool[page + k_offset<T>(static_cast<int>(off), static_cast<int>(d), dim, bs)] = k_new[e];
    v_pool[page + d * bs + off] = v_new[e];
  }
}

// --------------------------------------------------------- 8-bit pages ---
// Per-row absmax quantisation (vladkulikov.com notebook "Модуль 10", the
// KV-compression experiment): scale = max|x| / 127 (1 for a zero row), code =
// x / scale rounded to nearest even and clipped to [-127, 127], decided in
// float64; the page keeps the scale rounded to fp32.  This file is compiled
// without fast math, so the float64 division and rounding are the IEEE
// operations.
__device__ __forceinline__ int8_t q8_code(float x, double scale) {
  const double c = rint(static_cast<double>(x) / scale);
  return static_cast<int8_t>(static_cast<int>(fmin(fmax(c, -127.0), 127.0)));
}

__device__ __forceinline__ double q8_scale(float absmax) {
  const double s = static_cast<double>(absmax) / 127.0;
  return s == 0.0 ? 1.0 : s;
}

// E4M3 codes (bit 7 sign, exponent bias 7, no infinities): the value nearest
// to x / scale, decided in float64, ties to the even code, magnitudes above
// the largest value 448 to 448; a zero (of either sign) is code 0x00.
constexpr double kE4M3Max = 448.0;
__device__ __forceinline__ uint8_t f8_code(float x, double scale) {
  const double y = static_cast<double>(x) / scale;
  const double a = fmin(fabs(y), kE4M3Max);
  int k;
  (void)frexp(a, &k);                        // a = f * 2^k, f in [0.5, 1)
  const int e = max(k - 1, -6);              // exponent of a's binade (subnormals: -6)
  const double quantum = ldexp(1.0, e - 3);  // 3 mantissa bits
  const double r = rint(a / quantum) * quantum;
  if (r == 0.0) return 0;
  uint32_t mag;
  if (r < 0.015625) {  // below 2^-6: a subnormal m * 2^-9
    mag = static_cast<uint32_t>(r * 512.0);
  } else {
    int kr;
    (void)frexp(r, &kr);
    const int er = kr - 1;
    mag = (static_cast<uint32_t>(er + 7) << 3) | static_cast<uint32_t>(r / ldexp(1.0, er - 3) - 8.0);
  }
  return static_cast<uint8_t>((y < 0.0 ? 0x80u : 0u) | mag);
}

__device__ __forceinline__ double f8_scale(float absmax) {
  const double s = static_cast<double>(absmax) / kE4M3Max;
  return s == 0.0 ? 1.0 : s;
}

// Code and scale of a row, by code kind (1: int8, 2: E4M3).
template <int Q8>
__device__ __forceinline__ uint8_t row_code(float x, double scale) {
  if constexpr (Q8 == 2) return f8_code(x, scale);
  else return static_cast<uint8_t>(q8_code(x, scale));
}
template <int Q8>
__device__ __forceinline__ double row_scale(float absmax) {
  if constexpr (Q8 == 2) return f8_scale(absmax);
  else return q8_scale(absmax);
}

// One wave quantises one (row, head): K and V codes at their places in the
// page order (k8_offset, q8_v_offset), then the two fp32 scales.  D <= 512 (8 values per lane).
template <int Q8>
__device__ __forceinline__ void q8_store_row_head(uint8_t* k_pool, uint8_t* v_pool, const uint16_t* k_row,
                                                  const uint16_t* v_row, int64_t blk, int32_t off,
                                                  int32_t h, int32_t hkv, int32_t bs, int32_t dim, int lane) {
  float kx[8], vx[8];
  float kmax = 0.f, vmax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int d = lane + 64 * k;
    kx[k] = d < dim ? bf16_to_f32(k_row[d]) : 0.f;
    vx[k] = d < dim ? bf16_to_f32(v_row[d]) : 0.f;
    kmax = fmaxf(kmax, fabsf(kx[k]));
    vmax = fmaxf(vmax, fabsf(vx[k]));
  }
  kmax = wave_max(kmax);
  vmax = wave_max(vmax);
  const double ks = row_scale<Q8>(kmax), vs = row_scale<Q8>(vmax);
  const size_t page_bytes = static_cast<size_t>(bs) * dim + 4 * static_cast<size_t>(bs);
  uint8_t* kp = k_pool + (blk * hkv + h) * page_bytes;
  uint8_t* vp = v_pool + (blk * hkv + h) * page_bytes;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int d = lane + 64 * k;
    if (d < dim) {
      kp[k8_offset(off, d, dim)] = row_code<Q8>(kx[k], ks);
      vp[q8_v_offset(off, d, dim)] = row_code<Q8>(vx[k], vs);
    }
  }
  if (lane == 0) {
    reinterpret_cast<float*>(kp + static_cast<size_t>(bs) * dim)[off] = static_cast<float>(ks);
    reinterpret_cast<float*>(vp + static_cast<size_t>(bs) * dim)[off] = static_cast<float>(vs);
  }
}

// reshape_and_cache for 8-bit pools: one wave per (row i, head h).
template <int Q8>
__global__ __launch_bounds__(256) void reshape_and_cache_q8(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int64_t* __restrict__ slots, int64_t n, int32_t hkv,
    int32_t bs, int32_t dim, int64_t num_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = n * hkv;
  for (int64_t rh = blockIdx.x * 4ll + (threadIdx.x >> 6); rh < rows; rh += gridDim.x * 4ll) {
    const int64_t i = rh / hkv;
    const int32_t h = static_cast<int32_t>(rh - i * hkv);
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / bs;
    q8_store_row_head<Q8>(k_pool, v_pool, k_new + rh * dim, v_new + rh * dim, blk,
                          static_cast<int32_t>(slot - blk * bs), h, hkv, bs, dim, lane);
  }
}

// Decode-step prologue for 8-bit pools: blocks [0, nu) copy the plan, the
// others quantise and store the new rows (one wave per (row, head)).
template <int Q8>
__global__ __launch_bounds__(256) void step_prep_q8(
    const uint4* __restrict__ plan_src, uint4* __restrict__ plan_dst, int64_t n16, int nu,
    const int64_t* __restrict__ slots, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, int64_t n, int32_t hkv,
    int32_t bs, int32_t dim, int64_t num_slots) {
  if (static_cast<int>(blockIdx.x) < nu) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n16; i += nu * 256ll) plan_dst[i] = plan_src[i];
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t rows = n * hkv;
  const int64_t stride = (gridDim.x - nu) * 4ll;
  for (int64_t rh = (blockIdx.x - nu) * 4ll + (threadIdx.x >> 6); rh < rows; rh += stride) {
    const int64_t i = rh / hkv;
    const int32_t h = static_cast<int32_t>(rh - i * hkv);
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;
    const int64_t blk = slot / bs;
    q8_store_row_head<Q8>(k_pool, v_pool, k_new + rh * dim, v_new + rh * dim, blk,
                          static_cast<int32_t>(slot - blk * bs), h, hkv, bs, dim, lane);
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
    k_pool[page + k_offset<T>(static_cast<int>(off), static_cast<int>(d), dim, bs)] = k_new[e];
    v_pool[page + d * bs + off] = v_new[e];
  }
}

// Slot check of one reshape_and_cache call, before it writes anything
// (validate before mutate, as the [PagedPool] negative tests require of the
// bookkeeping): one workgroup walks the rows; a slot outside [0, num_slots)
// marks its row, and marks[slot] takes the call's stamp, so a row that finds
// the stamp already there names a slot another row of the same call names.
// result[0] / result[1] = the smallest row with a slot out of range / that
// found its slot taken, or -1.
__global__ __launch_bounds__(1024) void check_slots_kernel(const int64_t* __restrict__ slots, int32_t n,
                                                           int64_t num_slots, uint32_t* __restrict__ marks,
                                                           uint32_t stamp, int32_t* __restrict__ result) {
  __shared__ int32_t first_bad[2];
  if (threadIdx.x < 2) first_bad[threadIdx.x] = INT32_MAX;
  __syncthreads();
  for (int32_t i = threadIdx.x; i < n; i += 1024) {
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots)
      atomicMin(&first_bad[0], i);
    else if (atomicExch(&marks[slot], stamp) == stamp)
      atomicMin(&first_bad[1], i);
  }
  __syncthreads();
  if (threadIdx.x < 2) result[threadIdx.x] = first_bad[threadIdx.x] == INT32_MAX ? -1 : first_bad[threadIdx.x];
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += gridDim.x * 256ll) p[i] = 0u;
}

int grid_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return static_cast<int>(g);
}

}  // namespace

hipError_t launch_copy_blocks(const PoolGeom& geom, void* k_pool, void* v_pool,
                              const int32_t* src, const int32_t* dst, int n, hipStream_t stream,
                              const KernelEvents& ev) {
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
    PA_LAUNCH(ev, copy_blocks_16, grid, dim3(256), 0, stream, static_cast<uint4*>(k_pool),
                       static_cast<uint4*>(v_pool), list, words);
  } else {
    const int64_t words = static_cast<int64_t>(bytes / 2);
    dim3 grid(grid_for(words, 256, 1024), n, 2);
    PA_LAUNCH(ev, copy_blocks_2, grid, dim3(256), 0, stream, static_cast<uint16_t*>(k_pool),
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
                            const void* v_new, int32_t n, hipStream_t stream,
                            const KernelEvents& ev) {
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const int nu = grid_for(n16, 256, 32);
  const int64_t total = static_cast<int64_t>(n) * geom.num_kv_heads * geom.head_dim;
  const int nc = grid_for(total, 256, 4096);
  const int64_t num_slots = static_cast<int64_t>(geom.num_blocks) * geom.block_size;
  if (geom.q8()) {
    const int nq = grid_for(static_cast<int64_t>(n) * geom.num_kv_heads, 4, 4096);
    if (geom.fp8())
      PA_LAUNCH(ev, step_prep_q8<2>, dim3(nu + nq), dim3(256), 0, stream,
                static_cast<const uint4*>(plan_src), static_cast<uint4*>(plan_dst), n16, nu, slots,
                static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim, num_slots);
    else
      PA_LAUNCH(ev, step_prep_q8<1>, dim3(nu + nq), dim3(256), 0, stream,
                static_cast<const uint4*>(plan_src), static_cast<uint4*>(plan_dst), n16, nu, slots,
                static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
                static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim, num_slots);
    return hipGetLastError();
  }
  const dim3 grid(nu + nc);
  if (geom.dtype == 1)
    PA_LAUNCH(ev, step_prep_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(plan_src), static_cast<uint4*>(plan_dst), n16, nu, slots,
                       static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim, num_slots);
  else
    PA_LAUNCH(ev, step_prep_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const uint4*>(plan_src), static_cast<uint4*>(plan_dst), n16, nu, slots,
                       static_cast<float*>(k_pool), static_cast<float*>(v_pool),
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new),
                       static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim, num_slots);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const PoolGeom& geom, void* k_pool, void* v_pool,
                                    const void* k_new, const void* v_new, const int64_t* slots,
                                    int32_t n, hipStream_t stream, const KernelEvents& ev) {
  if (n <= 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(n) * geom.num_kv_heads * geom.head_dim;
  const int64_t num_slots = static_cast<int64_t>(geom.num_blocks) * geom.block_size;
  const int grid = grid_for(total, 256, 65536);
  if (geom.q8()) {
    const int gq = grid_for(static_cast<int64_t>(n) * geom.num_kv_heads, 4, 65536);
    if (geom.fp8())
      PA_LAUNCH(ev, reshape_and_cache_q8<2>, dim3(gq), dim3(256), 0, stream, static_cast<uint8_t*>(k_pool),
                static_cast<uint8_t*>(v_pool), static_cast<const uint16_t*>(k_new),
                static_cast<const uint16_t*>(v_new), slots, static_cast<int64_t>(n), geom.num_kv_heads,
                geom.block_size, geom.head_dim, num_slots);
    else
      PA_LAUNCH(ev, reshape_and_cache_q8<1>, dim3(gq), dim3(256), 0, stream, static_cast<uint8_t*>(k_pool),
                static_cast<uint8_t*>(v_pool), static_cast<const uint16_t*>(k_new),
                static_cast<const uint16_t*>(v_new), slots, static_cast<int64_t>(n), geom.num_kv_heads,
                geom.block_size, geom.head_dim, num_slots);
  } else if (geom.dtype == 1) {
    PA_LAUNCH(ev, reshape_and_cache_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slots, static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size,
                       geom.head_dim, num_slots);
  } else {
    PA_LAUNCH(ev, reshape_and_cache_kernel<float>, dim3(grid), dim3(256), 0, stream,
                       static_cast<float*>(k_pool), static_cast<float*>(v_pool),
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new), slots,
                       static_cast<int64_t>(n), geom.num_kv_heads, geom.block_size, geom.head_dim,
                       num_slots);
  }
  return hipGetLastError();
}

hipError_t launch_check_slots(const PoolGeom& geom, const int64_t* slots, int32_t n, uint32_t* marks,
                              uint32_t stamp, int32_t* result, hipStream_t stream) {
  const int64_t num_slots = static_cast<int64_t>(geom.num_blocks) * geom.block_size;
  hipLaunchKernelGGL(check_slots_kernel, dim3(1), dim3(1024), 0, stream, slots, n, num_slots, marks, stamp,
                     result);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(grid_for(n, 256, 4096)), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace pa
