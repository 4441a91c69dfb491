// C ABI of libpagedattn.so (declared in include/pagedattn.h).
//
// Host metadata lives in pa::BlockPool (pool.cpp); work plans in plan.cpp;
// kernels in cache.hip / decode.hip / prefill.hip.  This file validates
// arguments, moves plans into the caller's workspace through pinned staging
// buffers, orders pending copy-on-write copies before any other device work
// on the pool, and records optional per-kernel timing events.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "abi_internal.hpp"
#include "kernels.hpp"
#include "pagedattn.h"
#include "plan.hpp"
#include "pool.hpp"
#include "prefix.hpp"

namespace {

thread_local std::string g_err;

pa_status fail(int status, const std::string& msg) {
  g_err = msg;
  return static_cast<pa_status>(status);
}

pa_status ok() { return PA_OK; }

pa_status from(pa::Status s, const std::string& msg) {
  return s == pa::kOk ? ok() : fail(s, msg);
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

#define PA_HIP(call)                                  \
  do {                                                \
    hipError_t e_ = (call);                           \
    if (e_ != hipSuccess) return hip_fail(e_, #call); \
  } while (0)

// ------------------------------------------------------------------ timing
struct TimingRecord {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
uint32_t g_timing_mask = ~0u;  // kernel families that get events while timing is on
std::vector<TimingRecord> g_records;
std::vector<hipEvent_t> g_spare_events;  // drained events, reused by later launches
double g_total_ms[PA_KERNEL_COUNT] = {};
int64_t g_launches[PA_KERNEL_COUNT] = {};
std::vector<float> g_samples[PA_KERNEL_COUNT];  // per-launch ms since the last reset

// While timing is on, a launch of a selected kernel family takes two events
// that its dispatch itself fills with the kernel's start and end
// (hipExtLaunchKernel): nothing is recorded on the stream between kernels,
// so timing does not change the spacing of a step's kernels.
struct TimedLaunch {
  int kernel;
  pa::KernelEvents ev;
  explicit TimedLaunch(int k) : kernel(k) {
    std::lock_guard<std::mutex> lock(g_tmu);
    if (!g_timing || !(g_timing_mask & (1u << k))) return;
    if (!take(&ev.start) || !take(&ev.stop)) {
      if (ev.start) g_spare_events.push_back(ev.start);
      if (ev.stop) g_spare_events.push_back(ev.stop);
      ev = pa::KernelEvents{};
    }
  }
  const pa::KernelEvents& events() const { return ev; }
  static bool take(hipEvent_t* e) {
    if (!g_spare_events.empty()) {
      *e = g_spare_events.back();
      g_spare_events.pop_back();
      return true;
    }
    if (hipEventCreate(e) == hipSuccess) return true;
    *e = nullptr;
    return false;
  }
  // After the launch: keep the events for the next read (launched == false:
  // the dispatch failed and the events go back unused).
  void done(bool launched = true) {
    if (!ev.start) return;
    std::lock_guard<std::mutex> lock(g_tmu);
    if (launched) {
      g_records.push_back({kernel, ev.start, ev.stop});
    } else {
      g_spare_events.push_back(ev.start);
      g_spare_events.push_back(ev.stop);
    }
    ev = pa::KernelEvents{};
  }
};

void drain_timing_locked() {
  for (auto& r : g_records) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      g_total_ms[r.kernel] += ms;
      g_launches[r.kernel] += 1;
      g_samples[r.kernel].push_back(ms);
    }
    g_spare_events.push_back(r.start);
    g_spare_events.push_back(r.stop);
  }
  g_records.clear();
}

}  // namespace

// -------------------------------------------------------------------- pool
struct pa_pool {
  pa::BlockPool meta;
  pa::PrefixCache prefix;  // complete-block prefix keys -> pinned blocks
  pa::DecodePlan plan;     // the last decode plan; its buffer is reused by the next call
  pa::PoolGeom geom{};
  void* k = nullptr;
  void* v = nullptr;
  struct Staging {
    void* host = nullptr;
    void* dev = nullptr;  // device address of the same pinned buffer
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
  };
  static constexpr int kRing = 4;
  Staging ring[kRing];
  int next = 0;
  // Debug slot checks of pa_reshape_and_cache (pa_pool_set_slot_checks):
  // per-slot stamps and the check's result, device memory of the library.
  uint32_t* slot_marks = nullptr;
  int32_t* check_result = nullptr;
  uint32_t check_stamp = 0;

  bool has_device() const { return k != nullptr; }

  // Copy `bytes` of host data into the next pinned staging buffer and return
  // its device address; the buffer is reused only after the event recorded
  // behind its previous use (staged_done) has fired.  The ring is reserved
  // when the pool is created (reserve_staging); a plan larger than that
  // grows every idle buffer of the ring at once when `may_grow`, and is an
  // error otherwise (the entry point that allocates nothing).
  pa_status stage(const void* src, size_t bytes, const void** dev_copy, bool may_grow = true) {
    Staging& st = ring[next];
    const size_t padded = pa::align_up(bytes, 16);
    if (st.cap < padded && !may_grow)
      return fail(PA_ERR_INVALID_ARG, "plan of " + std::to_string(padded) +
                                          " bytes exceeds the pool's reserved staging buffers (" +
                                          std::to_string(st.cap) + " bytes; see pa_pool_reserve_staging)");
    if (st.pending) {
      PA_HIP(hipEventSynchronize(st.ev));
      st.pending = false;
    }
    if (st.cap < padded) {
      const size_t cap = pa::align_up(std::max<size_t>(padded + padded / 2, 1 << 16), 16);
      for (Staging& b : ring) {
        if (&b != &st && (b.pending || b.cap >= padded)) continue;
        const pa_status r = grow(b, cap);
        if (r != PA_OK) return r;
      }
    }
    std::memcpy(st.host, src, bytes);
    *dev_copy = st.dev;
    return ok();
  }

  // Grow every buffer of the ring to at least `bytes` (waiting for buffers
  // still in use); buffers already that large are kept.
  pa_status reserve_staging(size_t bytes) {
    const size_t cap = pa::align_up(std::max<size_t>(bytes, 16), 16);
    for (Staging& b : ring) {
      if (b.cap >= cap) continue;
      if (b.pending) {
        PA_HIP(hipEventSynchronize(b.ev));
        b.pending = false;
      }
      const pa_status r = grow(b, cap);
      if (r != PA_OK) return r;
    }
    return ok();
  }

  size_t staging_capacity() const {
    size_t cap = ring[0].cap;
    for (const Staging& b : ring) cap = std::min(cap, b.cap);
    return cap;
  }

  pa_status grow(Staging& b, size_t cap) {
    if (!b.ev) PA_HIP(hipEventCreateWithFlags(&b.ev, hipEventDisableTiming));
    if (b.host) PA_HIP(hipHostFree(b.host));
    b.host = b.dev = nullptr;
    b.cap = 0;
    PA_HIP(hipHostMalloc(&b.host, cap, hipHostMallocDefault));
    PA_HIP(hipHostGetDevicePointer(&b.dev, b.host, 0));
    b.cap = cap;
    return ok();
  }

  // Mark the buffer of the last stage() as in use by the work enqueued on
  // `stream` so far.  If the event cannot be recorded, wait for the stream
  // instead, so the buffer is free when the ring comes back to it.
  pa_status staged_done(hipStream_t stream) {
    Staging& st = ring[next];
    next = (next + 1) % kRing;
    const hipError_t e = hipEventRecord(st.ev, stream);
    if (e != hipSuccess) {
      (void)hipStreamSynchronize(stream);
      st.pending = false;
      return hip_fail(e, "hipEventRecord");
    }
    st.pending = true;
    return ok();
  }

  // Holds the buffer of the last stage() for everything a call enqueues
  // after it: the event is recorded when the guard ends, behind the call's
  // last kernel.  (An event recorded between two kernels makes the second
  // wait there for the first to complete and its results to be published,
  // ~8-10 us on the decode step.)
  struct StagedUse {
    pa_pool* pool = nullptr;
    hipStream_t stream = nullptr;
    StagedUse() = default;
    StagedUse(const StagedUse&) = delete;
    StagedUse& operator=(const StagedUse&) = delete;
    ~StagedUse() {
      if (pool) (void)pool->staged_done(stream);
    }
  };

  // Copy `bytes` of host data to device `dst` (which has room for `bytes`
  // rounded up to 16) on `stream`: a small kernel on the stream reads the
  // pinned buffer, so the data is in place when the stream's next kernel
  // starts, without a hand-off to a DMA engine.
  pa_status upload(const void* src, size_t bytes, void* dst, hipStream_t stream, StagedUse* use) {
    const void* staged = nullptr;
    pa_status r = stage(src, bytes, &staged);
    if (r != PA_OK) return r;
    hipError_t e = pa::launch_upload(staged, dst, pa::align_up(bytes, 16), stream);
    if (e != hipSuccess) return hip_fail(e, "upload launch");
    use->pool = this;
    use->stream = stream;
    return ok();
  }

  pa_status flush(hipStream_t stream) {
    auto copies = meta.take_pending_copies();
    if (!has_device() || copies.empty()) return ok();
    // Copies that touch a block an earlier copy of the same launch writes
    // (or reads) go to a later launch, so recording order is kept.
    size_t i = 0;
    while (i < copies.size()) {
      std::vector<int32_t> src, dst;
      while (i < copies.size() && static_cast<int>(src.size()) < pa::kMaxCopiesPerLaunch) {
        const int32_t s = copies[i].first, d = copies[i].second;
        bool clash = false;
        for (size_t j = 0; j < src.size() && !clash; ++j)
          clash = s == dst[j] || d == dst[j] || d == src[j];
        if (clash) break;
        src.push_back(s);
        dst.push_back(d);
        ++i;
      }
      TimedLaunch t(PA_KERNEL_COPY);
      hipError_t e = pa::launch_copy_blocks(geom, k, v, src.data(), dst.data(),
                                            static_cast<int>(src.size()), stream, t.events());
      t.done(e == hipSuccess);
      if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
    }
    return ok();
  }

  // Turn the slot checks on (allocating their device memory, zeroed on
  // `stream`) or off (freeing it once the device is idle).
  pa_status set_slot_checks(bool on, hipStream_t stream) {
    if (on == (slot_marks != nullptr)) return ok();
    if (!on) {
      PA_HIP(hipDeviceSynchronize());
      PA_HIP(hipFree(slot_marks));
      PA_HIP(hipFree(check_result));
      slot_marks = nullptr;
      check_result = nullptr;
      return ok();
    }
    const int64_t n = static_cast<int64_t>(geom.num_blocks) * geom.block_size;
    uint32_t* marks = nullptr;
    int32_t* result = nullptr;
    hipError_t e = hipMalloc(&marks, sizeof(uint32_t) * n);
    if (e == hipSuccess) e = hipMalloc(&result, 2 * sizeof(int32_t));
    if (e == hipSuccess) e = pa::launch_zero_u32(marks, n, stream);
    if (e != hipSuccess) {
      if (marks) (void)hipFree(marks);
      if (result) (void)hipFree(result);
      return hip_fail(e, "slot checks");
    }
    slot_marks = marks;
    check_result = result;
    check_stamp = 0;
    return ok();
  }

  // The debug check of n caller slots before a cache write: waits for it on
  // `stream` and fails naming the first offending row.
  pa_status check_slots(const int64_t* slots, int32_t n, hipStream_t stream) {
    if (++check_stamp == 0) {  // stamps wrapped: every mark is stale again
      PA_HIP(pa::launch_zero_u32(slot_marks, static_cast<int64_t>(geom.num_blocks) * geom.block_size, stream));
      check_stamp = 1;
    }
    PA_HIP(pa::launch_check_slots(geom, slots, n, slot_marks, check_stamp, check_result, stream));
    int32_t bad[2] = {-1, -1};
    PA_HIP(hipMemcpyAsync(bad, check_result, sizeof(bad), hipMemcpyDeviceToHost, stream));
    PA_HIP(hipStreamSynchronize(stream));
    for (int kind = 0; kind < 2; ++kind) {
      if (bad[kind] < 0) continue;
      int64_t slot = 0;
      PA_HIP(hipMemcpy(&slot, slots + bad[kind], sizeof(slot), hipMemcpyDeviceToHost));
      const int64_t limit = static_cast<int64_t>(geom.num_blocks) * geom.block_size;
      return fail(PA_ERR_INVALID_ARG,
                  "row " + std::to_string(bad[kind]) + " names slot " + std::to_string(slot) +
                      (kind == 0 ? ", outside [0, " + std::to_string(limit) + ")"
                                 : ", which another row of the same call also names"));
    }
    return ok();
  }

  ~pa_pool() {
    if (slot_marks) {
      (void)hipDeviceSynchronize();
      (void)hipFree(slot_marks);
      (void)hipFree(check_result);
    }
    for (auto& st : ring) {
      if (st.pending) (void)hipEventSynchronize(st.ev);
      if (st.ev) (void)hipEventDestroy(st.ev);
      if (st.host) (void)hipHostFree(st.host);
    }
  }
};

namespace {

bool desc_ok(const pa_pool_desc* d, std::string* msg) {
  if (!d) {
    *msg = "NULL descriptor";
    return false;
  }
  if (d->num_blocks <= 0 || d->block_size <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0) {
    *msg = "num_blocks, block_size, num_kv_heads and head_dim must be positive";
    return false;
  }
  if (d->head_dim > 512) {
    *msg = "head_dim must be at most 512";
    return false;
  }
  if (d->dtype != PA_DTYPE_F32 && d->dtype != PA_DTYPE_BF16 && d->dtype != PA_DTYPE_I8 &&
      d->dtype != PA_DTYPE_FP8) {
    *msg = "dtype must be PA_DTYPE_F32, PA_DTYPE_BF16, PA_DTYPE_I8 or PA_DTYPE_FP8";
    return false;
  }
  if ((d->dtype == PA_DTYPE_I8 || d->dtype == PA_DTYPE_FP8) && (d->block_size % 16 || d->head_dim % 16)) {
    *msg = "PA_DTYPE_I8 and PA_DTYPE_FP8 need block_size and head_dim to be multiples of 16";
    return false;
  }
  return true;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Decode page-range size in tokens: 0 = chosen per batch by the plan;
// PA_DECODE_TOKENS_PER_PART in the environment fixes it (tuning override).
int32_t decode_tokens_per_part() {
  static const int32_t v = [] {
    const char* s = std::getenv("PA_DECODE_TOKENS_PER_PART");
    return s ? std::max(0, std::atoi(s)) : 0;
  }();
  return v;
}

float scale_log2_for(int32_t head_dim) {
  return static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(head_dim)));
}

}  // namespace

extern "C" {

size_t pa_pool_bytes(const pa_pool_desc* desc) {
  std::string msg;
  if (!desc_ok(desc, &msg)) return 0;
  const pa::PoolGeom geom{desc->num_blocks, desc->block_size, desc->num_kv_heads, desc->head_dim,
                         desc->dtype};
  return static_cast<size_t>(desc->num_blocks) * geom.block_bytes();
}

namespace {

// Pinned staging bytes reserved per ring buffer when a pool with device
// memory is created: 8 bytes per pool block (a plan holds one 4-byte table
// entry per page of the batch, plus 64-byte work items per page range) and
// 256 KiB for per-sequence data, at most 8 MiB.  A decode plan of a batch
// whose tables reference each block about once fits.
size_t default_staging_bytes(const pa::PoolGeom& g) {
  const size_t bytes = 8 * static_cast<size_t>(g.num_blocks) + (size_t{256} << 10);
  return std::min(bytes, size_t{8} << 20);
}

}  // namespace

pa_status pa_pool_create(const pa_pool_desc* desc, const int32_t* allocation_order, void* k_pool,
                         void* v_pool, pa_pool** out) {
  std::string msg;
  if (!out) return fail(PA_ERR_INVALID_ARG, "NULL out pointer");
  if (!desc_ok(desc, &msg)) return fail(PA_ERR_INVALID_ARG, msg);
  if ((k_pool == nullptr) != (v_pool == nullptr))
    return fail(PA_ERR_INVALID_ARG, "k_pool and v_pool must both be NULL or both be set");
  if ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) % 16)
    return fail(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  pa::BlockPool meta;
  pa::Status s = pa::BlockPool::make(desc->num_blocks, desc->block_size, allocation_order, &meta, &msg);
  if (s != pa::kOk) return fail(s, msg);
  pa_pool* p = new pa_pool();
  p->meta = std::move(meta);
  p->geom = {desc->num_blocks, desc->block_size, desc->num_kv_heads, desc->head_dim, desc->dtype};
  p->k = k_pool;
  p->v = v_pool;
  if (p->has_device()) {
    const pa_status r = p->reserve_staging(default_staging_bytes(p->geom));
    if (r != PA_OK) {
      const std::string why = g_err;
      delete p;
      return fail(r, why);
    }
  }
  *out = p;
  return ok();
}

pa_status pa_pool_reserve_staging(pa_pool* pool, size_t plan_bytes, size_t* reserved) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  if (!pool->has_device()) return fail(PA_ERR_INVALID_ARG, "metadata-only pool has no device memory");
  if (plan_bytes > (size_t{1} << 32)) return fail(PA_ERR_INVALID_ARG, "plan_bytes above 4 GiB");
  const pa_status r = pool->reserve_staging(plan_bytes);
  if (r != PA_OK) return r;
  if (reserved) *reserved = pool->staging_capacity();
  return ok();
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

pa_status pa_pool_set_slot_checks(pa_pool* pool, int on, void* stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  if (!pool->has_device()) return fail(PA_ERR_INVALID_ARG, "metadata-only pool has no device memory");
  return pool->set_slot_checks(on != 0, as_stream(stream));
}

pa_status pa_seq_create(pa_pool* pool, int64_t seq) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.create(seq, &msg), msg);
}

pa_status pa_append(pa_pool* pool, int64_t seq, int32_t n_tokens, int64_t* slots_out) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.append(seq, n_tokens, slots_out, &msg), msg);
}

pa_status pa_append_batch(pa_pool* pool, const int64_t* seqs, const int32_t* n_tokens,
                          int32_t count, int64_t* slots_out) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.append_batch(seqs, n_tokens, count, slots_out, &msg), msg);
}

pa_status pa_share(pa_pool* pool, int64_t src, int64_t dst, int32_t prefix_tokens) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.share(src, dst, prefix_tokens, &msg), msg);
}

pa_status pa_fork(pa_pool* pool, int64_t src, int64_t dst) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.fork(src, dst, &msg), msg);
}

pa_status pa_release(pa_pool* pool, int64_t seq) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.release(seq, &msg), msg);
}

pa_status pa_seq_set_window(pa_pool* pool, int64_t seq, int32_t sink_tokens, int32_t recent_tokens) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.set_window(seq, sink_tokens, recent_tokens, &msg), msg);
}

pa_status pa_truncate(pa_pool* pool, int64_t seq, int32_t new_length) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.truncate(seq, new_length, &msg), msg);
}

pa_status pa_prefix_lookup(const pa_pool* pool, const char* scope, const char* revision,
                           const int32_t* tokens, int32_t n_tokens, int32_t* hit_tokens) {
  if (!pool || !scope || !revision || !hit_tokens || n_tokens < 0 || (n_tokens > 0 && !tokens))
    return fail(PA_ERR_INVALID_ARG, "bad arguments");
  *hit_tokens = static_cast<int32_t>(pool->prefix.lookup(scope, revision, tokens, n_tokens));
  return ok();
}

pa_status pa_prefix_attach(pa_pool* pool, int64_t seq, const char* scope, const char* revision,
                           const int32_t* tokens, int32_t n_tokens, int32_t* hit_tokens) {
  if (!pool || !scope || !revision || !hit_tokens) return fail(PA_ERR_INVALID_ARG, "bad arguments");
  std::string msg;
  int64_t hit = 0;
  pa::Status s = pool->prefix.attach(pool->meta, seq, scope, revision, tokens, n_tokens, &hit, &msg);
  if (s == pa::kOk) *hit_tokens = static_cast<int32_t>(hit);
  return from(s, msg);
}

pa_status pa_prefix_register(pa_pool* pool, int64_t seq, const char* scope, const char* revision,
                             const int32_t* tokens, int32_t n_tokens, int32_t* added_blocks) {
  if (!pool || !scope || !revision) return fail(PA_ERR_INVALID_ARG, "bad arguments");
  std::string msg;
  int64_t added = 0;
  pa::Status s = pool->prefix.add(pool->meta, seq, scope, revision, tokens, n_tokens, &added, &msg);
  if (s == pa::kOk && added_blocks) *added_blocks = static_cast<int32_t>(added);
  return from(s, msg);
}

pa_status pa_prefix_clear(pa_pool* pool, int32_t* dropped_entries) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  const int64_t n = pool->prefix.clear(pool->meta);
  if (dropped_entries) *dropped_entries = static_cast<int32_t>(n);
  return ok();
}

pa_status pa_prefix_entries(const pa_pool* pool, int64_t* entries) {
  if (!pool || !entries) return fail(PA_ERR_INVALID_ARG, "bad arguments");
  *entries = pool->prefix.size();
  return ok();
}

pa_status pa_pending_copies(const pa_pool* pool, int32_t* pairs_out, int32_t cap, int32_t* n) {
  if (!pool || !n || cap < 0 || (cap > 0 && !pairs_out)) return fail(PA_ERR_INVALID_ARG, "bad arguments");
  const auto& pending = pool->meta.pending_copies();
  *n = static_cast<int32_t>(pending.size());
  for (int32_t i = 0; i < cap && i < *n; ++i) {
    pairs_out[2 * i] = pending[i].first;
    pairs_out[2 * i + 1] = pending[i].second;
  }
  return ok();
}

pa_status pa_flush_copies(pa_pool* pool, void* stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  return pool->flush(as_stream(stream));
}

pa_status pa_reshape_and_cache(pa_pool* pool, const void* k_new, const void* v_new,
                               const int64_t* slots, int32_t n, void* stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  if (!pool->has_device()) return fail(PA_ERR_INVALID_ARG, "metadata-only pool has no device memory");
  if (n < 0 || (n > 0 && (!k_new || !v_new || !slots)))
    return fail(PA_ERR_INVALID_ARG, "n must be >= 0 with non-NULL k_new, v_new, slots");
  hipStream_t s = as_stream(stream);
  if (pool->slot_marks && n > 0) {
    const pa_status c = pool->check_slots(slots, n, s);
    if (c != PA_OK) return c;
  }
  pa_status st = pool->flush(s);
  if (st != PA_OK) return st;
  if (n == 0) return ok();  // nothing to launch (and nothing to time)
  TimedLaunch t(PA_KERNEL_CACHE);
  hipError_t e = pa::launch_reshape_and_cache(pool->geom, pool->k, pool->v, k_new, v_new, slots, n, s,
                                              t.events());
  t.done(e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "reshape_and_cache launch");
  return ok();
}

size_t pa_decode_workspace_bytes(const pa_pool* pool, const int64_t* seqs, int32_t B, int32_t num_heads) {
  if (!pool) return 0;
  pa::DecodePlan plan;
  std::string msg;
  if (pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                            pool->geom.head_dim, decode_tokens_per_part(), nullptr, nullptr, 0, &plan,
                            &msg) != pa::kOk)
    return 0;
  return plan.total_bytes;
}

}  // extern "C"

namespace {

// Arguments every decode entry point checks.
pa_status check_decode_args(const pa_pool* pool, int32_t num_heads, const void* q, const void* out,
                            const void* ws) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  if (!pool->has_device()) return fail(PA_ERR_INVALID_ARG, "metadata-only pool has no device memory");
  if (!q || !out || !ws) return fail(PA_ERR_INVALID_ARG, "q, out and ws must be non-NULL");
  if (reinterpret_cast<uintptr_t>(ws) % pa::kWsAlign)
    return fail(PA_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  if (num_heads <= 0 || num_heads % pool->geom.num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_heads must be a positive multiple of num_kv_heads");
  if (pool->geom.dtype != PA_DTYPE_F32 &&
      (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) % 16)
    return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  return ok();
}

// Decode partial kernel (+ merge) over a plan already on its way into `ws`.
pa_status launch_decode_plan(pa_pool* pool, const pa::DecodePlan& plan, int32_t B, int32_t num_heads,
                             const void* q, void* out, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  pa::DecodeArgs a{};
  a.k_pool = pool->k;
  a.v_pool = pool->v;
  a.q = q;
  a.out = out;
  a.ctx_len = reinterpret_cast<const int32_t*>(w + plan.ctx_off);
  a.tbl_off = reinterpret_cast<const int32_t*>(w + plan.tbl_off_off);
  a.tables = reinterpret_cast<const int32_t*>(w + plan.tables_off);
  a.work = reinterpret_cast<const int32_t*>(w + plan.work_off);
  a.part_base = reinterpret_cast<const int32_t*>(w + plan.base_off);
  a.part_m = reinterpret_cast<float*>(w + plan.part_m_off);
  a.part_l = reinterpret_cast<float*>(w + plan.part_l_off);
  a.part_acc = reinterpret_cast<float*>(w + plan.part_acc_off);
  a.q_start = reinterpret_cast<const int32_t*>(w + plan.qstart_off);
  a.merge_rows = reinterpret_cast<const int32_t*>(w + plan.merge_off);
  a.seq_win = reinterpret_cast<const int32_t*>(w + plan.win_off);
  a.n_parts_of = reinterpret_cast<const int32_t*>(w + plan.nparts_off);
  a.batch = B;
  a.num_heads = num_heads;
  a.num_kv_heads = pool->geom.num_kv_heads;
  a.group = num_heads / pool->geom.num_kv_heads;
  a.pages_per_part = plan.pages_per_part;
  a.n_work = plan.n_work;
  a.n_merge = plan.n_merge;
  a.max_cols = plan.max_q_len * a.group;
  a.scale_log2 = scale_log2_for(pool->geom.head_dim);
  {
    TimedLaunch t(PA_KERNEL_DECODE);
    hipError_t e = pa::launch_decode_partial(pool->geom, a, st, t.events());
    t.done(e == hipSuccess);
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  }
  if (a.n_merge > 0 && pa::decode_needs_merge_kernel(pool->geom, a.group)) {
    TimedLaunch t(PA_KERNEL_MERGE);
    hipError_t e = pa::launch_decode_merge(pool->geom, a, st, t.events());
    t.done(e == hipSuccess);
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return ok();
}

// Tokens each batch row will have gained after the step's appends of
// n_tokens[b] (1 each when NULL) tokens: a sequence listed twice gains both.
std::vector<int32_t> step_extra_tokens(const int64_t* seqs, const int32_t* n_tokens, int32_t B) {
  std::unordered_map<int64_t, int64_t> count;
  for (int32_t b = 0; b < B; ++b) count[seqs[b]] += n_tokens ? std::max(n_tokens[b], 0) : 1;
  std::vector<int32_t> extra(B);
  for (int32_t b = 0; b < B; ++b) extra[b] = static_cast<int32_t>(std::min<int64_t>(count[seqs[b]], INT32_MAX));
  return extra;
}

}  // namespace

namespace pa {

pa_status fail_status(pa_status status, const std::string& msg) { return fail(status, msg); }

pa_status fused_step(pa_pool* pool, const int64_t* seqs, const int32_t* n_tokens, int32_t B,
                     int32_t num_heads, const void* k_new, const void* v_new, const void* q, void* out,
                     const StepWorkspace& wsp, int64_t* slots_out, void* stream) {
  void* ws = wsp.ptr;
  const size_t ws_bytes = wsp.bytes;
  pa_status r = check_decode_args(pool, num_heads, q, out, ws);
  if (r != PA_OK) return r;
  if (!k_new || !v_new) return fail(PA_ERR_INVALID_ARG, "k_new and v_new must be non-NULL");
  if (B <= 0 || !seqs) return fail(PA_ERR_INVALID_ARG, "batch must be positive with a non-NULL seqs array");
  int64_t rows = B;
  int32_t max_q = 1;
  if (n_tokens) {
    std::unordered_map<int64_t, int32_t> seen;
    rows = 0;
    for (int32_t b = 0; b < B; ++b) {
      if (n_tokens[b] < 1) return fail(PA_ERR_INVALID_ARG, "q_lens[b] must be >= 1");
      if (seen[seqs[b]]++) return fail(PA_ERR_INVALID_ARG, "a sequence appears twice in a verify step");
      rows += n_tokens[b];
      max_q = std::max(max_q, n_tokens[b]);
    }
    if (rows > INT32_MAX / 2) return fail(PA_ERR_INVALID_ARG, "too many query rows");
    const int32_t group = num_heads / pool->geom.num_kv_heads;
    if (!pa::decode_handles_rows(pool->geom, group, max_q))
      return fail(PA_ERR_INVALID_ARG,
                  "verify step needs an MFMA decode shape (bf16 or 8-bit pages, head_dim 64/128, "
                  "block_size 16/32) and q_len * group <= 32");
  }
  std::string msg;
  // Size and validate against the lengths after the append, before anything changes.
  std::vector<int32_t> extra = step_extra_tokens(seqs, n_tokens, B);
  pa::DecodePlan sizing;
  pa::Status s = pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                                       pool->geom.head_dim, decode_tokens_per_part(), extra.data(),
                                       n_tokens, static_cast<int32_t>(rows), &sizing, &msg);
  if (s != pa::kOk) return fail(s, msg);
  if (ws_bytes < sizing.total_bytes) {
    if (wsp.static_scratch)
      return fail(PA_ERR_INVALID_ARG, "the step needs " + std::to_string(sizing.total_bytes) +
                                          " bytes of workspace, more than the " + std::to_string(ws_bytes) +
                                          " bytes of the static scratch");
    return fail(PA_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(sizing.total_bytes) +
                                        " bytes, got " + std::to_string(ws_bytes));
  }
  if (wsp.static_scratch && sizing.meta_bytes > pool->staging_capacity())
    return fail(PA_ERR_INVALID_ARG, "the step's plan of " + std::to_string(sizing.meta_bytes) +
                                        " bytes exceeds the pool's reserved staging buffers (" +
                                        std::to_string(pool->staging_capacity()) +
                                        " bytes; see pa_pool_reserve_staging)");
  pa::DecodePlan& plan = pool->plan;
  std::vector<int32_t> ones;
  if (!n_tokens) ones.assign(B, 1);
  std::vector<int64_t> slots(rows);
  s = pool->meta.append_batch(seqs, n_tokens ? n_tokens : ones.data(), B, slots.data(), &msg);
  if (s != pa::kOk) return fail(s, msg);
  // Same lengths as the sizing plan, so the same layout and size.
  s = pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                            pool->geom.head_dim, decode_tokens_per_part(), nullptr, n_tokens,
                            static_cast<int32_t>(rows), &plan, &msg);
  if (s != pa::kOk) return fail(s, msg);
  std::memcpy(reinterpret_cast<char*>(plan.meta.data()) + plan.slots_off, slots.data(),
              sizeof(int64_t) * rows);
  if (slots_out) std::memcpy(slots_out, slots.data(), sizeof(int64_t) * rows);
  hipStream_t st = as_stream(stream);
  r = pool->flush(st);  // copy-on-write copies of this append come first
  if (r != PA_OK) return r;
  const void* staged = nullptr;
  const size_t bytes = plan.meta.size() * sizeof(int32_t);
  r = pool->stage(plan.meta.data(), bytes, &staged, !wsp.static_scratch);
  if (r != PA_OK) return r;
  {
    TimedLaunch t(PA_KERNEL_CACHE);
    hipError_t e = pa::launch_step_prep(
        pool->geom, staged, ws, pa::align_up(bytes, 16),
        reinterpret_cast<const int64_t*>(static_cast<const char*>(staged) + plan.slots_off), pool->k,
        pool->v, k_new, v_new, static_cast<int32_t>(rows), st, t.events());
    t.done(e == hipSuccess);
    if (e != hipSuccess) return hip_fail(e, "decode step prologue launch");
  }
  pa_pool::StagedUse use;
  use.pool = pool;
  use.stream = st;
  return launch_decode_plan(pool, plan, B, num_heads, q, out, ws, st);
}

}  // namespace pa

namespace {

// Whether a prefill chunk goes through the split-K decode kernels (every
// q_len small enough for one workgroup's query columns).
bool prefill_via_decode(const pa_pool* pool, const int32_t* q_lens, int32_t B, int32_t num_heads) {
  if (!q_lens || B <= 0 || num_heads <= 0 || num_heads % pool->geom.num_kv_heads) return false;
  int32_t max_q = 0;
  for (int32_t b = 0; b < B; ++b) max_q = std::max(max_q, q_lens[b]);
  return max_q >= 1 && pa::decode_handles_rows(pool->geom, num_heads / pool->geom.num_kv_heads, max_q);
}

}  // namespace

extern "C" {

pa_status pa_decode(pa_pool* pool, const int64_t* seqs, int32_t B, int32_t num_heads, const void* q,
                    void* out, void* ws, size_t ws_bytes, void* stream) {
  pa_status r = check_decode_args(pool, num_heads, q, out, ws);
  if (r != PA_OK) return r;
  pa::DecodePlan& plan = pool->plan;
  std::string msg;
  pa::Status s = pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                                       pool->geom.head_dim, decode_tokens_per_part(), nullptr, nullptr,
                                       0, &plan, &msg);
  if (s != pa::kOk) return fail(s, msg);
  if (ws_bytes < plan.total_bytes)
    return fail(PA_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(plan.total_bytes) +
                                        " bytes, got " + std::to_string(ws_bytes));
  hipStream_t st = as_stream(stream);
  r = pool->flush(st);
  if (r != PA_OK) return r;
  pa_pool::StagedUse use;
  r = pool->upload(plan.meta.data(), plan.meta.size() * sizeof(int32_t), ws, st, &use);
  if (r != PA_OK) return r;
  return launch_decode_plan(pool, plan, B, num_heads, q, out, ws, st);
}

size_t pa_decode_step_workspace_bytes(const pa_pool* pool, const int64_t* seqs, int32_t B,
                                      int32_t num_heads) {
  if (!pool || B <= 0 || !seqs) return 0;
  std::vector<int32_t> extra = step_extra_tokens(seqs, nullptr, B);
  pa::DecodePlan plan;
  std::string msg;
  if (pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                            pool->geom.head_dim, decode_tokens_per_part(), extra.data(), nullptr, B,
                            &plan, &msg) != pa::kOk)
    return 0;
  return plan.total_bytes;
}

pa_status pa_decode_step(pa_pool* pool, const int64_t* seqs, int32_t B, int32_t num_heads,
                         const void* k_new, const void* v_new, const void* q, void* out, void* ws,
                         size_t ws_bytes, int64_t* slots_out, void* stream) {
  return pa::fused_step(pool, seqs, nullptr, B, num_heads, k_new, v_new, q, out, {ws, ws_bytes, false},
                        slots_out, stream);
}

size_t pa_verify_step_workspace_bytes(const pa_pool* pool, const int64_t* seqs, const int32_t* q_lens,
                                      int32_t B, int32_t num_heads) {
  if (!pool || B <= 0 || !seqs || !q_lens) return 0;
  int64_t rows = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (q_lens[b] < 1) return 0;
    rows += q_lens[b];
  }
  if (rows > INT32_MAX / 2) return 0;
  std::vector<int32_t> extra = step_extra_tokens(seqs, q_lens, B);
  pa::DecodePlan plan;
  std::string msg;
  if (pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                            pool->geom.head_dim, decode_tokens_per_part(), extra.data(), q_lens,
                            static_cast<int32_t>(rows), &plan, &msg) != pa::kOk)
    return 0;
  return plan.total_bytes;
}

pa_status pa_verify_step(pa_pool* pool, const int64_t* seqs, const int32_t* q_lens, int32_t B,
                         int32_t num_heads, const void* k_new, const void* v_new, const void* q, void* out,
                         void* ws, size_t ws_bytes, int64_t* slots_out, void* stream) {
  if (!q_lens) return fail(PA_ERR_INVALID_ARG, "q_lens must be non-NULL");
  return pa::fused_step(pool, seqs, q_lens, B, num_heads, k_new, v_new, q, out, {ws, ws_bytes, false},
                        slots_out, stream);
}

size_t pa_prefill_workspace_bytes(const pa_pool* pool, const int64_t* seqs, const int32_t* q_lens,
                                  int32_t B, int32_t num_heads) {
  if (!pool || num_heads <= 0 || num_heads % pool->geom.num_kv_heads) return 0;
  std::string msg;
  if (prefill_via_decode(pool, q_lens, B, num_heads)) {
    pa::DecodePlan dplan;
    if (pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                              pool->geom.head_dim, decode_tokens_per_part(), nullptr, q_lens, 0, &dplan,
                              &msg) != pa::kOk)
      return 0;
    return dplan.total_bytes;
  }
  pa::PrefillPlan plan;
  const int32_t group = num_heads / pool->geom.num_kv_heads;
  if (pa::build_prefill_plan(pool->meta, seqs, q_lens, B, num_heads, pool->geom.num_kv_heads,
                             pa::prefill_rows_per_tile(pool->geom, group), &plan, &msg) != pa::kOk)
    return 0;
  return plan.total_bytes;
}

pa_status pa_prefill_chunk(pa_pool* pool, const int64_t* seqs, const int32_t* q_lens, int32_t B,
                           int32_t num_heads, const void* q, void* out, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  if (!pool->has_device()) return fail(PA_ERR_INVALID_ARG, "metadata-only pool has no device memory");
  if (!q || !out || !ws) return fail(PA_ERR_INVALID_ARG, "q, out and ws must be non-NULL");
  if (reinterpret_cast<uintptr_t>(ws) % pa::kWsAlign)
    return fail(PA_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  if (num_heads <= 0 || num_heads % pool->geom.num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_heads must be a positive multiple of num_kv_heads");
  if (pool->geom.dtype != PA_DTYPE_F32 &&
      (reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) % 16)
    return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  const int32_t group = num_heads / pool->geom.num_kv_heads;
  std::string msg;
  if (prefill_via_decode(pool, q_lens, B, num_heads)) {
    // Short chunks (q_len * group <= 32): the split-K decode kernels, all
    // query rows of a sequence as MFMA columns of each K/V page.
    pa::DecodePlan dplan;
    pa::Status ds = pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                                          pool->geom.head_dim, decode_tokens_per_part(), nullptr, q_lens,
                                          0, &dplan, &msg);
    if (ds != pa::kOk) return fail(ds, msg);
    if (ws_bytes < dplan.total_bytes)
      return fail(PA_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(dplan.total_bytes) +
                                          " bytes, got " + std::to_string(ws_bytes));
    hipStream_t st = as_stream(stream);
    pa_status r = pool->flush(st);
    if (r != PA_OK) return r;
    pa_pool::StagedUse use;
    r = pool->upload(dplan.meta.data(), dplan.meta.size() * sizeof(int32_t), ws, st, &use);
    if (r != PA_OK) return r;
    return launch_decode_plan(pool, dplan, B, num_heads, q, out, ws, st);
  }
  pa::PrefillPlan plan;
  pa::Status s = pa::build_prefill_plan(pool->meta, seqs, q_lens, B, num_heads, pool->geom.num_kv_heads,
                                        pa::prefill_rows_per_tile(pool->geom, group), &plan, &msg);
  if (s != pa::kOk) return fail(s, msg);
  if (ws_bytes < plan.total_bytes)
    return fail(PA_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(plan.total_bytes) +
                                        " bytes, got " + std::to_string(ws_bytes));
  hipStream_t st = as_stream(stream);
  pa_status r = pool->flush(st);
  if (r != PA_OK) return r;
  pa_pool::StagedUse use;
  r = pool->upload(plan.meta.data(), plan.meta.size() * sizeof(int32_t), ws, st, &use);
  if (r != PA_OK) return r;
  char* w = static_cast<char*>(ws);
  pa::PrefillArgs a{};
  a.k_pool = pool->k;
  a.v_pool = pool->v;
  a.q = q;
  a.out = out;
  a.ctx_len = reinterpret_cast<const int32_t*>(w + plan.ctx_off);
  a.tbl_off = reinterpret_cast<const int32_t*>(w + plan.tbl_off_off);
  a.tables = reinterpret_cast<const int32_t*>(w + plan.tables_off);
  a.q_start = reinterpret_cast<const int32_t*>(w + plan.qstart_off);
  a.tiles = reinterpret_cast<const int32_t*>(w + plan.tiles_off);
  a.row_seq = reinterpret_cast<const int32_t*>(w + plan.rowseq_off);
  a.zeros = w + plan.zeros_off;
  a.seq_win = reinterpret_cast<const int32_t*>(w + plan.win_off);
  a.num_heads = num_heads;
  a.num_kv_heads = pool->geom.num_kv_heads;
  a.group = group;
  a.n_tiles = plan.n_tiles;
  a.n_rows = plan.n_rows;
  a.scale_log2 = scale_log2_for(pool->geom.head_dim);
  TimedLaunch t(PA_KERNEL_PREFILL);
  hipError_t e = pa::launch_prefill(pool->geom, a, st, t.events());
  t.done(e == hipSuccess);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

pa_status pa_seq_len(const pa_pool* pool, int64_t seq, int32_t* len) {
  if (!pool || !len) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  const pa::Sequence* s = pool->meta.find(seq);
  if (!s) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence: " + std::to_string(seq));
  *len = static_cast<int32_t>(s->length);
  return ok();
}

pa_status pa_block_table(const pa_pool* pool, int64_t seq, int32_t* out, int32_t cap, int32_t* n) {
  if (!pool || !n || cap < 0 || (cap > 0 && !out)) return fail(PA_ERR_INVALID_ARG, "bad arguments");
  const pa::Sequence* s = pool->meta.find(seq);
  if (!s) return fail(PA_ERR_UNKNOWN_SEQ, "unknown sequence: " + std::to_string(seq));
  *n = static_cast<int32_t>(s->table.size());
  for (int32_t i = 0; i < cap && i < *n; ++i) out[i] = s->table[i];
  return ok();
}

pa_status pa_refcount(const pa_pool* pool, int32_t block, int32_t* rc) {
  if (!pool || !rc || block < 0 || block >= pool->meta.num_blocks())
    return fail(PA_ERR_INVALID_ARG, "bad block id or NULL argument");
  *rc = pool->meta.refcount(block);
  return ok();
}

pa_status pa_stats(const pa_pool* pool, pa_pool_stats* stats) {
  if (!pool || !stats) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  pa::PoolStats s = pool->meta.stats();
  stats->allocated_blocks = s.allocated_blocks;
  stats->free_blocks = s.free_blocks;
  stats->physical_capacity_tokens = s.physical_capacity_tokens;
  stats->physical_payload_tokens = s.physical_payload_tokens;
  stats->logical_tokens = s.logical_tokens;
  stats->internal_waste_tokens = s.internal_waste_tokens;
  stats->sharing_savings_tokens = s.sharing_savings_tokens;
  return ok();
}

pa_status pa_validate(const pa_pool* pool) {
  if (!pool) return fail(PA_ERR_INVALID_ARG, "NULL pool");
  std::string msg;
  return from(pool->meta.validate(&msg), msg);
}

pa_status pa_decode_work_items(const pa_pool* pool, const int64_t* seqs, const int32_t* q_lens, int32_t B,
                               int32_t num_heads, int32_t* pages_per_range, int32_t* items, int32_t cap_items,
                               int32_t* n_items, int32_t* tables, int64_t cap_tables, int64_t* n_tables) {
  if (!pool || !pages_per_range || !n_items || !n_tables || cap_items < 0 || cap_tables < 0 ||
      (cap_items > 0 && !items) || (cap_tables > 0 && !tables))
    return fail(PA_ERR_INVALID_ARG, "bad arguments");
  pa::DecodePlan plan;
  std::string msg;
  const pa::Status s = pa::build_decode_plan(pool->meta, seqs, B, num_heads, pool->geom.num_kv_heads,
                                             pool->geom.head_dim, decode_tokens_per_part(), nullptr, q_lens, 0,
                                             &plan, &msg);
  if (s != pa::kOk) return fail(s, msg);
  const int32_t* meta = plan.meta.data();
  *pages_per_range = plan.pages_per_part;
  *n_items = plan.n_work;
  const int32_t* work = meta + plan.work_off / sizeof(int32_t);
  std::copy(work, work + pa::kWorkInts * static_cast<size_t>(std::min(cap_items, plan.n_work)), items);
  // The tables section runs to the slots section (4-word padding aside).
  const int32_t* toff = meta + plan.tbl_off_off / sizeof(int32_t);
  const int32_t* ctx = meta + plan.ctx_off / sizeof(int32_t);
  const int32_t* win = meta + plan.win_off / sizeof(int32_t);
  int64_t visited = 0;
  for (int32_t b = 0; b < B; ++b) {
    const int64_t nblk = (ctx[b] + pool->geom.block_size - 1) / pool->geom.block_size;
    visited = std::max<int64_t>(visited, toff[b] + nblk - win[4 * static_cast<size_t>(b) + 3]);
  }
  *n_tables = visited;
  const int32_t* tab = meta + plan.tables_off / sizeof(int32_t);
  std::copy(tab, tab + std::min(cap_tables, visited), tables);
  return ok();
}

pa_status pa_sequences(const pa_pool* pool, int64_t* ids_out, int32_t cap, int32_t* n) {
  if (!pool || !n || cap < 0 || (cap > 0 && !ids_out)) return fail(PA_ERR_INVALID_ARG, "bad arguments");
  std::vector<int64_t> ids = pool->meta.sequence_ids();
  *n = static_cast<int32_t>(ids.size());
  for (int32_t i = 0; i < cap && i < *n; ++i) ids_out[i] = ids[i];
  return ok();
}

const char* pa_last_error(void) { return g_err.c_str(); }

pa_status pa_timing_enable(int on) {
  std::lock_guard<std::mutex> lock(g_tmu);
  g_timing = on != 0;
  return ok();
}

pa_status pa_timing_select(uint32_t kernel_mask) {
  std::lock_guard<std::mutex> lock(g_tmu);
  g_timing_mask = kernel_mask;
  return ok();
}

pa_status pa_timing_reset(void) {
  std::lock_guard<std::mutex> lock(g_tmu);
  drain_timing_locked();
  for (int k = 0; k < PA_KERNEL_COUNT; ++k) {
    g_total_ms[k] = 0.0;
    g_launches[k] = 0;
    g_samples[k].clear();
  }
  return ok();
}

pa_status pa_timing_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= PA_KERNEL_COUNT || !total_ms || !launches)
    return fail(PA_ERR_INVALID_ARG, "bad kernel id or NULL argument");
  std::lock_guard<std::mutex> lock(g_tmu);
  drain_timing_locked();
  *total_ms = g_total_ms[kernel];
  *launches = g_launches[kernel];
  return ok();
}

pa_status pa_timing_samples(int32_t kernel, float* ms_out, int64_t cap, int64_t* n) {
  if (kernel < 0 || kernel >= PA_KERNEL_COUNT || !n || cap < 0 || (cap > 0 && !ms_out))
    return fail(PA_ERR_INVALID_ARG, "bad kernel id, cap or NULL argument");
  std::lock_guard<std::mutex> lock(g_tmu);
  drain_timing_locked();
  const std::vector<float>& s = g_samples[kernel];
  *n = static_cast<int64_t>(s.size());
  const size_t m = std::min<size_t>(s.size(), static_cast<size_t>(cap));
  std::copy(s.begin(), s.begin() + m, ms_out);
  return ok();
}

}  // extern "C"
