// Chunked causal prefill over the paged pool.
//
// What is computed (docs.rs ferrum-kv 0.4.0 src/attention.rs,
// paged_attention with q_tokens > 1): the q_len query rows of a sequence are
// its last q_len positions; row t sees keys j <= kv_len - q_len + t
// (bottom-right causal alignment, as CMU 11-667 lecture 19's CachedDecoder
// masks cached decoding).
//
// prefill_gqa_mfma<D, BS, CG>  (bf16, D in {64, 128}, BS in {16, 32}, G | 16)
//   One 256-thread workgroup = (sequence, block of query rows, KV head).  The
//   N dimension of the MFMA tiles packs (query row, head of the group) pairs:
//   column c of the workgroup is row t0 + c / G, head g*G + c % G, so every
//   K/V page read serves all G query heads of the KV head.  Each wave owns
//   CG groups of 16 columns and streams the pages its rows can see:
//     S^T[16 tok x 16 col]  = K_page . Q^T          (v_mfma_f32_16x16x32_bf16)
//     O^T[16 d   x 16 col] += V^T_page . P^T (hi+lo) (v_mfma_f32_16x16x16_bf16)
//   as in the decode kernel (the S^T accumulator layout is the P^T operand
//   layout).  Pages wholly below every row's limit need no mask; pages past
//   the wave's last row's limit are skipped; only diagonal pages are masked.
//   blockIdx % Hkv is the KV head, so with Hkv a multiple of 8 each XCD (and
//   its L2) serves one KV head of every sequence: a shared prefix is read
//   from HBM once per head and then hits in that XCD's L2.
#include <cmath>

#include "device.hpp"
#include "kernels.hpp"

namespace pa {

hipError_t launch_prefill_generic(const PoolGeom& geom, const PrefillArgs& a, hipStream_t stream);

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kPrefillWaves = 4;
constexpr int kPrefillCG = 2;  // 16-column groups per wave

template <int D, int BS, int CG>
__global__ __launch_bounds__(256) void prefill_gqa_mfma(PrefillArgs a) {
  constexpr int KS = D / 32;
  constexpr int TT = BS / 16;
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int Hkv = a.num_kv_heads, Hq = a.num_heads, G = a.group;
  const int tile = blockIdx.x / Hkv, g = blockIdx.x - tile * Hkv;
  const int b = a.tiles[2 * tile], t0 = a.tiles[2 * tile + 1];
  const int q0 = a.q_start[b];
  const int q_len = a.q_start[b + 1] - q0;
  const int L = a.ctx_len[b];
  const int off = L - q_len;  // row t sees keys 0 .. off + t
  const int32_t* table = a.tables + a.tbl_off[b];
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  const size_t page = static_cast<size_t>(BS) * D;

  const int wave_c0 = wave * CG * 16;
  const int t_first = t0 + wave_c0 / G;
  if (t_first >= q_len) return;  // ragged last row block: no rows for this wave
  const int t_last = min(q_len - 1, t0 + (wave_c0 + CG * 16 - 1) / G);
  const int last_key = off + t_last;       // largest key any column of the wave sees
  const int all_see = off + t_first;       // keys <= all_see are visible to every column
  const int n_pages = last_key / BS + 1;

  // This lane's column in each group, its row limit, and its Q^T operand.
  bf16x8 qv[CG][KS];
  int lim[CG], row[CG], head[CG];
#pragma unroll
  for (int k = 0; k < CG; ++k) {
    const int c = wave_c0 + k * 16 + n;
    row[k] = t0 + c / G;
    head[k] = g * G + c % G;
    // A column past the last row (ragged row block) is computed with the last
    // row's limit, so it stays finite, and is never stored.
    lim[k] = off + min(row[k], q_len - 1);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(q0 + row[k]) * Hq + head[k]) * D + 8 * grp;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (row[k] < q_len)
        qv[k][j] = *reinterpret_cast<const bf16x8*>(qrow + 32 * j);
      else
        qv[k][j] = bf16x8{};
    }
  }

  float m_run[CG], l_run[CG];
  f32x4 acc[CG][DT];
#pragma unroll
  for (int k = 0; k < CG; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) acc[k][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto load_page = [&](int pg, bf16x8 (&kr)[TT][KS], s16x4 (&vr)[DT][TT]) {
    const int blk = uniform(table[pg]);
    const uint16_t* kp = kpool + (static_cast<size_t>(blk) * Hkv + g) * page;
    const uint16_t* vp = vpool + (static_cast<size_t>(blk) * Hkv + g) * page;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int j = 0; j < KS; ++j)
        kr[tt][j] = *reinterpret_cast<const bf16x8*>(kp + (16 * tt + n) * D + 32 * j + 8 * grp);
#pragma unroll
    for (int nt = 0; nt < DT; ++nt)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        vr[nt][tt] = *reinterpret_cast<const s16x4*>(vp + (16 * nt + n) * BS + 16 * tt + 4 * grp);
  };

  auto process = [&](int pg, const bf16x8 (&kr)[TT][KS], const s16x4 (&vr)[DT][TT]) {
    const bool masked = pg * BS + BS - 1 > all_see;
#pragma unroll
    for (int k = 0; k < CG; ++k) {
      f32x4 s[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j)
          s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[tt][j], qv[k][j], s[tt], 0, 0, 0);
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[tt][i] * a.scale_log2;
          if (masked && pg * BS + 16 * tt + 4 * grp + i > lim[k]) x = -INFINITY;
          s[tt][i] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      // Every column sees key 0 on page 0, so m_run is finite from then on.
      const float m_new = fmaxf(m_run[k], mloc);
      const float alpha = exp2f(m_run[k] - m_new);
      m_run[k] = m_new;
      float psum = 0.f;
      s16x4 p_hi[TT], p_lo[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2f(s[tt][i] - m_new);
          const __bf16 hi = static_cast<__bf16>(e);
          const __bf16 lo = static_cast<__bf16>(e - static_cast<float>(hi));
          psum += e;
          p_hi[tt][i] = __builtin_bit_cast(short, hi);
          p_lo[tt][i] = __builtin_bit_cast(short, lo);
        }
      l_run[k] = l_run[k] * alpha + psum;
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) {
        acc[k][nt] *= alpha;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          acc[k][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[nt][tt], p_hi[tt], acc[k][nt], 0, 0, 0);
          acc[k][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[nt][tt], p_lo[tt], acc[k][nt], 0, 0, 0);
        }
      }
    }
  };

  {
    bf16x8 ka[TT][KS], kb[TT][KS];
    s16x4 va[DT][TT], vb[DT][TT];
    int p = 0;
    load_page(p, ka, va);
    while (p < n_pages) {
      if (p + 1 < n_pages) load_page(p + 1, kb, vb);
      process(p, ka, va);
      ++p;
      if (p >= n_pages) break;
      if (p + 1 < n_pages) load_page(p + 1, ka, va);
      process(p, kb, vb);
      ++p;
    }
  }

  // Normalise and store: lane (n, grp) holds d = 16nt + 4grp + i of its column.
#pragma unroll
  for (int k = 0; k < CG; ++k) {
    float l = l_run[k] + __shfl_xor(l_run[k], 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (row[k] >= q_len) continue;
    const float inv = 1.f / l;
    uint16_t* o = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(q0 + row[k]) * Hq + head[k]) * D;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      uint2 packed;
      packed.x = static_cast<uint32_t>(f32_to_bf16(acc[k][nt][0] * inv)) |
                 (static_cast<uint32_t>(f32_to_bf16(acc[k][nt][1] * inv)) << 16);
      packed.y = static_cast<uint32_t>(f32_to_bf16(acc[k][nt][2] * inv)) |
                 (static_cast<uint32_t>(f32_to_bf16(acc[k][nt][3] * inv)) << 16);
      *reinterpret_cast<uint2*>(o + 16 * nt + 4 * grp) = packed;
    }
  }
}

template <int D, int BS>
void launch_mfma(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid(a.n_tiles * a.num_kv_heads);
  hipLaunchKernelGGL((prefill_gqa_mfma<D, BS, kPrefillCG>), grid, dim3(64 * kPrefillWaves), 0, stream, a);
}

}  // namespace

bool prefill_uses_mfma(const PoolGeom& geom, int32_t group) {
  const bool d_ok = geom.head_dim == 64 || geom.head_dim == 128;
  const bool bs_ok = geom.block_size == 16 || geom.block_size == 32;
  const bool g_ok = group >= 1 && group <= 16 && 16 % group == 0;
  return geom.dtype == 1 && d_ok && bs_ok && g_ok;
}

int32_t prefill_rows_per_tile(const PoolGeom& geom, int32_t group) {
  if (!prefill_uses_mfma(geom, group)) return 64;
  return kPrefillWaves * kPrefillCG * 16 / group;
}

hipError_t launch_prefill(const PoolGeom& geom, const PrefillArgs& a, hipStream_t stream) {
  if (!prefill_uses_mfma(geom, a.group)) return launch_prefill_generic(geom, a, stream);
  const int D = geom.head_dim, BS = geom.block_size;
  if (D == 128 && BS == 16) launch_mfma<128, 16>(a, stream);
  else if (D == 128 && BS == 32) launch_mfma<128, 32>(a, stream);
  else if (D == 64 && BS == 16) launch_mfma<64, 16>(a, stream);
  else launch_mfma<64, 32>(a, stream);
  return hipGetLastError();
}

}  // namespace pa
