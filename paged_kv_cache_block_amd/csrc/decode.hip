// Paged decode attention for gfx950.
//
// What is computed (docs.rs ferrum-kv 0.4.0 src/attention.rs,
// paged_attention; abhik.ai "examples/pagedattention.py", region
// paged_attention): for sequence b of length L with q_len query rows (its
// last q_len positions; q_len = 1 for decode), row t, query head h, KV head
// g = h / G: scores s_j = q . K_j / sqrt(D) over the cached tokens
// j <= L - q_len + t, softmax, output sum_j p_j V_j, with K_j / V_j found
// through the block table.
//
// Kernels
//   decode_mfma      bf16 or 8-bit pages, D in {64, 128}, block_size in
//       {16, 32}, G <= 16, q_len * G <= 32 query columns per sequence.
//       One workgroup = (work item = (sequence, page range), KV head); its 4
//       waves stride over the pages of the range.  The query rows x heads of
//       the KV head form the N dimension of two MFMA contractions per page
//       (S^T = K . Q^T, then O^T += V^T . P^T, P kept in registers); the
//       transposed (bf16) or operand-ordered (8-bit) V page makes every V
//       operand a contiguous load.  Online softmax per page (exp2 with
//       log2(e) folded into the scale); the 4 waves merge in LDS; a range
//       that is the whole sequence writes bf16 output, otherwise fp32
//       partials (m, l, acc) for the merge kernel.
//   decode_merge     log-sum-exp combination of the partials of one
//       (query row, head): M = max m_c, o = sum e^(m_c-M) acc_c / sum e^(m_c-M) l_c
//       (CMU 11-667 lecture 19 section 3, online_softmax_stats, applied
//       across page ranges).
//   attn_generic     any dtype / head_dim <= 512 / block_size / group; one
//       wave per (query row, head), 64 keys per step, online softmax.  Used
//       for fp32 pools and shapes the MFMA kernel does not cover; it also
//       serves prefill rows (bottom-right causal mask).
#include <cmath>
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"

// Tile parameters (compile-time; variant builds override them with -D).
#ifndef PA_DECODE_WAVES_I8
#define PA_DECODE_WAVES_I8 3
#endif
#ifndef PA_DECODE_PERMLANE
#define PA_DECODE_PERMLANE 1  // cross-group reductions with permlane swaps (not LDS)
#endif
#ifndef PA_DECODE_TABLE_AHEAD
#define PA_DECODE_TABLE_AHEAD 1  // load each block id one page step before its page
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 1  // pages each wave loads ahead of the page it computes
#endif

namespace pa {

namespace {


// --------------------------------------------------------------- generic ---
struct GenericArgs {
  const void* k_pool;
  const void* v_pool;
  const void* q;
  void* out;
  const int32_t* ctx_len;
  const int32_t* tbl_off;
  const int32_t* tables;
  const int32_t* q_start;  // nullptr: decode, row r is sequence r with q_len 1
  const int32_t* row_seq;
  const int32_t* seq_win;  // [B][4]: sinks, recent (nullptr: no windows)
  int32_t num_heads, num_kv_heads, group, head_dim, block_size;
  float scale_log2;
};

// Q8: pages of 8-bit codes + fp32 row scales (1: int8, 2: E4M3; q / out
// bf16); T is the q / out element type.
template <typename T, int Q8>
__global__ __launch_bounds__(64) void attn_generic(GenericArgs a) {
  extern __shared__ float smem[];
  float* qs = smem;                                            // [D]
  float* ps = smem + a.head_dim;                               // [64]
  int* blks = reinterpret_cast<int*>(ps + 64);                 // [64]
  int* offs = blks + 64;                                       // [64]
  const int lane = threadIdx.x;
  const int r = blockIdx.x / a.num_heads, h = blockIdx.x - r * a.num_heads;
  int b, t, q_len;
  if (a.q_start) {
    b = a.row_seq[r];
    t = r - a.q_start[b];
    q_len = a.q_start[b + 1] - a.q_start[b];
  } else {
    b = r;
    t = 0;
    q_len = 1;
  }
  const int L = a.ctx_len[b];
  const int visible = L - q_len + t + 1;  // causal: keys 0 .. visible-1
  // Window: key j is kept if j < sinks or j >= visible - recent; keys in
  // released pages (table entry < 0) are gone.
  const int sinks = a.seq_win ? a.seq_win[4 * b] : 0;
  const int recent = a.seq_win ? a.seq_win[4 * b + 1] : kNoWindowRecent;
  const int win_lo = visible - recent;
  const int g = h / a.group;
  const int D = a.head_dim, BS = a.block_size, Hkv = a.num_kv_heads;
  const int32_t* table = a.tables + a.tbl_off[b];
  const T* K = static_cast<const T*>(a.k_pool);
  const T* V = static_cast<const T*>(a.v_pool);
  const size_t q8_page = static_cast<size_t>(BS) * D + 4 * static_cast<size_t>(BS);
  const T* q = static_cast<const T*>(a.q) + (static_cast<size_t>(r) * a.num_heads + h) * D;
  for (int d = lane; d < D; d += 64) qs[d] = Elt<T>::load(q + d);
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int c0 = 0; c0 < visible; c0 += 64) {
    const int j = c0 + lane;
    float s = -INFINITY;
    int blk = 0, off = 0;
    bool keep = j < visible && (j < sinks || j >= win_lo);
    if (keep) {
      // Decode plans list the visited pages only: page pg is entry pg below
      // the sink pages, then entry pg - gap; the gap's pages hold no key any
      // row sees (prefill plans have no gap).
      const int pg = j / BS;
      const int sp = a.seq_win ? a.seq_win[4 * b + 2] : 0, gp = a.seq_win ? a.seq_win[4 * b + 3] : 0;
      if (pg >= sp && pg < sp + gp) {
        keep = false;
      } else {
        blk = table[pg < sp ? pg : pg - gp];
        keep = blk >= 0;
      }
    }
    if (keep) {
      off = j - (j / BS) * BS;
      float dot = 0.f;
      if constexpr (Q8) {
        const uint8_t* kp = static_cast<const uint8_t*>(a.k_pool) + (static_cast<size_t>(blk) * Hkv + g) * q8_page;
        for (int d = 0; d < D; ++d) dot += qs[d] * code_value<Q8>(kp[k8_offset(off, d, D)]);
        dot *= reinterpret_cast<const float*>(kp + BS * D)[off];
      } else {
        const T* kp = K + (static_cast<size_t>(blk) * Hkv + g) * BS * D;
        if constexpr (sizeof(T) == 2) {
          for (int d = 0; d < D; ++d) dot += qs[d] * Elt<T>::load(kp + k16_offset(off, d, D, BS));
        } else {
          for (int d = 0; d < D; ++d) dot += qs[d] * Elt<T>::load(kp + off * D + d);
        }
      }
      s = dot * a.scale_log2;
    }
    const float m_new = fmaxf(m, wave_max(s));
    // No kept key so far (m_new = -inf): exponents against 0 give weight 0.
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m - m_ref);
    float p = keep ? exp2f(s - m_ref) : 0.f;
    l = l * alpha + wave_sum(p);
    if constexpr (Q8) {
      // The V scale joins the weight: sum_j p_j sv_j cv_j.
      if (keep)
        p *= reinterpret_cast<const float*>(static_cast<const uint8_t*>(a.v_pool) +
                                            (static_cast<size_t>(blk) * Hkv + g) * q8_page + BS * D)[off];
    }
    ps[lane] = p;
    blks[lane] = keep ? blk : -1;  // -1: not kept (its page may be released)
    offs[lane] = off;
    __syncthreads();
    const int nj = min(64, visible - c0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = lane + 64 * k;
      float x = acc[k] * alpha;
      if (d < D) {
        if constexpr (Q8) {
          const uint8_t* vb = static_cast<const uint8_t*>(a.v_pool);
          for (int jj = 0; jj < nj; ++jj)
            if (blks[jj] >= 0)
              x += ps[jj] * code_value<Q8>(vb[(static_cast<size_t>(blks[jj]) * Hkv + g) * q8_page +
                                               q8_v_offset(offs[jj], d, D)]);
        } else {
          for (int jj = 0; jj < nj; ++jj)
            if (blks[jj] >= 0)
              x += ps[jj] * Elt<T>::load(V + ((static_cast<size_t>(blks[jj]) * Hkv + g) * D + d) * BS + offs[jj]);
        }
      }
      acc[k] = x;
    }
    m = m_new;
    __syncthreads();
  }
  T* o = static_cast<T*>(a.out) + (static_cast<size_t>(r) * a.num_heads + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int d = lane + 64 * k;
    if (d < D) Elt<T>::store(o + d, acc[k] * inv);
  }
}

// ------------------------------------------------------------ GQA / MFMA ---
// One page of one KV head, as one lane holds it.
//   bf16: k[tt][j] = K[16tt + n][32j + 8grp .. +8], v[nt][tt] = V^T[16nt + n][16tt + 4grp .. +4]
//   codes: kc[tt][.] = K codes of token 16tt + n, d in [grp * D/4, +D/4) (the QK
//         contraction runs over that permuted d order, Q takes the same),
//         vc[tt][nt] = V codes of d = 16nt + n, tokens 16tt + 4grp .. +4,
//         ks / vs = the row scales of tokens 16tt + 4grp .. +4.
template <int D, int BS, int Q8> struct PageRegs {  // 8-bit codes
  uint32_t kc[BS / 16][D / 16];
  uint32_t vc[BS / 16][D / 16];
  f32x4 ks[BS / 16], vs[BS / 16];
};
template <int D, int BS> struct PageRegs<D, BS, 0> {
  bf16x8 k[BS / 16][D / 32];
  s16x4 v[D / 16][BS / 16];
};

// Minimum waves per SIMD a decode kernel variant is compiled for (its
// register budget).  8-bit pages move fewer bytes per load, so the 16-column
// 8-bit kernels ask for 3 resident waves to keep enough bytes in flight; the
// d 128 / 32-slot / 32-column variants hold two 32-token pages for two
// column tiles and would spill under 2, so they take what they need.
template <int D, int BS, int CT, int Q8>
constexpr int decode_waves() {
  if (Q8 && CT == 1 && BS == 16) return PA_DECODE_WAVES_I8;
  if (D == 128 && BS == 32 && CT == 2) return 1;
  return 2;
}

// decode_mfma: split-K paged attention for query rows that are the last
// q_len positions of their sequence (q_len = 1: decode).
//
// What is computed (docs.rs ferrum-kv 0.4.0 src/attention.rs,
// paged_attention: GQA head g = h / G, scale 1/sqrt(D), query row t of q_len
// sees keys j <= L - q_len + t), over the page range of one work item; with
// Q8 over pages of 8-bit codes (1: int8, 2: E4M3) whose rows read back as
// value(code) * scale (vladkulikov.com notebook "Модуль 10", KV-compression
// experiment; the E4M3 codes extend its integer ones):
//   s_j = (q . ck_j) * sk_j / sqrt(D),  o = sum_j p_j sv_j cv_j / sum_j p_j
// with sk folded into the scores and sv into the P operand.
//
// One workgroup = (work item = (sequence, page range), KV head); its 4 waves
// stride over the pages.  The MFMA N dimension holds CT tiles of 16 columns;
// column col = (t, hn) = (col / G, col % G) is query row t of head g*G + hn,
// so the q_len * G columns of a sequence share every K/V page load:
//   S^T[16 tok x 16 col]  = K_page[16 x D] . Q^T[D x 16]      (16x16x32)
//   O^T[16 d   x 16 col] += V^T_page[16 x 16] . P^T[16 x 16]  (16x16x16)
// The C layout of the first (lane = 4 tokens of one column) is the B layout
// of the second, so P never leaves registers.  Online softmax per page, P
// split into bf16 hi + lo terms (~16 mantissa bits of p); the 4 waves merge
// in LDS; a range that is the whole sequence writes bf16 output, otherwise
// fp32 partials (m, l, acc) for the merge kernel.
template <int D, int BS, int CT, int Q8>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(decode_waves<D, BS, CT, Q8>())))
void decode_mfma(DecodeArgs a) {
  constexpr int KS = D / 32;   // k-steps of the 16x16x32 QK contraction
  constexpr int TT = BS / 16;  // 16-token tiles per page
  constexpr int DT = D / 16;   // 16-wide d tiles of the P.V contraction
  constexpr int W = kDecodeWaves;
  constexpr int ROW = D + 4;   // padded LDS row of one column's accumulator
  constexpr size_t PB = Q8 ? static_cast<size_t>(BS) * D + 4 * BS : static_cast<size_t>(BS) * D * 2;
  __shared__ float s_m[W][16];
  __shared__ float s_l[W][16];
  // [W][Cn][ROW]: the live columns of one 16-column tile, staged for the wave merge.
  extern __shared__ float s_acc[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int Hkv = a.num_kv_heads, Hq = a.num_heads, G = a.group;
  const int wid = blockIdx.x / Hkv, g = blockIdx.x - wid * Hkv;
  const int32_t* item = a.work + kWorkInts * wid;
  const int c = item[1];  // item[0] is the sequence (its data is in the item)
  const int L = item[2];
  const int row0 = item[3], qlen = item[4];
  const int C = qlen * G;  // live columns
  const int nblk = (L + BS - 1) / BS;
  // Window of the sequence: sinks, recent, and the visited pages (compact
  // index i < nvis is page i below the sink pages, else page i + gap).
  const int sinks = item[5], recent = item[6];
  const int sink_pages = item[7], gap = item[8];
  const int nvis = nblk - gap;
  const int p0 = c * a.pages_per_part;
  const int p1 = min(nvis, p0 + a.pages_per_part);
  // Pages from mask0 on hold keys some column must not see (or past-end
  // slots); pages starting before win_hi may hold keys left of a window.
  const int mask0 = (L - qlen + 1) / BS;
  const int win_hi = L - recent;
  const int32_t* table = a.tables + item[9];
  const char* kpool = static_cast<const char*>(a.k_pool);
  const char* vpool = static_cast<const char*>(a.v_pool);

  // Q^T operand and visible-key limit of this lane's column in each tile.
  bf16x8 qv[CT][KS];
  int lim[CT], wlo[CT];  // column sees key p iff p < lim and (p < sinks or p >= wlo)
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = 16 * ct + n;
    const int t = col / G, hn = col - t * G;
    const bool live = col < C;
    lim[ct] = live ? L - qlen + t + 1 : L;
    wlo[ct] = lim[ct] - recent;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(row0 + (live ? t : 0)) * Hq + g * G + hn) * D +
                           (Q8 ? (D / 4) * grp : 8 * grp);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      if (live)
        qv[ct][j] = *reinterpret_cast<const bf16x8*>(qrow + (Q8 ? 8 * j : 32 * j));
      else
        qv[ct][j] = bf16x8{};
    }
  }
  // The 32-column variants read their Q operands from LDS on every page
  // (written once by wave 0: the four waves share the columns), leaving the
  // registers to the page ring and the accumulators.
  constexpr bool kQInLds = CT == 2;
  __shared__ bf16x8 s_q[kQInLds ? CT * KS : 1][64];
  if constexpr (kQInLds) {
    if (wave == 0) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int j = 0; j < KS; ++j) s_q[ct * KS + j][lane] = qv[ct][j];
    }
    __syncthreads();
  }

  float m_run[CT], l_run[CT];
  f32x4 acc[CT][DT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) acc[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  using Page = PageRegs<D, BS, Q8>;
  auto page_of = [&](int ci) { return ci < sink_pages ? ci : ci + gap; };
  // Tables list the visited pages.  A scalar load (counted by lgkmcnt), so
  // waiting for a block id never waits behind the wave's page loads.
  auto block_of = [&](int ci) { return scalar_load(table, uniform(ci)); };
  auto load_page_blk = [&](int blk, Page& P) {
    const char* kp = kpool + (static_cast<size_t>(blk) * Hkv + g) * PB;
    const char* vp = vpool + (static_cast<size_t>(blk) * Hkv + g) * PB;
    // Every page byte is read once per launch: all page loads carry the
    // non-temporal (streaming) hint.  K pages (and 8-bit V pages) are in the
    // page order of k16_offset / k8_offset / q8_v_offset, so each load
    // instruction reads 1 KB of consecutive bytes (lane l: bytes 16l ..
    // 16l + 15 of a 1 KB run), already in operand order.
    if constexpr (Q8) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const u32x4* ks = reinterpret_cast<const u32x4*>(kp + 16 * tt * D) + lane;
        const u32x4* vs = reinterpret_cast<const u32x4*>(vp + 16 * tt * D) + lane;
#pragma unroll
        for (int w = 0; w < DT / 4; ++w) {
          const u32x4 x = __builtin_nontemporal_load(ks + 64 * w), y = __builtin_nontemporal_load(vs + 64 * w);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            P.kc[tt][4 * w + i] = x[i];
            P.vc[tt][4 * w + i] = y[i];
          }
        }
        P.ks[tt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kp + BS * D + 4 * (16 * tt + 4 * grp)));
        P.vs[tt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vp + BS * D + 4 * (16 * tt + 4 * grp)));
      }
    } else {
      const uint16_t* k16 = reinterpret_cast<const uint16_t*>(kp);
      const uint16_t* v16 = reinterpret_cast<const uint16_t*>(vp);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int j = 0; j < KS; ++j)
          P.k[tt][j] = __builtin_nontemporal_load(
              reinterpret_cast<const bf16x8*>(k16 + 16 * tt * D + (64 * j + lane) * 8));
#pragma unroll
      for (int nt = 0; nt < DT; ++nt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          P.v[nt][tt] = __builtin_nontemporal_load(
              reinterpret_cast<const s16x4*>(v16 + (16 * nt + n) * BS + 16 * tt + 4 * grp));
    }
  };

  auto load_page = [&](int ci, Page& P) { load_page_blk(block_of(ci), P); };

  // EDGE: the page holds keys some column must not see (causal limit,
  // window, past-end slots); other pages take the path without masks.
  auto process_page = [&](int ci, const Page& P, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int pg = page_of(ci);
    // s[ct][tt][i] = score of token pg*BS + 16tt + 4grp + i for column 16ct + n.
    f32x4 s[CT][TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      bf16x8 kop[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        if constexpr (Q8)
          kop[j] = codes8_to_bf16x8<Q8>(P.kc[tt][2 * j], P.kc[tt][2 * j + 1]);
        else
          kop[j] = P.k[tt][j];
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        s[ct][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j)
          s[ct][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j], kQInLds ? s_q[ct * KS + j][lane] : qv[ct][j],
                                                              s[ct][tt], 0, 0, 0);
      }
    }
    s16x4 p_hi[CT][TT], p_lo[CT][TT];
    float alpha[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float mloc = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[ct][tt][i];
          if constexpr (Q8)
            x *= P.ks[tt][i] * a.scale_log2;
          else
            x *= a.scale_log2;
          if constexpr (EDGE) {
            const int pos = pg * BS + 16 * tt + 4 * grp + i;
            if (pos >= lim[ct] || (pos >= sinks && pos < wlo[ct])) x = -INFINITY;
          }
          s[ct][tt][i] = x;
          mloc = fmaxf(mloc, x);
        }
#if PA_DECODE_PERMLANE
      mloc = rows4_max(mloc);
#else
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
#endif
      const float m_new = fmaxf(m_run[ct], mloc);
      // A column with no visible key so far keeps m = -inf; exponents are
      // then taken against 0, giving weight 0 instead of -inf - -inf.
      const float m_ref = m_new == -INFINITY ? 0.f : m_new;
      alpha[ct] = exp2_flush(m_run[ct] - m_ref);
      m_run[ct] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = exp2_flush(s[ct][tt][i] - m_ref);
          psum += e;
          float w = e;
          if constexpr (Q8) {
            w = e * P.vs[tt][i];
            // A masked or past-end slot may hold any scale bits: weight 0.
            if constexpr (EDGE) {
              const int pos = pg * BS + 16 * tt + 4 * grp + i;
              if (pos >= lim[ct] || (pos >= sinks && pos < wlo[ct])) w = 0.f;
            }
          }
          const __bf16 hi = static_cast<__bf16>(w);
          const __bf16 lo = static_cast<__bf16>(w - static_cast<float>(hi));
          p_hi[ct][tt][i] = __builtin_bit_cast(short, hi);
          p_lo[ct][tt][i] = __builtin_bit_cast(short, lo);
        }
      l_run[ct] = l_run[ct] * alpha[ct] + psum;
    }
    // Past-end slots of the last page have weight 0 and their values are
    // zeroed too, so 0 * V cannot meet non-finite bits left there (int8
    // codes are always finite; bf16 and E4M3 bytes may be NaN).
    const bool tail = EDGE && Q8 != 1 && pg == nblk - 1;
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct][nt] *= alpha[ct];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        s16x4 v;
        if constexpr (Q8) v = codes4_to_bf16x4<Q8>(P.vc[tt][nt]);
        else v = P.v[nt][tt];
        if (tail) {
          const int live = L - (pg * BS + 16 * tt + 4 * grp);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i >= live) v[i] = 0;
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          acc[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, p_hi[ct][tt], acc[ct][nt], 0, 0, 0);
          acc[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, p_lo[ct][tt], acc[ct][nt], 0, 0, 0);
        }
      }
    }
  };

  auto process = [&](int ci, const Page& P) {
    const int pg = page_of(ci);
    if (pg >= mask0 || (pg * BS < win_hi && pg * BS + BS > sinks))
      process_page(ci, P, std::true_type{});
    else
      process_page(ci, P, std::false_type{});
  };

  // Page loop: each wave keeps DEPTH pages in flight ahead of the one it
  // computes, in a ring of DEPTH + 1 register buffers (the loop is unrolled
  // over the ring so every buffer index is static).  Loads are issued
  // unconditionally (past the range end a wave re-loads its current page,
  // an L2 hit): with the same number of loads in flight on every path, the
  // wait before a page's first use covers only that page's loads.
  {
    constexpr int DEPTH = PA_DECODE_DEPTH;
    constexpr int NP = DEPTH + 1;
    Page buf[NP];
    int p = p0 + wave;
    if (p < p1) {
      // The first page's block id comes with the work item (no table hop).
      load_page_blk(item[12 + wave], buf[0]);
#pragma unroll
      for (int k = 1; k < DEPTH; ++k) load_page(p + k * W < p1 ? p + k * W : p, buf[k]);
#if PA_DECODE_TABLE_AHEAD
      // The block id of the page to load next iteration is fetched one
      // iteration early, so its scalar load is back before it is needed.
      int blk_ahead = block_of(min(p + DEPTH * W, p1 - 1));
#endif
      while (true) {
#pragma unroll
        for (int u = 0; u < NP; ++u) {
#if PA_DECODE_TABLE_AHEAD
          load_page_blk(blk_ahead, buf[(u + DEPTH) % NP]);
          blk_ahead = block_of(min(p + (DEPTH + 1) * W, p1 - 1));
#else
          const int ahead = p + DEPTH * W;
          load_page(ahead < p1 ? ahead : p, buf[(u + DEPTH) % NP]);
#endif
          process(p, buf[u]);
          p += W;
          if (p >= p1) goto pages_done;
        }
      }
    }
  pages_done:;
  }

  // Per-column totals over the 4 lane groups, then merge the 4 waves, one
  // 16-column tile at a time (LDS holds one tile of the 4 waves).
  const int base = item[10];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int Cn = min(16, C - 16 * ct);  // live columns of this tile (uniform)
    if (Cn <= 0) break;
    if (ct > 0) __syncthreads();  // the previous tile's readers are done
#if PA_DECODE_PERMLANE
    const float l_tot = rows4_sum(l_run[ct]);
#else
    float l_tot = l_run[ct] + __shfl_xor(l_run[ct], 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
#endif
    if (grp == 0) {
      s_m[wave][n] = m_run[ct];
      s_l[wave][n] = l_tot;
    }
    if (n < Cn) {
      float* dst = s_acc + (wave * Cn + n) * ROW + 4 * grp;
#pragma unroll
      for (int nt = 0; nt < DT; ++nt) *reinterpret_cast<f32x4*>(dst + 16 * nt) = acc[ct][nt];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Cn * D; idx += 256) {
      const int cn = idx / D, d = idx - cn * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][cn]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        // A wave without visible keys has m = -inf and contributes nothing.
        const float e = s_m[w][cn] == -INFINITY ? 0.f : exp2f(s_m[w][cn] - M);
        num += e * s_acc[(w * Cn + cn) * ROW + d];
        den += e * s_l[w][cn];
      }
      const int col = 16 * ct + cn;
      const int t = col / G, h = g * G + (col - t * G);
      if (base < 0) {
        static_cast<uint16_t*>(a.out)[(static_cast<size_t>(row0 + t) * Hq + h) * D + d] = f32_to_bf16(num / den);
      } else {
        const size_t row = static_cast<size_t>(base) + (static_cast<size_t>(c) * qlen + t) * Hq + h;
        a.part_acc[row * D + d] = num;
        if (d == 0) {
          a.part_m[row] = M;
          a.part_l[row] = den;
        }
      }
    }
  }
}

// ----------------------------------------------------------------- merge ---
// Log-sum-exp combination of the partials of one (query row, head) of a
// split sequence: M = max m_c, o = sum e^(m_c - M) acc_c / sum e^(m_c - M) l_c
// (CMU 11-667 lecture 19 section 3, online_softmax_stats, applied across
// page ranges).  A range with no visible key has m = -inf and weight 0.
template <int D, typename T>
__global__ __launch_bounds__(256) void decode_merge(DecodeArgs a) {
  // One workgroup per (split query row, head).  Thread (r, v) owns float4 v
  // of the partial rows c = r, r + R, ...: it loads kBatch of them at once
  // (their m, l and acc chunk, all issued before any is used) and folds them
  // into a running (max, numerator, denominator) with the log-sum-exp rule;
  // a split of up to R * kBatch partial rows thus costs one memory round
  // trip.  The R running triples then combine through LDS.
  constexpr int V4 = D / 4;      // float4 lanes per partial row
  constexpr int R = 256 / V4;    // partial rows in flight
  constexpr int kBatch = 4;      // partial rows per thread per round trip
  __shared__ float s_m[R], s_den[R];
  __shared__ f32x4 s_num[R][V4];
  const int tid = threadIdx.x;
  const int Hq = a.num_heads;
  const int mi = blockIdx.x / Hq, h = blockIdx.x - mi * Hq;
  // The merge entry carries everything (one scalar load, no second hop).
  const int32_t* entry = a.merge_rows + 4 * mi;
  const int out_row = entry[0], first = entry[1], stride = entry[2], np = entry[3];
  auto prow = [&](int c) { return static_cast<size_t>(first) + h + static_cast<size_t>(c) * stride; };
  const int r = tid / V4, v = tid - r * V4;

  float m_t = -INFINITY, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = r; c0 < np; c0 += R * kBatch) {
    float mc[kBatch], lc[kBatch];
    f32x4 xc[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = c0 + k * R;
      if (c < np) {
        const size_t row = prow(c);
        mc[k] = a.part_m[row];
        lc[k] = a.part_l[row];
        xc[k] = reinterpret_cast<const f32x4*>(a.part_acc + row * D)[v];
      } else {
        mc[k] = -INFINITY;
        lc[k] = 0.f;
        xc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    float mm = m_t;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) mm = fmaxf(mm, mc[k]);
    if (mm == -INFINITY) continue;  // nothing visible yet (window ranges)
    const float keep = m_t == -INFINITY ? 0.f : exp2f(m_t - mm);
    num *= keep;
    den *= keep;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = mc[k] == -INFINITY ? 0.f : exp2f(mc[k] - mm);
      num += w * xc[k];
      den += w * lc[k];
    }
    m_t = mm;
  }
  s_num[r][v] = num;
  if (v == 0) {
    s_m[r] = m_t;
    s_den[r] = den;
  }
  __syncthreads();
  if (tid < V4) {
    float M = s_m[0];
#pragma unroll
    for (int k = 1; k < R; ++k) M = fmaxf(M, s_m[k]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float dtot = 0.f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float w = s_m[k] == -INFINITY ? 0.f : exp2f(s_m[k] - M);
      tot += w * s_num[k][tid];
      dtot += w * s_den[k];
    }
    const float inv = 1.f / dtot;
    T* o = static_cast<T*>(a.out) + (static_cast<size_t>(out_row) * Hq + h) * D + 4 * tid;
#pragma unroll
    for (int i = 0; i < 4; ++i) Elt<T>::store(o + i, tot[i] * inv);
  }
}

template <int D, int BS, int CT, int Q8>
void launch_mfma(const DecodeArgs& a, int groups, hipStream_t stream, const KernelEvents& ev) {
  const size_t shmem = static_cast<size_t>(kDecodeWaves) * min(a.max_cols, 16) * (D + 4) * sizeof(float);
  PA_LAUNCH(ev, (decode_mfma<D, BS, CT, Q8>), dim3(groups), dim3(256), shmem, stream, a);
}

template <int CT, int Q8>
void launch_mfma_shape(const PoolGeom& geom, const DecodeArgs& a, hipStream_t stream, const KernelEvents& ev) {
  const int groups = a.n_work * a.num_kv_heads;
  const int D = geom.head_dim, BS = geom.block_size;
  if (D == 128 && BS == 16) launch_mfma<128, 16, CT, Q8>(a, groups, stream, ev);
  else if (D == 128 && BS == 32) launch_mfma<128, 32, CT, Q8>(a, groups, stream, ev);
  else if (D == 64 && BS == 16) launch_mfma<64, 16, CT, Q8>(a, groups, stream, ev);
  else launch_mfma<64, 32, CT, Q8>(a, groups, stream, ev);
}

void launch_generic(const PoolGeom& geom, const GenericArgs& g, dim3 grid, hipStream_t stream,
                    const KernelEvents& ev) {
  const size_t shmem = (geom.head_dim + 64) * sizeof(float) + 128 * sizeof(int);
  if (geom.fp8())
    PA_LAUNCH(ev, (attn_generic<uint16_t, 2>), grid, dim3(64), shmem, stream, g);
  else if (geom.q8())
    PA_LAUNCH(ev, (attn_generic<uint16_t, 1>), grid, dim3(64), shmem, stream, g);
  else if (geom.dtype == 1)
    PA_LAUNCH(ev, (attn_generic<uint16_t, 0>), grid, dim3(64), shmem, stream, g);
  else
    PA_LAUNCH(ev, (attn_generic<float, 0>), grid, dim3(64), shmem, stream, g);
}

}  // namespace

DecodeKernel pick_decode_kernel(const PoolGeom& geom, int32_t group) {
  const bool d_ok = geom.head_dim == 64 || geom.head_dim == 128;
  const bool bs_ok = geom.block_size == 16 || geom.block_size == 32;
  if (d_ok && bs_ok && group <= 16) {
    if (geom.dtype == 1) return DecodeKernel::kGqaMfma;
    if (geom.q8()) return DecodeKernel::kQ8Mfma;
  }
  return DecodeKernel::kGeneric;
}

bool decode_handles_rows(const PoolGeom& geom, int32_t group, int32_t max_q_len) {
  return pick_decode_kernel(geom, group) != DecodeKernel::kGeneric &&
         static_cast<int64_t>(max_q_len) * group <= kDecodeMaxCols;
}

hipError_t launch_decode_partial(const PoolGeom& geom, const DecodeArgs& a, hipStream_t stream,
                                 const KernelEvents& ev) {
  const DecodeKernel k = pick_decode_kernel(geom, a.group);
  if (k != DecodeKernel::kGeneric && a.max_cols > kDecodeMaxCols) return hipErrorInvalidValue;
  if (k == DecodeKernel::kGeneric && a.max_cols > a.group) return hipErrorInvalidValue;  // q_len 1 only
  const bool two = a.max_cols > 16;
  switch (k) {
    case DecodeKernel::kGqaMfma:
      if (two) launch_mfma_shape<2, 0>(geom, a, stream, ev);
      else launch_mfma_shape<1, 0>(geom, a, stream, ev);
      break;
    case DecodeKernel::kQ8Mfma:
      if (geom.fp8()) {
        if (two) launch_mfma_shape<2, 2>(geom, a, stream, ev);
        else launch_mfma_shape<1, 2>(geom, a, stream, ev);
      } else {
        if (two) launch_mfma_shape<2, 1>(geom, a, stream, ev);
        else launch_mfma_shape<1, 1>(geom, a, stream, ev);
      }
      break;
    default: {
      GenericArgs g{a.k_pool, a.v_pool, a.q, a.out, a.ctx_len, a.tbl_off, a.tables, nullptr, nullptr,
                    a.seq_win, a.num_heads, a.num_kv_heads, a.group, geom.head_dim, geom.block_size,
                    a.scale_log2};
      launch_generic(geom, g, dim3(a.batch * a.num_heads), stream, ev);
      break;
    }
  }
  return hipGetLastError();
}

bool decode_needs_merge_kernel(const PoolGeom& geom, int32_t group) {
  return pick_decode_kernel(geom, group) != DecodeKernel::kGeneric;  // the generic kernel never splits
}

hipError_t launch_decode_merge(const PoolGeom& geom, const DecodeArgs& a, hipStream_t stream,
                               const KernelEvents& ev) {
  if (a.n_merge == 0 || !decode_needs_merge_kernel(geom, a.group)) return hipSuccess;
  const dim3 grid(a.n_merge * a.num_heads);
  if (geom.head_dim == 128)
    PA_LAUNCH(ev, (decode_merge<128, uint16_t>), grid, dim3(256), 0, stream, a);
  else
    PA_LAUNCH(ev, (decode_merge<64, uint16_t>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Prefill through the generic kernel (query rows with their causal limits).
hipError_t launch_prefill_generic(const PoolGeom& geom, const PrefillArgs& a, hipStream_t stream,
                                  const KernelEvents& ev) {
  GenericArgs g{a.k_pool, a.v_pool, a.q, a.out, a.ctx_len, a.tbl_off, a.tables, a.q_start,
                a.row_seq, a.seq_win, a.num_heads, a.num_kv_heads, a.group, geom.head_dim,
                geom.block_size, a.scale_log2};
  launch_generic(geom, g, dim3(a.n_rows * a.num_heads), stream, ev);
  return hipGetLastError();
}

}  // namespace pa
