// Chunked causal prefill over the paged pool.
//
// What is computed (docs.rs ferrum-kv 0.4.0 src/attention.rs,
// paged_attention with q_tokens > 1): the q_len query rows of a sequence are
// its last q_len positions; row t sees keys j <= kv_len - q_len + t
// (bottom-right causal alignment, as CMU 11-667 lecture 19's CachedDecoder
// masks cached decoding).  The one-pass running max / sum per key tile is
// lecture 19's tiled_attention recurrence.
//
// Two kernels share the plan (tiles of query rows) and the key-tile walk:
// prefill_bf16_mfma32 (bf16 pages, 32x32x16 MFMA tiles, further below) and
// prefill_q8_mfma (8-bit pages, 16x16x32 tiles over bf16 operands converted
// in LDS).
//
// prefill_q8_mfma<D, BS, CG, NW, S, Q8>  (Q8 1 int8 / 2 E4M3 codes; D in {64, 128},
//                                        BS in {16, 32}, G | 16)
//   One workgroup of NW waves = (sequence, block of query rows, KV head).
//   The MFMA N dimension packs (query row, head of the group) pairs: column c
//   of the workgroup is row t0 + c / G, head g*G + c % G, so each key tile
//   serves all G query heads of its KV head.  Each wave owns CG groups of 16
//   columns (Q^T operands and O^T accumulators stay in registers).
//
//   Keys advance in tiles of 32 tokens (two 16-slot pages or one 32-slot
//   page).  Per tile:
//     S^T[16 tok x 16 col] = K_tile . Q^T     (x2 token halves)  v_mfma_f32_16x16x32_bf16
//     O^T[16 d  x 16 col] += V^T_tile . P^T   (x D/16 d tiles)   v_mfma_f32_16x16x32_bf16
//   Row m of the QK tile tt is token 8*(m/4) + 4*tt + m%4, so the lane that
//   ends up holding S^T rows 4*grp .. 4*grp+3 of both tiles holds tokens
//   8*grp .. 8*grp+7: its P^T operand for the 32-token P.V step is its own
//   accumulator, and the matching V^T operand is 16 contiguous bytes of one
//   page row.  Every K and V operand of a tile is therefore one 16-byte
//   chunk per lane, and the tile is NB blocks of 64 such chunks.
//
//   (The ring, staging, masks and windows below are described for bf16
//   operand tiles; prefill_bf16_mfma32 stages exactly so, and this kernel
//   stages raw 8-bit tiles and converts them, see the last paragraph.)
//   The workgroup keeps an S-stage ring of tiles in LDS.  Each block is
//   fetched with one direct global->LDS load (global_load_lds_dwordx4; lane l
//   writes bytes 16l..16l+15 of the block), already in operand order, so the
//   MFMA operand reads are conflict-free 16-byte LDS reads and no register
//   holds in-flight data; loads run S-1 tiles ahead, and one barrier per
//   tile (after each wave's own vmcnt wait) publishes a tile and frees the
//   stage read in the previous step.  Slots past the sequence end are staged
//   from a zero region (and the tail tile's V operands are masked), so
//   0 * V never meets stale or non-finite bits.
//   Tiles wholly below every row's limit are not masked; tiles past a
//   wave's last row's limit are skipped by that wave.  blockIdx % Hkv is the
//   KV head: with Hkv a multiple of 8 each XCD (and its L2) serves one KV
//   head of every sequence, so a shared prefix is read from HBM once per
//   head.
//
//   Windows (sinks + recent, at page granularity): a windowed workgroup walks
//   the key tiles holding sink keys, then those from its first row's window
//   start on, all on the masked path: key j is visible to a row at position
//   p if j <= p and (j < sinks or j >= p + 1 - recent) and its page is still
//   resident (released pages are -1 in the table, staged as zeros and
//   masked).
//
//   8-bit pages (the [KVquant] rows: int8 or E4M3 codes plus one fp32 scale
//   per token and KV head): the ring holds tiles as the pages store them (K codes, V codes
//   in their operand order, the 64 scales; 16-byte chunks permuted so every
//   LDS access is conflict-free), fetched with the same direct loads; each
//   step four waves convert the next tile's K operand blocks and four its V
//   blocks to bf16 (exact for both code kinds) into one of two operand-ordered
//   tiles, so the MFMA part is the bf16 one.  The scales stay
//   in fp32: K's multiply the scores, V's the weights entering P.V (l sums
//   the weights without them).
#include <cmath>
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"
#include "launch.hpp"

#ifndef PA_PREFILL_CG
#define PA_PREFILL_CG 1
#endif
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
#ifndef PA_PREFILL_STAGES_Q8
#define PA_PREFILL_STAGES_Q8 4
#endif
#ifndef PA_PREFILL32_WAVES
#define PA_PREFILL32_WAVES 4
#endif
#ifndef PA_PREFILL32_STAGES
#define PA_PREFILL32_STAGES 3
#endif
#ifndef PA_PREFILL32_Q_LDS
#define PA_PREFILL32_Q_LDS 0
#endif
#ifndef PA_PREFILL_WAVES_PER_EU
#define PA_PREFILL_WAVES_PER_EU 0  // occupancy hint (0 = none)
#endif
#if PA_PREFILL_WAVES_PER_EU > 0
#define PA_PREFILL_OCC __attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU)))
#else
#define PA_PREFILL_OCC
#endif

namespace pa {

hipError_t launch_prefill_generic(const PoolGeom& geom, const PrefillArgs& a, hipStream_t stream,
                                  const KernelEvents& ev);

namespace {


constexpr int kPrefillCG = PA_PREFILL_CG;          // 16-column groups per wave
constexpr int kPrefillWaves = PA_PREFILL_WAVES;    // waves per workgroup
constexpr int kPrefillStagesQ8 = PA_PREFILL_STAGES_Q8;  // raw 8-bit tiles in the LDS ring
constexpr int kPrefill32Waves = PA_PREFILL32_WAVES;     // waves per 32x32-tile workgroup
constexpr int kPrefill32Stages = PA_PREFILL32_STAGES;   // key tiles in its LDS ring
constexpr int kTile = 32;                          // key tokens per step
constexpr float kSlackLog2 = 8.f;                  // largest softmax weight, log2

// A wave-uniform pointer kept in scalar registers (the compiler would
// otherwise fold a per-lane choice between two such pointers into the
// arithmetic that forms them, and do that arithmetic per lane).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return reinterpret_cast<const T*>(lo | (hi << 32));
}


template <int D, int BS, int CG, int NW, int S, int Q8>
__global__ __launch_bounds__(NW * 64) PA_PREFILL_OCC void prefill_q8_mfma(PrefillArgs a) {
  static_assert(Q8 == 1 || Q8 == 2, "bf16 pages take prefill_bf16_mfma32");
  constexpr int KS = D / 32;         // k-steps of QK per token half
  constexpr int DT = D / 16;         // d tiles of P.V
  constexpr int KB = 2 * KS;         // K operand blocks per key tile
  constexpr int NB = KB + DT;        // operand blocks per key tile
  constexpr int PAGES = kTile / BS;  // pages per key tile
  static_assert(NB % NW == 0, "each wave stages the same number of blocks");
  constexpr int BPW = NB / NW;       // blocks staged (bf16) or converted (8-bit) by each wave per tile
  static_assert((S - 2) * BPW < 64, "vmcnt range");
  // 8-bit pages: a tile as the pages hold it (K codes, V codes, K scales, V
  // scales of its 32 tokens), moved by kCodeLoads 1 KB wave loads of codes
  // plus one 256-byte load of scales.
  constexpr int kRawBytes = 2 * kTile * D + 2 * kTile * 4;
  constexpr int kCodeLoads = 2 * kTile * D / 1024;
  constexpr int kRowChunks = D / 16;      // 16-byte chunks per K row
  constexpr int kRowChunksV = D / 64;     // 16-byte chunks per V operand-order row (D / 4 bytes)
  // Chunk permutations of the raw 8-bit tile in LDS (each an involution on
  // its range).  K: chunk c of token t's row sits at c ^ q8_k_swizzle(t), so
  // the 32 lanes of an 8-byte conversion read (16 tokens x 2 halves of a
  // chunk) cover all 64 banks.  V (d 128, two chunks per row): chunk q of a
  // subtile sits at q with bit 0 flipped by bit 4, so the 16 lanes of a
  // 16-byte read (rows n = 0..15) hit distinct bank groups; d 64 rows are
  // one chunk and already do.
  auto q8_k_swizzle = [](int t) {
    if constexpr (D == 128) return ((t >> 1) & 1) | ((t >> 2) & 6);
    else return (t >> 3) & 3;
  };
  auto q8_v_swizzle = [](int q) {
    if constexpr (D == 128) return q ^ ((q >> 4) & 1);
    else return q;
  };
  static_assert(!Q8 || (S >= 4 && kCodeLoads <= NW && kCodeLoads % 2 == 0), "8-bit ring");
  // bf16: an S-stage ring of operand-ordered tiles.  8-bit: an S-stage ring of
  // raw tiles and two operand-ordered bf16 tiles converted from them.
  __shared__ uint4 ring[2][NB][64];
  __shared__ uint4 raw[S][kRawBytes / 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int n = lane & 15, grp = lane >> 4;
  const int Hkv = a.num_kv_heads, Hq = a.num_heads, G = a.group;
  const int tile = blockIdx.x / Hkv, g = blockIdx.x - tile * Hkv;
  const int b = a.tiles[2 * tile], t0 = a.tiles[2 * tile + 1];
  const int q0 = a.q_start[b];
  const int q_len = a.q_start[b + 1] - q0;
  const int L = a.ctx_len[b];
  const int off = L - q_len;  // row t sees keys 0 .. off + t
  const int nblk = (L + BS - 1) / BS;
  const int32_t* table = a.tables + a.tbl_off[b];
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  const size_t page = static_cast<size_t>(BS) * D;  // bf16 elements per page
  const uint8_t* kq = static_cast<const uint8_t*>(a.k_pool);
  const uint8_t* vq = static_cast<const uint8_t*>(a.v_pool);
  const size_t q8_page = static_cast<size_t>(BS) * D + 4 * BS;  // bytes per 8-bit page (codes, scales)

  // Rows of the workgroup and of this wave.
  const int wg_rows = NW * CG * 16 / G;
  const int wg_last = min(q_len - 1, t0 + wg_rows - 1);
  const int n_tiles = (off + wg_last) / kTile + 1;  // key tiles any row of the workgroup sees
  const int wave_c0 = wave * CG * 16;
  const int t_first = t0 + wave_c0 / G;
  const bool wave_live = t_first < q_len;
  const int t_last = min(q_len - 1, t0 + (wave_c0 + CG * 16 - 1) / G);
  const int wave_keys = off + t_last;  // last key of any column of the wave
  const float slack = kSlackLog2 / a.scale_log2;  // in raw-score units
  // The sequence's window (none: no sinks, a recent range beyond any length).
  // A windowed workgroup walks the tiles holding sink keys, then the tiles
  // from its first row's window start on; iteration i works on tile_of(i).
  const int win_sinks = a.seq_win[4 * b], win_recent = a.seq_win[4 * b + 1];
  const bool windowed = win_recent < kNoWindowRecent;
  const int t_win = windowed ? max(0, off + t0 + 1 - win_recent) / kTile : 0;
  const int n_sink = windowed ? min(t_win, (win_sinks + kTile - 1) / kTile) : 0;
  const int n_iter = n_sink + n_tiles - t_win;
  const int lo_wave = off + t_first + 1 - win_recent;  // window start of the wave's first row

  bf16x8 qv[CG][KS];
  int lim[CG], row[CG], head[CG];
#pragma unroll
  for (int k = 0; k < CG; ++k) {
    const int c = wave_c0 + k * 16 + n;
    row[k] = t0 + c / G;
    head[k] = g * G + c % G;
    // Columns past the last row are computed with its limit and not stored.
    lim[k] = off + min(row[k], q_len - 1);
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(q0 + min(row[k], q_len - 1)) * Hq + head[k]) * D + 8 * grp;
#pragma unroll
    for (int j = 0; j < KS; ++j) qv[k][j] = *reinterpret_cast<const bf16x8*>(qrow + 32 * j);
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

  // 8-bit: stage raw tile T into raw slot st.  Wave w < kCodeLoads moves 1 KB
  // of codes (the first half of the loads K codes, the second V codes) in
  // 16-byte chunks: token t's K codes fill row t (D bytes) with the chunks
  // permuted by q8_k_swizzle(t); each 16-token subtile of V codes keeps the
  // pages' operand order with its chunks permuted by q8_v_swizzle, so the
  // conversion reads below hit distinct LDS banks.  Wave 0's lanes 0-15 also
  // move the 32 K and 32 V row scales.  Pages past the sequence's last read zeros; slots
  // past its end inside the last page are staged as they are (finite codes;
  // their scales are never used, see the masked softmax).
  auto stage_q8 = [&](int T, int st) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(&raw[st][0]);
    int ent[PAGES];
#pragma unroll
    for (int p = 0; p < PAGES; ++p) {
      const int pg = T * PAGES + p;
      ent[p] = (T < n_tiles && pg < nblk) ? scalar_load(table, pg) : -1;
    }
    if (wave < kCodeLoads) {
      constexpr int kHalf = kCodeLoads / 2;  // loads per code region
      const bool isv = wave >= kHalf;
      const int o0 = (isv ? wave - kHalf : wave) * 1024;  // wave's first byte in the region
      const int P = o0 / 16 + lane;                        // 16-byte chunk this lane fills
      // The chunk's token (K) or first token of its 16-token subtile (V),
      // and its byte offset in the page (page order: k8_offset,
      // q8_v_offset; a 16-byte chunk is 16 consecutive codes of one K row
      // or of one V operand row).
      int tok0, at;
      if (!isv) {
        tok0 = P / kRowChunks;
        at = k8_offset(tok0 % BS, 16 * ((P % kRowChunks) ^ q8_k_swizzle(tok0)), D);
      } else {
        tok0 = 16 * (P / D);
        const int q = q8_v_swizzle(P % D);  // chunk q of the subtile: row q / (D/64), part q % (D/64)
        at = (tok0 % BS) * D + 16 * ((q % kRowChunksV) * 64 + q / kRowChunksV);
      }
      const int pgi = tok0 / BS;
      const int blk = pgi ? ent[PAGES - 1] : ent[0];
      const void* src = a.zeros;
      if (blk >= 0)
        src = (isv ? vq : kq) + (static_cast<size_t>(blk) * Hkv + g) * q8_page + at;
      __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)(dst + (isv ? kTile * D : 0) + o0), 16, 0, 0);
    }
    if (wave == 0 && lane < 16) {
      // Lane l: the scales of tokens 4(l % 8) .. +3, K for l < 8, V after.
      const int tok = 4 * (lane & 7);
      const int pgi = tok / BS;
      const int blk = pgi ? ent[PAGES - 1] : ent[0];
      const void* src = a.zeros;
      if (blk >= 0)
        src = (lane >= 8 ? vq : kq) + (static_cast<size_t>(blk) * Hkv + g) * q8_page + BS * D + 4 * (tok % BS);
      __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)(dst + 2 * kTile * D), 16, 0, 0);
    }
  };
  // Loads a wave issues per 8-bit tile, and waits that leave at most `tiles`
  // later tiles' loads outstanding (a wave-uniform count).
  const int q8_loads = (wave < kCodeLoads ? 1 : 0) + (wave == 0 ? 1 : 0);
  auto q8_wait = [&](auto tiles_c) {
    constexpr int kT = decltype(tiles_c)::value;
    if (q8_loads == 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kT, 0));
    else if (q8_loads == 1)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(kT, 0));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  };
  // 8-bit: convert raw slot rs into bf16 operand tile os (the operand order
  // of the bf16 ring; codes are exact in bf16, the scales stay apart in
  // fp32).  Waves 0-3 convert the K blocks (8 codes per lane, one 8-byte
  // read), waves 4-7 the V blocks: a lane reads the 16-byte chunks of its
  // two V rows (tokens 8grp .. +3 and +4 .. +7 of d = 16nt + n) once for all
  // the blocks it converts.
  static_assert(!Q8 || (NW == 8 && KB % 4 == 0 && DT % 4 == 0), "8-bit conversion split");
  constexpr int kKPW = KB / 4, kVPW = DT / 4;  // blocks per K / V converting wave
  int cv_off[kKPW > 0 ? kKPW : 1];
  int cv_vlo = 0, cv_vhi = 0;
  if (wave < 4) {
#pragma unroll
    for (int r = 0; r < kKPW; ++r) {
      const int blkid = wave * kKPW + r;
      const int tt = blkid / KS, j = blkid - tt * KS;
      const int tok = 8 * (n >> 2) + 4 * tt + (n & 3);
      const int c = 2 * j + (grp >> 1);  // 16-byte chunk of the row holding d = 32j + 8grp
      cv_off[r] = 16 * (tok * kRowChunks + (c ^ q8_k_swizzle(tok))) + 8 * (grp & 1);
    }
  } else {
    const int h = 4 * (wave - 4) * kVPW / 16;  // chunk of the row (4 bytes per d tile)
    const int row = 32 * (grp & 1) + n;        // operand-order row of tokens 8grp .. +3, d % 16 = n
    const int q_lo = kRowChunksV * row + h, q_hi = q_lo + 16 * kRowChunksV;
    cv_vlo = kTile * D + (grp >> 1) * 16 * D + 16 * q8_v_swizzle(q_lo);
    cv_vhi = kTile * D + (grp >> 1) * 16 * D + 16 * q8_v_swizzle(q_hi);
  }
  auto convert_q8 = [&](int rs, int os) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(&raw[rs][0]);
    if (wave < 4) {
#pragma unroll
      for (int r = 0; r < kKPW; ++r) {
        const uint2 c = *reinterpret_cast<const uint2*>(src + cv_off[r]);
        ring[os][wave * kKPW + r][lane] = __builtin_bit_cast(uint4, codes8_to_bf16x8<Q8>(c.x, c.y));
      }
    } else {
      const uint4 lo = *reinterpret_cast<const uint4*>(src + cv_vlo);
      const uint4 hi = *reinterpret_cast<const uint4*>(src + cv_vhi);
      const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w}, hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int r = 0; r < kVPW; ++r) {
        const int nt = (wave - 4) * kVPW + r;
        ring[os][KB + nt][lane] = __builtin_bit_cast(uint4, codes8_to_bf16x8<Q8>(lw[nt & 3], hw[nt & 3]));
      }
    }
  };

  // One key tile.  kMasked: some key of the tile lies past some column's
  // limit (the causal diagonal or the sequence end); kTail: the tile reaches
  // past the sequence end, so a V chunk that straddles it may hold stale
  // bits in its later slots, which are zeroed before they meet P = 0.  Tiles
  // every column sees whole take the instantiation with neither.
  auto compute_tile = [&](int T, int st, int rs, auto masked_c, auto tail_c, auto win_c) {
    constexpr bool kMasked = decltype(masked_c)::value;
    constexpr bool kTail = decltype(tail_c)::value;
    constexpr bool kWin = decltype(win_c)::value;
    static_assert(kMasked || !kWin, "windowed tiles are masked");
    // Under a window a page of the tile may have been released (-1 in the
    // table, staged as zeros): its keys are gone.  Pages past the sequence
    // end are not in the table; their keys lie past every limit anyway.
    bool lane_hole = false;
    if constexpr (kWin) {
      const int pg = T * PAGES + (8 * grp) / BS;
      const int e0 = T * PAGES < nblk ? scalar_load(table, T * PAGES) : 0;
      const int e1 = (PAGES > 1 && T * PAGES + 1 < nblk) ? scalar_load(table, T * PAGES + 1) : 0;
      lane_hole = pg < nblk && ((pg == T * PAGES) ? e0 : e1) < 0;
    }
    const bf16x8* blocks = reinterpret_cast<const bf16x8*>(&ring[st][0][0]);
    f32x4 s[CG][2];
#pragma unroll
    for (int k = 0; k < CG; ++k) s[k][0] = s[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The operands are read next to their MFMAs (this path converts the
    // next tile meanwhile; reading them all ahead was slower).
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const bf16x8 kop = blocks[(tt * KS + j) * 64 + lane];
#pragma unroll
        for (int k = 0; k < CG; ++k)
          s[k][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qv[k][j], s[k][tt], 0, 0, 0);
      }
    // s[k][tt][i] is the score of token T*32 + 8*grp + 4*tt + i for column n.
    // The row scales of this lane's 8 tokens: K's scale the scores, V's the
    // weights that enter P.V (not l).
    float sk[8], sv[8];
    {
      const float4* sc = reinterpret_cast<const float4*>(
          reinterpret_cast<const uint8_t*>(&raw[rs][0]) + 2 * kTile * D + 32 * grp);
      const float4 k0 = sc[0], k1 = sc[1], v0 = sc[kTile / 4], v1 = sc[kTile / 4 + 1];
      sk[0] = k0.x, sk[1] = k0.y, sk[2] = k0.z, sk[3] = k0.w;
      sk[4] = k1.x, sk[5] = k1.y, sk[6] = k1.z, sk[7] = k1.w;
      sv[0] = v0.x, sv[1] = v0.y, sv[2] = v0.z, sv[3] = v0.w;
      sv[4] = v1.x, sv[5] = v1.y, sv[6] = v1.z, sv[7] = v1.w;
    }
    bf16x8 p_hi[CG], p_lo[CG];
#pragma unroll
    for (int k = 0; k < CG; ++k) {
      float mloc = -INFINITY;
      // Key T*32 + 8*grp + x of this lane is visible to column n if x <= room
      // and, under a window, it is a sink (x < sink_rel) or inside the
      // column's recent range (x >= lo_rel), and its page is resident.
      const int base = T * kTile + 8 * grp;
      const int room = kMasked ? lim[k] - base : 0;
      const int lo_rel = kWin ? lim[k] + 1 - win_recent - base : 0;
      const int sink_rel = kWin ? win_sinks - base : 0;
      auto visible = [&](int x) {
        if constexpr (kWin) return x <= room && !lane_hole && (x < sink_rel || x >= lo_rel);
        return x <= room;
      };
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[k][tt][i];
          x *= sk[4 * tt + i];
          if (kMasked && !visible(4 * tt + i)) x = -INFINITY;
          s[k][tt][i] = x;
          mloc = fmaxf(mloc, x);
        }
      // The exponent reference m_run moves only when a score passes it by
      // more than `slack` (2^kSlackLog2 in weight), so weights stay at most
      // 2^kSlackLog2 and the accumulators are rescaled on few tiles: mostly
      // the first, where m_run is -inf and the factor is 0.  Every column
      // sees key 0 in tile 0, so m_run is finite from then on.  A lane's own
      // maximum decides whether any column may need it; only then does the
      // wave reduce each column's maximum over its four lanes (m_run stays
      // the same on the four).
      if (__builtin_amdgcn_ballot_w64(mloc > m_run[k] + slack)) {
        const float mcol = rows4_max(mloc);
        if (mcol > m_run[k] + slack) {
          const float alpha = exp2_flush((m_run[k] - mcol) * a.scale_log2);
          l_run[k] *= alpha;
#pragma unroll
          for (int nt = 0; nt < DT; ++nt) acc[k][nt] *= alpha;
          m_run[k] = mcol;
        }
      }
      // A column that has seen no visible key yet (m_run still -inf; only
      // on masked tiles) has every weight 0.
      const float ms = (kMasked && m_run[k] == -INFINITY) ? 0.f : m_run[k] * a.scale_log2;
      float psum = 0.f;
      uint32_t hi_w[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // Weights of tokens 2w, 2w+1 of this lane's 8.
        float e[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int idx = 2 * w + h;
          const float w8 = exp2_flush(fmaf(s[k][idx / 4][idx % 4], a.scale_log2, -ms));
          // A slot past the sequence end may hold any scale bits: its
          // weight is exactly 0 and must stay so.
          e[h] = w8 * sv[idx];
          if (kMasked && !visible(idx)) e[h] = 0.f;
          // hi = e with the low 16 bits cleared (a bf16 value); e - hi is exact
          // and enters P.V as a second bf16 term.
          const float lo = e[h] - __uint_as_float(__float_as_uint(e[h]) & 0xffff0000u);
          p_lo[k][idx] = static_cast<__bf16>(lo);
          psum += w8;
        }
        hi_w[w] = __builtin_amdgcn_perm(__float_as_uint(e[1]), __float_as_uint(e[0]), 0x07060302u);
      }
      p_hi[k] = __builtin_bit_cast(bf16x8, (uint4{hi_w[0], hi_w[1], hi_w[2], hi_w[3]}));
      l_run[k] += psum;
    }
    const int live = kTail ? L - (T * kTile + 8 * grp) : kTile;  // tokens of this lane's 8 inside the sequence
#pragma unroll
    for (int nt = 0; nt < DT; ++nt) {
      bf16x8 vop = blocks[(KB + nt) * 64 + lane];
      if constexpr (kTail && Q8 != 1) {  // int8 codes are always finite; E4M3 bytes may be NaN
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= live) vop[e] = static_cast<__bf16>(0.f);
      }
#pragma unroll
      for (int k = 0; k < CG; ++k) {
        acc[k][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, p_hi[k], acc[k][nt], 0, 0, 0);
        acc[k][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, p_lo[k], acc[k][nt], 0, 0, 0);
      }
    }
  };

  // Tiles below t_split are seen whole by every row of the workgroup and take
  // the unmasked path; the few after it (the causal diagonal, the sequence
  // end) take the masked one, which also keeps slots past the sequence end
  // out of P.V.  A windowed workgroup takes the masked path with the window
  // rule on all its tiles.  Every wave runs the same steps (the barrier
  // counts all of them).
  const int t_split = min(n_tiles, (off + t0 + 1) / kTile);
  auto tile_of = [&](int i) { return i < n_sink ? i : t_win + i - n_sink; };
  auto wave_sees = [&](int T) {
    return T * kTile <= wave_keys && (T * kTile < win_sinks || T * kTile + kTile - 1 >= lo_wave);
  };
  using F = std::false_type;
  using Tr = std::true_type;
  {
    // 8-bit step i: this wave's loads of the raw tile of iteration i+1 have
    // landed once at most those of iteration i+2 are outstanding; the barrier
    // publishes that raw tile and the bf16 tile of iteration i (converted in
    // step i-1) and guarantees every wave has left step i-1, the last reader
    // of raw slot (i-1) % S (its scales) and of bf16 tile (i+1) % 2 (then
    // iteration i-1's).  Step i stages the raw tile of iteration i+S-1 into
    // the former, converts iteration i+1's into the latter and computes
    // iteration i's.
    auto step = [&](int i) {
      q8_wait(std::integral_constant<int, S - 3>{});
      __builtin_amdgcn_s_barrier();
      stage_q8(tile_of(i + S - 1), (i + S - 1) % S);
      convert_q8((i + 1) % S, (i + 1) & 1);
    };
#pragma unroll
    for (int i = 0; i < S - 1; ++i) stage_q8(tile_of(i), i);
    q8_wait(std::integral_constant<int, S - 2>{});  // the first raw tile
    __builtin_amdgcn_s_barrier();
    convert_q8(0, 0);
    int i = 0;
    if (!wave_live) {
      for (; i < n_iter; ++i) step(i);
    } else if (!windowed) {
      for (; i < t_split; ++i) {
        step(i);
        compute_tile(i, i & 1, i % S, F{}, F{}, F{});
      }
      for (; i < n_tiles; ++i) {
        step(i);
        if (i * kTile <= wave_keys) compute_tile(i, i & 1, i % S, Tr{}, Tr{}, F{});
      }
    } else {
      for (; i < n_iter; ++i) {
        step(i);
        const int T = tile_of(i);
        if (wave_sees(T)) compute_tile(T, i & 1, i % S, Tr{}, Tr{}, Tr{});
      }
    }
  }
  // Drain the zero-tile loads still in flight before the workgroup's LDS is
  // released.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  if (!wave_live) return;
#pragma unroll
  for (int k = 0; k < CG; ++k) {
    const float l = rows4_sum(l_run[k]);
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

// prefill_bf16_mfma32<D, BS, NW, S>  (bf16 pages; D in {64, 128}, BS in {16, 32}, G | 16)
//   The same computation on v_mfma_f32_32x32x16_bf16 tiles: one workgroup of
//   NW waves = (sequence, block of query rows, KV head); each wave owns 32
//   columns (query row, head) and each lane exactly one of them (column
//   lane % 32; lanes l and l ^ 32 share it).  Per 32-token key tile:
//     S^T[32 tok x 32 col] = K_tile . Q^T      (D/16 k-steps)
//     O^T[32 d x 32 col] += V^T_tile . P^T     (2 token k-steps x D/32 d blocks, P as hi + lo)
//   Each 1 KB operand read from LDS feeds a 32x32x16 MFMA (twice the flops
//   of a 16x16x32 one), and the per-tile softmax bookkeeping is shared by
//   32 columns.  Row m of the QK tile is token 16*(m/16) + 8*((m/4)%2) +
//   4*((m/8)%2) + m%4, so accumulator element j of lane l is token 16*(j/8) +
//   8*(l/32) + j%8: the lane's P^T operand of token k-step s is its own
//   elements 8s .. 8s+7, and the matching V^T operand (d = 32db + l%32,
//   tokens 16s + 8*(l/32) .. +7) is 16 contiguous bytes of a V page row.
//   Staging, windows, masks and the exponent reference follow
//   prefill_q8_mfma above (with bf16 operand tiles staged directly).  Each
//   workgroup uses a 48 KB ring and 168 registers per lane, so a CU holds
//   three of them (three waves per SIMD).  The staging step fetches the
//   block-table entries of the next tile one step ahead, so their scalar
//   loads are never waited for on a tile's path.
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D, int BS, int NW, int S>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3))) void prefill_bf16_mfma32(PrefillArgs a) {
  constexpr int KS = D / 16;         // QK k-steps (16 d each) per key tile
  constexpr int DB = D / 32;         // 32-row d blocks of P.V
  constexpr int KB = KS;             // K operand blocks per key tile
  constexpr int NB = KB + 2 * DB;    // operand blocks per key tile (V: token k-step s, d block db)
  constexpr int PAGES = kTile / BS;  // pages per key tile
  static_assert(NB % NW == 0, "each wave stages the same number of blocks");
  constexpr int BPW = NB / NW;
  static_assert((S - 2) * BPW < 64, "vmcnt range");
  // Optionally the Q^T operands live in LDS (each wave reads only its own)
  // instead of 8 registers per k-step.
  constexpr bool kQInLds = PA_PREFILL32_Q_LDS != 0;
  __shared__ uint4 ring[S][NB][64];
  __shared__ uint4 qlds[kQInLds ? NW : 1][kQInLds ? KS : 1][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int cl = lane & 31, hf = lane >> 5;  // column of the lane in the wave, half of the wave
  const int Hkv = a.num_kv_heads, Hq = a.num_heads, G = a.group;
  const int tile = blockIdx.x / Hkv, g = blockIdx.x - tile * Hkv;
  const int b = a.tiles[2 * tile], t0 = a.tiles[2 * tile + 1];
  const int q0 = a.q_start[b];
  const int q_len = a.q_start[b + 1] - q0;
  const int L = a.ctx_len[b];
  const int off = L - q_len;  // row t sees keys 0 .. off + t
  const int nblk = (L + BS - 1) / BS;
  const int32_t* table = a.tables + a.tbl_off[b];
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  const size_t page = static_cast<size_t>(BS) * D;

  const int wg_rows = NW * 32 / G;
  const int wg_last = min(q_len - 1, t0 + wg_rows - 1);
  const int n_tiles = (off + wg_last) / kTile + 1;
  const int wave_c0 = wave * 32;
  const int t_first = t0 + wave_c0 / G;
  const bool wave_live = t_first < q_len;
  const int t_last = min(q_len - 1, t0 + (wave_c0 + 31) / G);
  const int wave_keys = off + t_last;
  const float slack = kSlackLog2 / a.scale_log2;
  const int win_sinks = a.seq_win[4 * b], win_recent = a.seq_win[4 * b + 1];
  const bool windowed = win_recent < kNoWindowRecent;
  const int t_win = windowed ? max(0, off + t0 + 1 - win_recent) / kTile : 0;
  const int n_sink = windowed ? min(t_win, (win_sinks + kTile - 1) / kTile) : 0;
  const int n_iter = n_sink + n_tiles - t_win;
  const int lo_wave = off + t_first + 1 - win_recent;

  const int c = wave_c0 + cl;
  const int row = t0 + c / G, head = g * G + c % G;
  const int lim = off + min(row, q_len - 1);  // columns past the last row use its limit, not stored
  bf16x8 qv[kQInLds ? 1 : KS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<size_t>(q0 + min(row, q_len - 1)) * Hq + head) * D + 8 * hf;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qrow + 16 * j);
      if constexpr (kQInLds) qlds[wave][j][lane] = __builtin_bit_cast(uint4, v);
      else qv[j] = v;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;

  // Per-lane offsets of this wave's blocks inside their page and the page of
  // the tile each comes from.
  int blk_off[BPW], blk_pgi[BPW];
#pragma unroll
  for (int r = 0; r < BPW; ++r) {
    const int blkid = wave * BPW + r;
    if (blkid < KB) {
      const int m = cl;
      const int tok = 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
      blk_pgi[r] = tok / BS;
      blk_off[r] = k16_offset(tok % BS, 16 * blkid + 8 * hf, D, BS);
    } else {
      const int v = blkid - KB, ks = v / DB, db = v - ks * DB;
      const int tok = 16 * ks + 8 * hf;
      blk_pgi[r] = tok / BS;
      blk_off[r] = (32 * db + cl) * BS + tok % BS;
    }
  }

  // Table entries of tile T's pages (-1: released by a window; -2: past the
  // sequence or past the last tile), fetched one staging step before they
  // are used so the scalar loads are not waited for on the tile's path.
  auto load_ent = [&](int T, int* ent) {
#pragma unroll
    for (int p = 0; p < PAGES; ++p) {
      const int pg = T * PAGES + p;
      ent[p] = (T < n_tiles && pg < nblk) ? scalar_load(table, pg) : -2;
    }
  };
  auto stage = [&](int T, int st, const int* ent) {
    if (T < n_tiles && T * kTile + kTile <= L && ent[0] >= 0 && ent[PAGES - 1] >= 0) {
#pragma unroll
      for (int r = 0; r < BPW; ++r) {
        const int blkid = wave * BPW + r;
        const uint16_t* pool = blkid < KB ? kpool : vpool;
        const uint16_t* base0 = uniform_ptr(pool + (static_cast<size_t>(ent[0]) * Hkv + g) * page);
        const uint16_t* base1 = uniform_ptr(pool + (static_cast<size_t>(ent[PAGES - 1]) * Hkv + g) * page);
        const uint16_t* src = (blk_pgi[r] ? base1 : base0) + blk_off[r];
        __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)&ring[st][blkid][0], 16, 0, 0);
      }
      return;
    }
    // Slow path: the tile reaches past the sequence end, a page was
    // released, or the tile is past the last one (kept for uniform vmcnt).
#pragma unroll
    for (int r = 0; r < BPW; ++r) {
      const int blkid = wave * BPW + r;
      int tok;
      if (blkid < KB) {
        const int m = cl;
        tok = 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
      } else {
        const int v = blkid - KB, ks = v / DB;
        tok = 16 * ks + 8 * hf;
      }
      const int pgi = tok / BS;
      const int blk = pgi ? ent[PAGES - 1] : ent[0];
      const void* src = a.zeros;
      if (T * kTile + tok < L && blk >= 0)
        src = (blkid < KB ? kpool : vpool) + (static_cast<size_t>(blk) * Hkv + g) * page + blk_off[r];
      __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)&ring[st][blkid][0], 16, 0, 0);
    }
  };

  // S^T of the tile in ring slot st: D/16 MFMAs over K operands read from
  // LDS ahead of the first one.
  auto qk = [&](int st) {
    const bf16x8* blocks = reinterpret_cast<const bf16x8*>(&ring[st][0][0]);
    bf16x8 kops[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) kops[i] = blocks[i * 64 + lane];
    f32x16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      bf16x8 qop;
      if constexpr (kQInLds) qop = __builtin_bit_cast(bf16x8, qlds[wave][j][lane]);
      else qop = qv[j];
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kops[j], qop, sc, 0, 0, 0);
    }
    return sc;
  };

  // Softmax of tile T's scores `sc` (masks per kMasked / kWin, see above)
  // and its P.V step over the V operands of ring slot st.
  auto soft_pv = [&](int T, int st, f32x16 sc, auto masked_c, auto tail_c, auto win_c) {
    constexpr bool kMasked = decltype(masked_c)::value;
    constexpr bool kTail = decltype(tail_c)::value;
    constexpr bool kWin = decltype(win_c)::value;
    static_assert(kMasked || !kWin, "windowed tiles are masked");
    // Released pages under a window: token k-step s of this lane lies in
    // page T*PAGES + 16s/BS.
    bool hole[2] = {false, false};
    if constexpr (kWin) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int pg = T * PAGES + (16 * s2) / BS;
        hole[s2] = pg < nblk && scalar_load(table, pg) < 0;
      }
    }
    const bf16x8* blocks = reinterpret_cast<const bf16x8*>(&ring[st][0][0]);
    // sc[j] is the score of key T*32 + 16*(j/8) + 8*hf + j%8 for this column.
    const int base = T * kTile + 8 * hf;
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float x = sc[j];
      if constexpr (kMasked) {
        const int key = base + 16 * (j >> 3) + (j & 7);
        bool vis = key <= lim;
        if constexpr (kWin) vis = vis && !hole[j >> 3] && (key < win_sinks || key > lim - win_recent);
        if (!vis) x = -INFINITY;
      }
      sc[j] = x;
      mloc = fmaxf(mloc, x);
    }
    // Lazy exponent reference (as above): moves only when a score passes it
    // by more than `slack`; the column's two lanes agree on it.
    if (__builtin_amdgcn_ballot_w64(mloc > m_run + slack)) {
      auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
      const float mcol = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      if (mcol > m_run + slack) {
        const float alpha = exp2_flush((m_run - mcol) * a.scale_log2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        m_run = mcol;
      }
    }
    const float ms = (kMasked && m_run == -INFINITY) ? 0.f : m_run * a.scale_log2;
    float psum = 0.f;
    bf16x8 p_hi[2], p_lo[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      uint32_t hw[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float e[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int j = 8 * s2 + 2 * w + h2;
          e[h2] = exp2_flush(fmaf(sc[j], a.scale_log2, -ms));
          const float lo = e[h2] - __uint_as_float(__float_as_uint(e[h2]) & 0xffff0000u);
          p_lo[s2][2 * w + h2] = static_cast<__bf16>(lo);
          psum += e[h2];
        }
        hw[w] = __builtin_amdgcn_perm(__float_as_uint(e[1]), __float_as_uint(e[0]), 0x07060302u);
      }
      p_hi[s2] = __builtin_bit_cast(bf16x8, (uint4{hw[0], hw[1], hw[2], hw[3]}));
    }
    l_run += psum;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int live = kTail ? L - (base + 16 * s2) : 8;  // keys of the lane's 8 inside the sequence
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8 vop = blocks[(KB + s2 * DB + db) * 64 + lane];
        if constexpr (kTail) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= live) vop[e] = static_cast<__bf16>(0.f);
        }
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, p_hi[s2], acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, p_lo[s2], acc[db], 0, 0, 0);
      }
    }
  };

  const int t_split = min(n_tiles, (off + t0 + 1) / kTile);
  auto tile_of = [&](int i) { return i < n_sink ? i : t_win + i - n_sink; };
  auto wave_sees = [&](int T) {
    return T * kTile <= wave_keys && (T * kTile < win_sinks || T * kTile + kTile - 1 >= lo_wave);
  };
  using F = std::false_type;
  using Tr = std::true_type;
  int ent_next[PAGES];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) {
    load_ent(tile_of(i), ent_next);
    stage(tile_of(i), i, ent_next);
  }
  load_ent(tile_of(S - 1), ent_next);
  auto step = [&](int i) {
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((S - 2) * BPW, 0));
    __builtin_amdgcn_s_barrier();
    stage(tile_of(i + S - 1), (i + S - 1) % S, ent_next);
    load_ent(tile_of(i + S), ent_next);
  };
  int i = 0;
  if (!wave_live) {
    for (; i < n_iter; ++i) step(i);
  } else if (!windowed) {
    for (; i < t_split; ++i) {
      step(i);
      soft_pv(i, i % S, qk(i % S), F{}, F{}, F{});
    }
    for (; i < n_tiles; ++i) {
      step(i);
      if (i * kTile <= wave_keys) soft_pv(i, i % S, qk(i % S), Tr{}, Tr{}, F{});
    }
  } else {
    for (; i < n_iter; ++i) {
      step(i);
      const int T = tile_of(i);
      if (wave_sees(T)) soft_pv(T, i % S, qk(i % S), Tr{}, Tr{}, Tr{});
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  if (!wave_live) return;
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
  const float l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (row >= q_len) return;
  const float inv = 1.f / l;
  uint16_t* o = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(q0 + row) * Hq + head) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // acc[db][4 q4 + r] is d = 32 db + 8 q4 + 4 hf + r.
      uint2 packed;
      packed.x = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * q4 + 0] * inv)) |
                 (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * q4 + 1] * inv)) << 16);
      packed.y = static_cast<uint32_t>(f32_to_bf16(acc[db][4 * q4 + 2] * inv)) |
                 (static_cast<uint32_t>(f32_to_bf16(acc[db][4 * q4 + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(o + 32 * db + 8 * q4 + 4 * hf) = packed;
    }
}

template <int D, int BS, int Q8>
void launch_mfma(const PrefillArgs& a, hipStream_t stream, const KernelEvents& ev) {
  const dim3 grid(a.n_tiles * a.num_kv_heads);
  if constexpr (Q8 == 0) {
    PA_LAUNCH(ev, (prefill_bf16_mfma32<D, BS, kPrefill32Waves, kPrefill32Stages>), grid,
              dim3(64 * kPrefill32Waves), 0, stream, a);
  } else {
    PA_LAUNCH(ev, (prefill_q8_mfma<D, BS, kPrefillCG, kPrefillWaves, kPrefillStagesQ8, Q8>), grid,
              dim3(64 * kPrefillWaves), 0, stream, a);
  }
}

template <int Q8>
void launch_mfma_shape(int D, int BS, const PrefillArgs& a, hipStream_t stream, const KernelEvents& ev) {
  if (D == 128 && BS == 16) launch_mfma<128, 16, Q8>(a, stream, ev);
  else if (D == 128 && BS == 32) launch_mfma<128, 32, Q8>(a, stream, ev);
  else if (D == 64 && BS == 16) launch_mfma<64, 16, Q8>(a, stream, ev);
  else launch_mfma<64, 32, Q8>(a, stream, ev);
}

}  // namespace

bool prefill_uses_mfma(const PoolGeom& geom, int32_t group) {
  const bool d_ok = geom.head_dim == 64 || geom.head_dim == 128;
  const bool bs_ok = geom.block_size == 16 || geom.block_size == 32;
  const bool g_ok = group >= 1 && group <= 16 && 16 % group == 0;
  return (geom.dtype == 1 || geom.q8()) && d_ok && bs_ok && g_ok;
}

int32_t prefill_rows_per_tile(const PoolGeom& geom, int32_t group) {
  if (!prefill_uses_mfma(geom, group)) return 64;
  if (!geom.q8()) return kPrefill32Waves * 32 / group;
  return kPrefillWaves * kPrefillCG * 16 / group;
}

hipError_t launch_prefill(const PoolGeom& geom, const PrefillArgs& a, hipStream_t stream,
                          const KernelEvents& ev) {
  if (!prefill_uses_mfma(geom, a.group)) return launch_prefill_generic(geom, a, stream, ev);
  if (geom.fp8()) launch_mfma_shape<2>(geom.head_dim, geom.block_size, a, stream, ev);
  else if (geom.q8()) launch_mfma_shape<1>(geom.head_dim, geom.block_size, a, stream, ev);
  else launch_mfma_shape<0>(geom.head_dim, geom.block_size, a, stream, ev);
  return hipGetLastError();
}

}  // namespace pa
