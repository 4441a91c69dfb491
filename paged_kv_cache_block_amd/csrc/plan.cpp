// Decode / prefill work plans.  See plan.hpp.
#include "plan.hpp"

#include <algorithm>
#include <numeric>

namespace pa {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Append `n` zero words to `meta`, 4-word aligned, and return the byte offset.
size_t reserve(std::vector<int32_t>& meta, size_t n) {
  size_t at = align_up(meta.size(), 4);
  meta.resize(at + n, 0);
  return at * sizeof(int32_t);
}

int32_t* at_bytes(std::vector<int32_t>& meta, size_t byte_off) {
  return meta.data() + byte_off / sizeof(int32_t);
}

// Workgroups a decode launch aims for: two resident groups (8 waves) on each
// of the 256 CUs.  Longer page ranges mean fewer split-K partials to write,
// merge and reduce across waves; measured against a target of 2048 groups,
// 4-row verify steps ran 9% faster, long contexts 4% and windowed steps 7%,
// one-row decode the same.
#ifndef PA_DECODE_TARGET_GROUPS
#define PA_DECODE_TARGET_GROUPS 512
#endif
constexpr int64_t kTargetGroups = PA_DECODE_TARGET_GROUPS;
// Rows of about equal visited length (the longest at most 5/4 of the mean)
// that already give each of the 256 CUs a workgroup are not split: ranges
// would only add split-K partial rows and the merge kernel.  Measured on 32
// windowed rows of 66 pages each (256 workgroups): step 35.6 vs 40.1 us,
// kernel 25.2-25.7 vs 26.4-30.2 us.
constexpr int64_t kUnsplitGroups = 256;

struct Item { int32_t b, c, pages; };

// Per-thread scratch of build_decode_plan, reused across calls so that a
// steady stream of decode steps allocates nothing on the host.
struct DecodeScratch {
  std::vector<const Sequence*> rows;
  std::vector<int64_t> len, nblk, nvis;
  std::vector<int32_t> qlen, win, n_parts_of, part_base, merge;
  std::vector<Item> items, tails;
};

DecodeScratch& decode_scratch() {
  thread_local DecodeScratch scratch;
  return scratch;
}

}  // namespace

Status build_decode_plan(const BlockPool& pool, const int64_t* seqs, int32_t B, int32_t num_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t tokens_per_part,
                         const int32_t* extra_tokens, const int32_t* q_lens, int32_t slot_count,
                         DecodePlan* plan, std::string* msg) {
  if (B <= 0 || !seqs) {
    *msg = "batch must be positive with a non-NULL seqs array";
    return kInvalidArg;
  }
  if (num_heads <= 0 || num_heads % num_kv_heads) {
    *msg = "num_heads must be a positive multiple of num_kv_heads";
    return kInvalidArg;
  }
  const int32_t bs = pool.block_size();
  DecodeScratch& scr = decode_scratch();
  std::vector<const Sequence*>& rows = scr.rows;
  std::vector<int64_t>&len = scr.len, &nblk = scr.nblk, &nvis = scr.nvis;
  rows.assign(B, nullptr);
  len.assign(B, 0);
  nblk.assign(B, 0);
  nvis.assign(B, 0);
  int64_t total_pages = 0;
  for (int32_t b = 0; b < B; ++b) {
    rows[b] = pool.find(seqs[b]);
    if (!rows[b]) {
      *msg = "unknown sequence: " + std::to_string(seqs[b]);
      return kUnknownSeq;
    }
    len[b] = rows[b]->length + (extra_tokens ? extra_tokens[b] : 0);
    nblk[b] = ceil_div(len[b], bs);
    if (len[b] == 0) {
      *msg = "kv_len must be positive (sequence " + std::to_string(seqs[b]) + " is empty)";
      return kInvalidArg;
    }
    if (q_lens && (q_lens[b] < 1 || q_lens[b] > len[b])) {
      *msg = "q_lens[b] must be in 1..length(seq) (the rows are the last positions)";
      return kInvalidArg;
    }
    total_pages += nblk[b];
  }
  std::vector<int32_t>& qlen = scr.qlen;
  std::vector<int32_t>& win = scr.win;
  qlen.assign(B, 1);
  win.assign(4 * static_cast<size_t>(B), 0);
  int64_t n_rows = B;
  int32_t max_q = 1;
  if (q_lens) {
    n_rows = 0;
    for (int32_t b = 0; b < B; ++b) {
      qlen[b] = q_lens[b];
      n_rows += qlen[b];
      max_q = std::max(max_q, qlen[b]);
    }
    if (n_rows > INT32_MAX / 2) {
      *msg = "too many query rows";
      return kInvalidArg;
    }
  }
  // Pages each sequence's rows may see: the sink pages, then from the first
  // page of row 0's window (or the first resident page after released ones).
  for (int32_t b = 0; b < B; ++b) {
    const Sequence& s = *rows[b];
    int32_t* w = &win[4 * static_cast<size_t>(b)];
    if (!s.windowed()) {
      w[0] = 0;
      w[1] = kNoWindowRecent;
      w[2] = static_cast<int32_t>(nblk[b]);
      w[3] = 0;
      nvis[b] = nblk[b];
      continue;
    }
    if (len[b] - qlen[b] < pool.evicted_end(s)) {
      *msg = "a query row of sequence " + std::to_string(seqs[b]) + " lies in a released page";
      return kInvalidArg;
    }
    const int64_t sink_pages = std::min<int64_t>(ceil_div(s.sinks, bs), nblk[b]);
    const int64_t lo = std::max<int64_t>(0, len[b] - qlen[b] + 1 - s.recent);
    int64_t start = std::max<int64_t>(lo / bs, sink_pages);
    start = std::max<int64_t>(start, pool.evicted_end(s) / bs);
    start = std::min<int64_t>(start, nblk[b]);
    w[0] = s.sinks;
    w[1] = s.recent;
    w[2] = static_cast<int32_t>(sink_pages);
    w[3] = static_cast<int32_t>(start - sink_pages);
    nvis[b] = nblk[b] - (start - sink_pages);
  }

  // Pages per partition: the largest candidate that still yields enough
  // workgroups; each partition is split over kDecodeWaves waves.
  auto pages_for = [&](int64_t tokens) {
    int64_t p = std::max<int64_t>(1, tokens / bs);
    return static_cast<int32_t>(align_up(static_cast<size_t>(p), kDecodeWaves));
  };
  auto groups_for = [&](int32_t ppp) {
    int64_t g = 0;
    for (int32_t b = 0; b < B; ++b) g += ceil_div(nvis[b], ppp);
    return g * num_kv_heads;
  };
  int64_t max_vis = 0, sum_vis = 0;
  for (int32_t b = 0; b < B; ++b) {
    max_vis = std::max(max_vis, nvis[b]);
    sum_vis += nvis[b];
  }
  int32_t ppp;
  if (tokens_per_part > 0) {
    ppp = pages_for(tokens_per_part);
  } else if (static_cast<int64_t>(B) * num_kv_heads >= kUnsplitGroups &&
             4 * static_cast<int64_t>(B) * max_vis <= 5 * sum_vis) {
    ppp = static_cast<int32_t>(align_up(static_cast<size_t>(max_vis), kDecodeWaves));
  } else {
    static const int64_t kCandidates[] = {4096, 2048, 1024, 512, 256, 128};
    ppp = pages_for(128);
    for (int64_t tok : kCandidates) {
      int32_t p = pages_for(tok);
      if (groups_for(p) >= kTargetGroups) {
        ppp = p;
        break;
      }
    }
  }

  std::vector<int32_t>& n_parts_of = scr.n_parts_of;
  n_parts_of.assign(B, 0);
  // Longest page ranges first so short tails fill in at the end: the full
  // ranges in sequence order, then the shorter last ranges (at most one per
  // sequence) by decreasing length, ties in sequence order.
  // A sizing-only plan (extra_tokens) counts the items and merge rows
  // without listing them.
  const bool sizing = extra_tokens != nullptr;
  std::vector<Item>&items = scr.items, &tails = scr.tails;
  items.clear();
  tails.clear();
  std::vector<int32_t>&part_base = scr.part_base, &merge = scr.merge;
  part_base.assign(B, -1);
  merge.clear();
  int32_t n_parts = 0;
  int64_t row_heads = 0, n_work = 0, n_merge = 0, row_start = 0;
  for (int32_t b = 0; b < B; ++b) {
    int32_t nb = static_cast<int32_t>(nvis[b]);
    int32_t np = static_cast<int32_t>(ceil_div(nb, ppp));
    n_parts_of[b] = np;
    n_work += np;
    if (!sizing) {
      for (int32_t c = 0; c < np; ++c) {
        const int32_t pages = std::min(ppp, nb - c * ppp);
        (pages == ppp ? items : tails).push_back({b, c, pages});
      }
    }
    if (np > 1) {
      if (row_heads + static_cast<int64_t>(np) * qlen[b] * num_heads > INT32_MAX) {
        *msg = "too many split-K partial rows";
        return kInvalidArg;
      }
      part_base[b] = static_cast<int32_t>(row_heads);
      row_heads += static_cast<int64_t>(np) * qlen[b] * num_heads;
      n_parts += np;
      n_merge += qlen[b];
      if (!sizing) {
        for (int32_t t = 0; t < qlen[b]; ++t) {
          merge.push_back(static_cast<int32_t>(row_start + t));
          merge.push_back(part_base[b] + t * num_heads);
          merge.push_back(qlen[b] * num_heads);
          merge.push_back(np);
        }
      }
    }
    row_start += qlen[b];
  }
  std::stable_sort(tails.begin(), tails.end(),
                   [](const Item& x, const Item& y) { return x.pages > y.pages; });
  items.insert(items.end(), tails.begin(), tails.end());

  DecodePlan p;
  p.batch = B;
  p.pages_per_part = ppp;
  p.n_work = static_cast<int32_t>(n_work);
  p.n_merge = static_cast<int32_t>(n_merge);
  p.n_parts = n_parts;
  p.n_rows = static_cast<int32_t>(n_rows);
  p.max_q_len = max_q;
  p.total_pages = total_pages;
  // Section offsets (4-word aligned), then one allocation for all of them.
  size_t words = 0;
  auto place = [&](size_t n) {
    const size_t at = align_up(words, 4);
    words = at + n;
    return at * sizeof(int32_t);
  };
  p.ctx_off = place(B);
  p.tbl_off_off = place(B);
  p.qstart_off = place(B + 1);
  p.base_off = place(B);
  p.nparts_off = place(B);
  p.win_off = place(4 * static_cast<size_t>(B));
  p.work_off = place(kWorkInts * static_cast<size_t>(n_work));
  p.merge_off = place(std::max<size_t>(4, 4 * static_cast<size_t>(n_merge)));
  // Tables hold the visited pages only (a windowed sequence: its sink pages,
  // then its pages from the first row's window on), indexed by the compact
  // page index the kernels walk.
  int64_t visited_pages = 0;
  for (int32_t b = 0; b < B; ++b) visited_pages += nvis[b];
  p.tables_off = place(static_cast<size_t>(visited_pages));
  p.slots_off = place(2 * static_cast<size_t>(std::max(slot_count, 0)));
  const size_t rows_hq = static_cast<size_t>(row_heads);
  p.meta_bytes = align_up(words * sizeof(int32_t), kWsAlign);
  p.part_m_off = p.meta_bytes;
  p.part_l_off = p.part_m_off + align_up(rows_hq * sizeof(float), kWsAlign);
  p.part_acc_off = p.part_l_off + align_up(rows_hq * sizeof(float), kWsAlign);
  p.total_bytes = p.part_acc_off + align_up(rows_hq * head_dim * sizeof(float), kWsAlign);
  if (sizing) {  // sizing only: the sections are not filled
    *plan = std::move(p);
    return kOk;
  }
  // The caller's previous plan buffer is reused (no allocation once it is
  // large enough).  Every section is written below; the alignment padding
  // between sections is never read, so the buffer is not cleared.
  std::vector<int32_t>& meta = p.meta;
  meta = std::move(plan->meta);
  meta.resize(words);
  int32_t* ctx = at_bytes(meta, p.ctx_off);
  int32_t* toff = at_bytes(meta, p.tbl_off_off);
  int32_t* base = at_bytes(meta, p.base_off);
  int32_t* npo = at_bytes(meta, p.nparts_off);
  int32_t* work = at_bytes(meta, p.work_off);
  int32_t* mrg = at_bytes(meta, p.merge_off);
  int32_t* tables = at_bytes(meta, p.tables_off);
  int32_t* qs = at_bytes(meta, p.qstart_off);
  int64_t cursor = 0;
  int32_t row = 0;
  for (int32_t b = 0; b < B; ++b) {
    qs[b] = row;
    row += qlen[b];
    ctx[b] = static_cast<int32_t>(len[b]);
    toff[b] = static_cast<int32_t>(cursor);
    base[b] = part_base[b];
    npo[b] = n_parts_of[b];
    const int32_t* w8 = &win[4 * static_cast<size_t>(b)];
    const std::vector<int32_t>& tb = rows[b]->table;  // nblk[b] entries (not a sizing plan)
    std::copy(tb.begin(), tb.begin() + w8[2], tables + cursor);
    std::copy(tb.begin() + w8[2] + w8[3], tb.begin() + nblk[b], tables + cursor + w8[2]);
    cursor += nvis[b];
  }
  for (size_t i = 0; i < items.size(); ++i) {
    const int32_t b = items[i].b, c = items[i].c;
    const int32_t* w8 = &win[4 * static_cast<size_t>(b)];
    int32_t* w = work + kWorkInts * i;
    w[0] = b;
    w[1] = c;
    w[2] = ctx[b];
    w[3] = qs[b];
    w[4] = qlen[b];
    w[5] = w8[0];
    w[6] = w8[1];
    w[7] = w8[2];
    w[8] = w8[3];
    w[9] = toff[b];
    w[10] = part_base[b];
    w[11] = 0;
    const int64_t p0 = static_cast<int64_t>(c) * ppp, p1 = std::min<int64_t>(nvis[b], p0 + ppp);
    for (int32_t wave = 0; wave < kDecodeWaves; ++wave) {
      const int64_t ci = p0 + wave;
      const int64_t page = ci < w8[2] ? ci : ci + w8[3];
      w[12 + wave] = (ci < p1 && static_cast<size_t>(page) < rows[b]->table.size())
                         ? rows[b]->table[static_cast<size_t>(page)]
                         : 0;
    }
  }
  qs[B] = row;
  std::copy(merge.begin(), merge.end(), mrg);
  std::copy(win.begin(), win.end(), at_bytes(meta, p.win_off));
  *plan = std::move(p);
  return kOk;
}

Status build_prefill_plan(const BlockPool& pool, const int64_t* seqs, const int32_t* q_lens,
                          int32_t B, int32_t num_heads, int32_t num_kv_heads, int32_t rows_per_tile,
                          PrefillPlan* plan, std::string* msg) {
  if (B <= 0 || !seqs || !q_lens) {
    *msg = "batch must be positive with non-NULL seqs and q_lens";
    return kInvalidArg;
  }
  if (num_heads <= 0 || num_heads % num_kv_heads) {
    *msg = "num_heads must be a positive multiple of num_kv_heads";
    return kInvalidArg;
  }
  std::vector<const Sequence*> rows(B);
  int64_t total_pages = 0, total_rows = 0;
  for (int32_t b = 0; b < B; ++b) {
    rows[b] = pool.find(seqs[b]);
    if (!rows[b]) {
      *msg = "unknown sequence: " + std::to_string(seqs[b]);
      return kUnknownSeq;
    }
    if (q_lens[b] < 1 || q_lens[b] > rows[b]->length) {
      *msg = "q_lens[b] must be in 1..length(seq) (the rows are the last positions)";
      return kInvalidArg;
    }
    if (rows[b]->length - q_lens[b] < pool.evicted_end(*rows[b])) {
      *msg = "a query row of sequence " + std::to_string(seqs[b]) + " lies in a released page";
      return kInvalidArg;
    }
    total_pages += static_cast<int64_t>(rows[b]->table.size());
    total_rows += q_lens[b];
  }
  if (total_rows > INT32_MAX / 2) {
    *msg = "too many query rows";
    return kInvalidArg;
  }
  struct Tile { int32_t b, t0; int64_t keys; };
  std::vector<Tile> tiles;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t t0 = 0; t0 < q_lens[b]; t0 += rows_per_tile) {
      int32_t last = std::min(q_lens[b], t0 + rows_per_tile) - 1;
      int64_t keys = rows[b]->length - q_lens[b] + last + 1;
      if (rows[b]->windowed())  // the sinks and the rows' windows
        keys = std::min<int64_t>(keys, static_cast<int64_t>(rows[b]->sinks) + rows[b]->recent + rows_per_tile);
      tiles.push_back({b, t0, keys});
    }
  // Tiles that see the most keys first.
  std::stable_sort(tiles.begin(), tiles.end(),
                   [](const Tile& x, const Tile& y) { return x.keys > y.keys; });

  PrefillPlan p;
  p.batch = B;
  p.n_tiles = static_cast<int32_t>(tiles.size());
  p.n_rows = static_cast<int32_t>(total_rows);
  std::vector<int32_t>& meta = p.meta;
  p.ctx_off = reserve(meta, B);
  p.tbl_off_off = reserve(meta, B);
  p.qstart_off = reserve(meta, B + 1);
  p.tiles_off = reserve(meta, 2 * tiles.size());
  p.rowseq_off = reserve(meta, static_cast<size_t>(total_rows));
  p.zeros_off = reserve(meta, 16);  // 64 bytes, left zero
  p.win_off = reserve(meta, 4 * static_cast<size_t>(B));
  p.tables_off = reserve(meta, static_cast<size_t>(total_pages));
  int32_t* ctx = at_bytes(meta, p.ctx_off);
  int32_t* toff = at_bytes(meta, p.tbl_off_off);
  int32_t* qs = at_bytes(meta, p.qstart_off);
  int32_t* tl = at_bytes(meta, p.tiles_off);
  int32_t* rs = at_bytes(meta, p.rowseq_off);
  int32_t* tables = at_bytes(meta, p.tables_off);
  int64_t cursor = 0, row = 0;
  for (int32_t b = 0; b < B; ++b) {
    ctx[b] = static_cast<int32_t>(rows[b]->length);
    toff[b] = static_cast<int32_t>(cursor);
    qs[b] = static_cast<int32_t>(row);
    for (int32_t t = 0; t < q_lens[b]; ++t) rs[row + t] = b;
    row += q_lens[b];
    std::copy(rows[b]->table.begin(), rows[b]->table.end(), tables + cursor);
    cursor += static_cast<int64_t>(rows[b]->table.size());
    int32_t* w = at_bytes(meta, p.win_off) + 4 * static_cast<size_t>(b);
    w[0] = rows[b]->windowed() ? rows[b]->sinks : 0;
    w[1] = rows[b]->windowed() ? rows[b]->recent : kNoWindowRecent;
  }
  qs[B] = static_cast<int32_t>(row);
  for (size_t i = 0; i < tiles.size(); ++i) {
    tl[2 * i] = tiles[i].b;
    tl[2 * i + 1] = tiles[i].t0;
  }
  p.meta_bytes = align_up(meta.size() * sizeof(int32_t), kWsAlign);
  p.total_bytes = p.meta_bytes;
  *plan = std::move(p);
  return kOk;
}

}  // namespace pa
