// Host-side planning: validation, tile classification, work list.
//
// The mask is the MAGI-1 block-causal rule (paperlayer summary §2 / Figure 1,
// paper-notes §2 / Figure 1): a query of chunk c in video s attends to the
// keys [kv_offsets[first chunk of s], kv_offsets[c + 1]), i.e. its own chunk
// in full and every earlier chunk of the same video; nothing of other videos
// (paper-notes Figure 15, varlen block-causal). Every query token therefore
// has one contiguous key interval [lo, hi), and a (query tile, key tile) pair
// is "full" when every row's interval covers the key tile, "empty" when no
// row's interval touches it, and "boundary" otherwise. Empty pairs are never
// launched; only boundary pairs pay for the per-element mask.
//
// Work order: the pages' dispatch solver sorts chunks by descending area and
// hands each to the least-loaded bucket (paperlayer §B.1). The same
// longest-first rule orders the workgroups of one GPU, with one bucket per
// XCD: workgroup i runs on XCD i % 8, so items that stream the same KV head
// are placed on the same XCD and share its L2.
//
// The text cross-attention (paperlayer §2.2.2, §2.2.3; paper-notes §3.2.2,
// §3.2.6) is one more rule for the same per-row intervals: the rows of chunk
// c see the text keys [text_begin[c], text_end[c]). A parallel plan holds
// both attentions as two phases of one work list, so the short text items
// are ordered after the long self-attention items and fill the launch's tail.
//
// A KV range R (paperlayer §2.4.4) moves each row's lower bound to chunk
// c - R + 1; a last global block (paper-notes Figure 15(g)) gives its rows
// the whole key stream. Both keep one interval per row.
//
// A training plan adds the backward's lists: dq items as the forward's (never
// split), and dk/dv items per (key block, KV head) over the token tiles that
// see the block. A key is seen by at most two token ranges (its own video's
// later chunks, and a global block's rows; for the text, at most two runs of
// chunks sharing its prompt), so a (token tile, key block) pair is classified
// full, boundary or empty as in the forward. With fewer such items than CUs
// the lists are cut into pieces whose partial sums a merge adds in order.
#include "plan.hpp"

#include "kernels.hpp"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <numeric>

namespace magi {

namespace {

bool supported(int dtype, int d) {
  if (dtype == MAGI_DTYPE_BF16) return d == 64 || d == 128;
  if (dtype == MAGI_DTYPE_FP32) return d == 64 || d == 128;
  return false;
}

}  // namespace

magi_status_t validate_layout(const magi_attn_layout_t* L, std::string& err) {
  if (!L) { err = "layout is NULL"; return MAGI_ERR_INVALID_ARG; }
  if (L->n_chunks < 1) { err = "n_chunks must be >= 1"; return MAGI_ERR_INVALID_ARG; }
  if (L->n_seqs < 1) { err = "n_seqs must be >= 1"; return MAGI_ERR_INVALID_ARG; }
  if (!L->seq_chunks || !L->q_offsets) { err = "seq_chunks and q_offsets must not be NULL"; return MAGI_ERR_INVALID_ARG; }
  const int32_t* kv = L->kv_offsets ? L->kv_offsets : L->q_offsets;
  if (L->seq_chunks[0] != 0 || L->seq_chunks[L->n_seqs] != L->n_chunks) {
    err = "seq_chunks must start at 0 and end at n_chunks"; return MAGI_ERR_INVALID_ARG;
  }
  for (int s = 0; s < L->n_seqs; ++s)
    if (L->seq_chunks[s + 1] <= L->seq_chunks[s]) { err = "seq_chunks must be strictly increasing"; return MAGI_ERR_INVALID_ARG; }
  if (L->q_offsets[0] != 0 || kv[0] != 0) { err = "q_offsets and kv_offsets must start at 0"; return MAGI_ERR_INVALID_ARG; }
  for (int c = 0; c < L->n_chunks; ++c) {
    if (L->q_offsets[c + 1] < L->q_offsets[c]) { err = "q_offsets must be non-decreasing"; return MAGI_ERR_INVALID_ARG; }
    if (kv[c + 1] < kv[c]) { err = "kv_offsets must be non-decreasing"; return MAGI_ERR_INVALID_ARG; }
  }
  if (L->kv_range < 0) { err = "kv_range must be >= 0"; return MAGI_ERR_INVALID_ARG; }
  if (L->last_global != 0 && L->last_global != 1) { err = "last_global must be 0 or 1"; return MAGI_ERR_INVALID_ARG; }
  for (int s = 0; s < L->n_seqs; ++s) {
    for (int c = L->seq_chunks[s]; c < L->seq_chunks[s + 1]; ++c)
      if (L->q_offsets[c + 1] > L->q_offsets[c] &&
          (global_video(L, s) ? kv[L->n_chunks] == 0 : kv[c + 1] <= kv[first_visible_chunk(L, s, c)])) {
        err = "chunk " + std::to_string(c) + " owns queries but sees no key"; return MAGI_ERR_INVALID_ARG;
      }
  }
  if (L->n_q_heads < 1 || L->n_kv_heads < 1 || L->n_q_heads % L->n_kv_heads != 0) {
    err = "n_q_heads must be a positive multiple of n_kv_heads"; return MAGI_ERR_INVALID_ARG;
  }
  if (L->n_q_heads >= 65536) { err = "n_q_heads too large"; return MAGI_ERR_UNSUPPORTED; }
  if (L->dtype != MAGI_DTYPE_BF16 && L->dtype != MAGI_DTYPE_FP32) { err = "unknown dtype"; return MAGI_ERR_INVALID_ARG; }
  if (L->head_dim < 1) { err = "head_dim must be positive"; return MAGI_ERR_INVALID_ARG; }
  if (!supported(L->dtype, L->head_dim)) {
    err = "unsupported head_dim " + std::to_string(L->head_dim) + " (64 or 128)";
    return MAGI_ERR_UNSUPPORTED;
  }
  const int64_t esize = L->dtype == MAGI_DTYPE_BF16 ? 2 : 4;
  // bf16 keys/values are re-laid out in 32-key tiles: count whole tiles
  const int64_t tk_pad = L->dtype == MAGI_DTYPE_BF16 ? (int64_t(kv[L->n_chunks]) + 31) / 32 * 32 : kv[L->n_chunks];
  const int64_t kv_bytes = tk_pad * L->n_kv_heads * L->head_dim * esize;
  const int64_t q_elems = int64_t(L->q_offsets[L->n_chunks]) * L->n_q_heads;
  if (kv_bytes >= (int64_t(1) << 31)) { err = "K/V tensors must be smaller than 2 GiB each"; return MAGI_ERR_UNSUPPORTED; }
  if (q_elems >= (int64_t(1) << 31)) { err = "T_q * n_q_heads must be below 2^31"; return MAGI_ERR_UNSUPPORTED; }
  // token indices plus a tile length stay far from int32 overflow, and the
  // per-row host tables stay below 512 MiB
  if (L->q_offsets[L->n_chunks] >= (int32_t(1) << 26)) { err = "T_q must be below 2^26 tokens"; return MAGI_ERR_UNSUPPORTED; }
  return MAGI_OK;
}

magi_status_t validate_text(const magi_attn_layout_t* L, const magi_attn_text_t* T, int32_t kind,
                            std::string& err) {
  if (!T) { err = "text is NULL"; return MAGI_ERR_INVALID_ARG; }
  if (T->t_text < 0) { err = "t_text must be >= 0"; return MAGI_ERR_INVALID_ARG; }
  if (!T->text_begin || !T->text_end) { err = "text_begin and text_end must not be NULL"; return MAGI_ERR_INVALID_ARG; }
  for (int c = 0; c < L->n_chunks; ++c) {
    const int32_t b = T->text_begin[c], e = T->text_end[c];
    if (b < 0 || e < b || e > T->t_text) {
      err = "chunk " + std::to_string(c) + ": text range must satisfy 0 <= begin <= end <= t_text";
      return MAGI_ERR_INVALID_ARG;
    }
  }
  const int64_t esize = L->dtype == MAGI_DTYPE_BF16 ? 2 : 4;
  const int64_t row_bytes = int64_t(L->n_kv_heads) * L->head_dim * esize;
  auto padded = [&](int64_t t) { return L->dtype == MAGI_DTYPE_BF16 ? (t + 31) / 32 * 32 : t; };
  if (padded(T->t_text) * row_bytes >= (int64_t(1) << 31)) {
    err = "text K/V tensors must be smaller than 2 GiB each"; return MAGI_ERR_UNSUPPORTED;
  }
  if (kind == kPlanParallel) {
    const int32_t* kv = L->kv_offsets ? L->kv_offsets : L->q_offsets;
    if ((padded(kv[L->n_chunks]) + padded(T->t_text)) * row_bytes >= (int64_t(1) << 31)) {
      err = "video and text keys together must be smaller than 2 GiB"; return MAGI_ERR_UNSUPPORTED;
    }
  }
  return MAGI_OK;
}

Tiling choose_tiling(int dtype, int head_dim, int group) {
  (void)head_dim;
  Tiling t{};
  if (dtype == MAGI_DTYPE_BF16) {
    // kBf16RowsPerItem (token, head) rows per workgroup: 8 waves x 48 rows.
    // The largest divisor of the GQA group size that also divides the row
    // count gives the heads per workgroup (all of them when possible), so
    // one K/V tile in LDS serves all of them.
    int hpw = 1;
    for (int h = 1; h <= group; ++h)
      if (group % h == 0 && kBf16RowsPerItem % h == 0) hpw = h;
    t.heads_per_item = hpw;
    t.tile_q = kBf16RowsPerItem / hpw;
    t.tile_kv = 32;
  } else {
    t.heads_per_item = 1;
    t.tile_q = 64;
    t.tile_kv = 32;
  }
  return t;
}

Tiling choose_bwd_tiling(int dtype, int head_dim, int group) {
  Tiling t = choose_tiling(dtype, head_dim, group);
  if (dtype == MAGI_DTYPE_BF16) {
    // kBwdRowsPerItem rows per dq workgroup: 8 waves x 32 rows, each wave's
    // rows one 32-token image of one head, so the item's token tile must be a
    // multiple of 32: heads per item divide both the group and 256 / 32.
    int hpw = 1;
    for (int h = 1; h <= group; ++h)
      if (group % h == 0 && (kBwdRowsPerItem / 32) % h == 0) hpw = h;
    t.heads_per_item = hpw;
    t.tile_q = kBwdRowsPerItem / hpw;
  }
  return t;
}

void key_bounds(const magi_attn_layout_t* L, std::vector<KeyBounds>& keys) {
  // Query chunk c sees key chunk j of its video when j <= c and, with a KV
  // range R, c <= j + R - 1: the queries of chunks [j, last] for the last such
  // chunk, one contiguous token range. A last global block's queries (the
  // stream's last tokens) see every key: a second range for keys of other
  // videos, the only range for its own keys.
  const int32_t* kv = L->kv_offsets ? L->kv_offsets : L->q_offsets;
  const int32_t tq = L->q_offsets[L->n_chunks];
  const int32_t g0 = L->last_global ? L->q_offsets[L->seq_chunks[L->n_seqs - 1]] : tq;
  keys.assign(kv[L->n_chunks], KeyBounds{0, 0, 0, 0});
  for (int s = 0; s < L->n_seqs; ++s)
    for (int j = L->seq_chunks[s]; j < L->seq_chunks[s + 1]; ++j) {
      int last = L->seq_chunks[s + 1] - 1;
      if (L->kv_range > 0 && j + L->kv_range - 1 < last) last = j + L->kv_range - 1;
      KeyBounds b{L->q_offsets[j], L->q_offsets[last + 1], g0, tq};
      if (global_video(L, s)) b = KeyBounds{g0, tq, 0, 0};
      for (int32_t t = kv[j]; t < kv[j + 1]; ++t) keys[t] = b;
    }
}

magi_status_t text_key_bounds(const magi_attn_layout_t* L, const magi_attn_text_t* T, std::vector<KeyBounds>& keys,
                              std::string& err) {
  // Chunks in order: a chunk's rows either extend the key's latest range
  // (they start where it ends) or open its next one.
  keys.assign(T->t_text, KeyBounds{0, 0, 0, 0});
  for (int c = 0; c < L->n_chunks; ++c) {
    const int32_t r0 = L->q_offsets[c], r1 = L->q_offsets[c + 1];
    if (r0 == r1) continue;
    for (int32_t j = T->text_begin[c]; j < T->text_end[c]; ++j) {
      KeyBounds& b = keys[j];
      if (b.glo < b.ghi) {
        if (b.ghi != r0) {
          err = "text token " + std::to_string(j) +
                " is seen by more than two separate runs of chunks (the backward supports two)";
          return MAGI_ERR_UNSUPPORTED;
        }
        b.ghi = r1;
      } else if (b.lo < b.hi) {
        if (b.hi == r0) b.hi = r1;
        else b.glo = r0, b.ghi = r1;
      } else {
        b.lo = r0, b.hi = r1;
      }
    }
  }
  return MAGI_OK;
}

int classify_key_pair(const std::vector<KeyBounds>& iv, int64_t t0, int64_t t1, int64_t tq) {
  if (iv.empty()) return 0;
  bool all = true, any = false;
  for (const KeyBounds& b : iv) {
    const int64_t lo = b.lo, hi = std::min<int64_t>(b.hi, tq), glo = b.glo, ghi = std::min<int64_t>(b.ghi, tq);
    const bool r1 = lo < hi, r2 = glo < ghi;
    auto covers = [&](int64_t a0, int64_t a1) { return a0 <= t0 && t1 <= a1; };
    bool cover = (r1 && covers(lo, hi)) || (r2 && covers(glo, ghi));
    if (!cover && r1 && r2 && std::max(lo, glo) <= std::min(hi, ghi))      // the two ranges touch: one range
      cover = covers(std::min(lo, glo), std::max(hi, ghi));
    if (!cover) all = false;
    if ((r1 && lo < t1 && t0 < hi) || (r2 && glo < t1 && t0 < ghi)) any = true;
  }
  return all ? 2 : (any ? 1 : 0);
}

void row_bounds(const magi_attn_layout_t* L, std::vector<RowBounds>& rows) {
  const int32_t* kv = L->kv_offsets ? L->kv_offsets : L->q_offsets;
  rows.assign(L->q_offsets[L->n_chunks], RowBounds{0, 0});
  for (int s = 0; s < L->n_seqs; ++s)
    for (int c = L->seq_chunks[s]; c < L->seq_chunks[s + 1]; ++c) {
      const RowBounds b = global_video(L, s) ? RowBounds{0, kv[L->n_chunks]}
                                             : RowBounds{kv[first_visible_chunk(L, s, c)], kv[c + 1]};
      for (int32_t t = L->q_offsets[c]; t < L->q_offsets[c + 1]; ++t) rows[t] = b;
    }
}

void text_row_bounds(const magi_attn_layout_t* L, const magi_attn_text_t* T, std::vector<RowBounds>& rows) {
  rows.assign(L->q_offsets[L->n_chunks], RowBounds{0, 0});
  for (int c = 0; c < L->n_chunks; ++c)
    for (int32_t t = L->q_offsets[c]; t < L->q_offsets[c + 1]; ++t)
      rows[t] = RowBounds{T->text_begin[c], T->text_end[c]};
}

void tile_intervals(const std::vector<RowBounds>& rows, int64_t r0, int64_t r1, std::vector<RowBounds>& out) {
  out.clear();
  for (int64_t r = r0; r < r1; ++r) {
    const RowBounds b = rows[r];
    if (out.empty() || out.back().lo != b.lo || out.back().hi != b.hi) out.push_back(b);
  }
}

int classify_pair(const std::vector<RowBounds>& iv, int64_t k0, int64_t k1, int64_t tk) {
  bool all = true, any = false;
  for (const RowBounds& b : iv) {
    const int64_t lo = b.lo, hi = std::min<int64_t>(b.hi, tk);
    if (!(lo <= k0 && k1 <= hi)) all = false;
    if (lo < hi && lo < k1 && k0 < hi) any = true;    // an empty interval touches nothing
  }
  if (iv.empty()) return 0;
  return all ? 2 : (any ? 1 : 0);
}


// Tiles per piece for a phase of n_whole items holding total_cost key tiles.
// Items run one per CU at a time, so cutting every item into p pieces takes
// ceil(n_whole p / kNumCu) rounds of (mean / p + kPieceOverheadTiles) tiles;
// p is the smallest count that minimises that time, up to kMaxPieces and
// with pieces of at least kMinPieceTiles.
int64_t split_piece_tiles(int64_t n_whole, int64_t total_cost) {
  const double mean = double(total_cost) / double(n_whole);
  int best_p = 1;
  double best = 0.0;
  for (int p = 1; p <= kMaxPieces && (p == 1 || mean / p >= kMinPieceTiles); ++p) {
    const double rounds = double((n_whole * p + kNumCu - 1) / kNumCu);
    const double t = rounds * (mean / p + kPieceOverheadTiles);
    if (p == 1 || t < best * (1.0 - 1e-9)) {
      best = t;
      best_p = p;
    }
  }
  return std::max<int64_t>(1, int64_t(std::ceil(mean / best_p)));
}

magi_status_t build_host_plan(int32_t kind, const magi_attn_layout_t* L, const magi_attn_text_t* T,
                              const Tiling& tiling, HostPlan& P, std::string& err, bool allow_split, int split_below) {
  const int32_t* kv = L->kv_offsets ? L->kv_offsets : L->q_offsets;
  P.kind = kind;
  P.n_phases = kind == kPlanParallel ? 2 : 1;
  P.n_chunks = L->n_chunks;
  P.n_seqs = L->n_seqs;
  P.hq = L->n_q_heads;
  P.hk = L->n_kv_heads;
  P.d = L->head_dim;
  P.dtype = L->dtype;
  P.tq = L->q_offsets[L->n_chunks];
  P.tk = kind == kPlanCross ? T->t_text : kv[L->n_chunks];
  P.tk_x = kind == kPlanParallel ? T->t_text : 0;
  P.tiling = tiling;

  // Per-phase key bounds of every query token, phase p at p * tq.
  std::vector<RowBounds> tmp;
  if (kind == kPlanCross) text_row_bounds(L, T, P.rows);
  else row_bounds(L, P.rows);
  if (kind == kPlanParallel) {
    text_row_bounds(L, T, tmp);
    P.rows.insert(P.rows.end(), tmp.begin(), tmp.end());
  }

  const int bm = tiling.tile_q, bn = tiling.tile_kv;
  const int64_t n_qt = (P.tq + bm - 1) / bm;
  const int group = P.hq / P.hk;
  const int hpw = tiling.heads_per_item;
  const int groups_per_kvh = group / hpw;
  const int64_t phase_tk[2] = {P.tk, P.tk_x};
  const int64_t phase_nkt[2] = {(P.tk + bn - 1) / bn, (P.tk_x + bn - 1) / bn};
  const int64_t phase_img0[2] = {0, phase_nkt[0]};         // first image tile of each phase's keys
  P.n_kt_img = phase_nkt[0] + (P.n_phases == 2 ? phase_nkt[1] : 0);

  magi_attn_stats_t& S = P.stats;
  std::memset(&S, 0, sizeof(S));
  for (const RowBounds& b : P.rows) S.unmasked_pairs += int64_t(b.hi - b.lo);

  const int64_t n_lists = P.n_phases * n_qt;
  // The kernels index the tile lists with int32: bound every list by the key
  // tiles its rows' [lo, hi) span (plus the padding), in int64, and refuse the
  // layout before building anything that could pass INT32_MAX entries.
  {
    int64_t bound = 0;
    for (int ph = 0; ph < P.n_phases; ++ph)
      for (int64_t qt = 0; qt < n_qt; ++qt) {
        const int64_t r0 = qt * bm, r1 = std::min<int64_t>(P.tq, r0 + bm);
        int64_t lo = INT64_MAX, hi = 0;
        for (int64_t r = r0; r < r1; ++r) {
          const RowBounds& b = P.rows[size_t(ph * P.tq + r)];
          if (b.hi > b.lo) { lo = std::min<int64_t>(lo, b.lo); hi = std::max<int64_t>(hi, b.hi); }
        }
        bound += kTilePad + (hi > lo ? (hi + bn - 1) / bn - lo / bn : 0);
      }
    if (bound > INT32_MAX) {
      err = "the layout's tile lists would pass 2^31 entries (" + std::to_string(bound) + ")";
      return MAGI_ERR_UNSUPPORTED;
    }
  }
  P.tile_codes.clear();
  P.qt_tiles.assign(n_lists + 1, 0);
  P.qt_ntiles.assign(n_lists, 0);
  P.qt_full.assign(n_lists, 0);
  std::vector<int32_t> masked_codes;
  std::vector<RowBounds> iv;
  for (int ph = 0; ph < P.n_phases; ++ph) {
    const std::vector<RowBounds> rows_ph(P.rows.begin() + ph * P.tq, P.rows.begin() + (ph + 1) * P.tq);
    const int64_t tk = phase_tk[ph];
    for (int64_t qt = 0; qt < n_qt; ++qt) {
      const int64_t li = ph * n_qt + qt;
      const int64_t r0 = qt * bm, r1 = std::min<int64_t>(P.tq, r0 + bm);
      tile_intervals(rows_ph, r0, r1, iv);
      int64_t lo = INT64_MAX, hi = 0;
      for (const RowBounds& b : iv)
        if (b.hi > b.lo) { lo = std::min<int64_t>(lo, b.lo); hi = std::max<int64_t>(hi, b.hi); }
      P.qt_tiles[li] = int32_t(P.tile_codes.size());
      masked_codes.clear();
      if (hi > lo) {
        for (int64_t kt = lo / bn; kt < (hi + bn - 1) / bn; ++kt) {
          const int cls = classify_pair(iv, kt * bn, kt * bn + bn, tk);
          if (cls == 2) ++S.full_pairs;
          if (cls == 1) ++S.boundary_pairs;
          if (cls == 0) continue;
          if (cls == 1) masked_codes.push_back(tile_code(kt, 1));
          else P.tile_codes.push_back(tile_code(kt, 0));
          S.executed_pairs += (r1 - r0) * int64_t(bn);
        }
      }
      P.qt_full[li] = int32_t(P.tile_codes.size()) - P.qt_tiles[li];
      P.tile_codes.insert(P.tile_codes.end(), masked_codes.begin(), masked_codes.end());
      P.qt_ntiles[li] = int32_t(P.tile_codes.size()) - P.qt_tiles[li];
      P.tile_codes.insert(P.tile_codes.end(), kTilePad, -1);
    }
    S.empty_pairs += n_qt * phase_nkt[ph];
  }
  P.qt_tiles[n_lists] = int32_t(P.tile_codes.size());
  S.empty_pairs -= S.full_pairs + S.boundary_pairs;
  // Copy offsets of the bf16 path's per-tile image blocks ([tile][KV head];
  // phase 1's tiles follow phase 0's).
  const int64_t image_bytes = int64_t(bn) * P.d * 2;
  P.tile_soff.resize(P.tile_codes.size());
  for (int ph = 0; ph < P.n_phases; ++ph)
    for (int32_t t = P.qt_tiles[ph * n_qt]; t < P.qt_tiles[(ph + 1) * n_qt]; ++t)
      P.tile_soff[t] = P.tile_codes[t] < 0
                           ? kNoTileOffset
                           : uint32_t((phase_img0[ph] + (P.tile_codes[t] >> 1)) * P.hk * image_bytes);

  // Work items: (phase, query tile, KV head, group of hpw query heads), cut
  // into pieces of their tile list when the phase has too few of them (the
  // decision is per phase: a parallel plan's many short text items do not
  // fill the GPU for the long self-attention items). Query tiles without any
  // key in a phase become merge entries without pieces (their rows get
  // out = 0, lse = -inf).
  struct Cand { int64_t cost; int32_t ph, qt, kvh, hg, begin, end, slot; };
  std::vector<Cand> cands;
  P.merges.clear();
  P.n_slots = 0;
  for (int ph = 0; ph < P.n_phases; ++ph) {
    int64_t n_whole = 0, total_cost = 0;
    for (int64_t qt = 0; qt < n_qt; ++qt)
      if (P.qt_ntiles[ph * n_qt + qt] > 0) {
        n_whole += int64_t(P.hk) * groups_per_kvh;
        total_cost += int64_t(P.qt_ntiles[ph * n_qt + qt]) * P.hk * groups_per_kvh;
      }
    const bool split = allow_split && P.dtype == MAGI_DTYPE_BF16 && n_whole > 0 && n_whole < split_below;
    const int64_t piece = split ? split_piece_tiles(n_whole, total_cost) : int64_t(1) << 40;
    for (int kvh = 0; kvh < P.hk; ++kvh)
      for (int64_t qt = 0; qt < n_qt; ++qt) {
        const int64_t li = ph * n_qt + qt;
        const int32_t nt = P.qt_ntiles[li];
        const int32_t b0 = P.qt_tiles[li];
        const int64_t want = (nt + piece / 2) / piece;                      // pieces of about `piece` tiles
        const int n_pieces =
            nt == 0 ? 0
            : split ? int(std::max<int64_t>(1, std::min<int64_t>({want, int64_t(kMaxPieces), nt / kMinPieceTiles})))
                    : 1;
        for (int hg = 0; hg < groups_per_kvh; ++hg) {
          if (n_pieces == 1) {
            cands.push_back(Cand{nt, ph, int32_t(qt), kvh, hg, b0, b0 + nt, -1});
            continue;
          }
          const int h0 = kvh * group + hg * hpw;
          P.merges.push_back(MergeItem{int32_t(qt * bm), (kvh << 16) | h0, P.n_slots, n_pieces, ph, {0, 0, 0}});
          for (int k = 0; k < n_pieces; ++k) {
            const int32_t pb = b0 + int32_t(int64_t(nt) * k / n_pieces);
            const int32_t pe = b0 + int32_t(int64_t(nt) * (k + 1) / n_pieces);
            cands.push_back(Cand{pe - pb, ph, int32_t(qt), kvh, hg, pb, pe, P.n_slots + k});
          }
          P.n_slots += n_pieces;
        }
      }
  }
  // Longest first; among equals, consecutive query tiles and head groups of
  // one KV head stay adjacent so concurrently running workgroups read the
  // same key tiles.
  std::stable_sort(cands.begin(), cands.end(), [](const Cand& a, const Cand& b) {
    if (a.cost != b.cost) return a.cost > b.cost;
    if (a.ph != b.ph) return a.ph < b.ph;
    if (a.kvh != b.kvh) return a.kvh < b.kvh;
    if (a.qt != b.qt) return a.qt < b.qt;
    return a.hg < b.hg;
  });
  std::vector<std::vector<WorkItem>> queues(kNumXcd);
  std::vector<int64_t> load(kNumXcd, 0);
  auto make_item = [&](const Cand& c) {
    const int h0 = c.kvh * group + c.hg * hpw;
    // full tiles come first in the list: the piece's share of them
    const int64_t li = c.ph * n_qt + c.qt;
    const int32_t full_end = P.qt_tiles[li] + P.qt_full[li];
    const int32_t n_full = std::max<int32_t>(0, std::min<int32_t>(c.end, full_end) - c.begin);
    return WorkItem{int32_t(c.qt * bm), (c.kvh << 16) | h0, c.begin, c.end, n_full, c.slot, c.ph, 0};
  };
  if (P.hk % kNumXcd == 0 || kNumXcd % P.hk == 0) {
    // Each KV head owns a fixed set of XCDs (or each XCD owns a fixed set of
    // KV heads); longest-first to the least-loaded XCD of that set.
    const int per_head = P.hk >= kNumXcd ? 1 : kNumXcd / P.hk;
    for (const Cand& c : cands) {
      int best = -1;
      for (int j = 0; j < per_head; ++j) {
        const int x = (P.hk >= kNumXcd) ? (c.kvh % kNumXcd) : (c.kvh * per_head + j);
        if (best < 0 || load[x] < load[best]) best = x;
      }
      queues[best].push_back(make_item(c));
      load[best] += c.cost;
    }
  } else {
    for (const Cand& c : cands) {
      const int best = int(std::min_element(load.begin(), load.end()) - load.begin());
      queues[best].push_back(make_item(c));
      load[best] += c.cost;
    }
  }
  size_t maxlen = 0;
  for (auto& q : queues) maxlen = std::max(maxlen, q.size());
  P.items.clear();
  P.items.reserve(maxlen * kNumXcd);
  for (size_t j = 0; j < maxlen; ++j)
    for (int x = 0; x < kNumXcd; ++x)
      P.items.push_back(j < queues[x].size() ? queues[x][j] : WorkItem{0, 0, 0, 0, 0, -1, 0, 0});
  // Drop trailing padding.
  while (!P.items.empty() && P.items.back().tile_begin == P.items.back().tile_end) P.items.pop_back();

  S.tile_q = bm;
  S.tile_kv = bn;
  S.heads_per_item = hpw;
  S.n_items = int32_t(P.items.size());
  return MAGI_OK;
}

magi_status_t build_bwd_plan(const magi_attn_layout_t* L, const magi_attn_text_t* T, BwdHostPlan& B,
                             std::string& err) {
  const int group = L->n_q_heads / L->n_kv_heads;
  const Tiling tiling = choose_bwd_tiling(L->dtype, L->head_dim, group);
  if (L->dtype == MAGI_DTYPE_BF16 && tiling.tile_q % 32 != 0) {
    err = "internal: backward query tile not a multiple of 32 tokens";
    return MAGI_ERR_UNSUPPORTED;
  }
  magi_status_t s = build_host_plan(T ? kPlanCross : kPlanSelf, L, T, tiling, B.dq, err, /*allow_split=*/true,
                                    kBwdDqSplitBelowItems);
  if (s != MAGI_OK) return s;
  // Query blocks without any key have no dq item (their merge entries hold no
  // pieces): their dq is zero. Entries with pieces are split dq items.
  B.dq_zero.clear();
  B.dq_merges.clear();
  for (const MergeItem& m : B.dq.merges)
    if (m.n_pieces == 0) {
      B.dq_zero.push_back(m.t0);
      B.dq_zero.push_back(m.heads & 0xffff);
    } else {
      B.dq_merges.push_back(m);
    }
  const int32_t* kv = L->kv_offsets ? L->kv_offsets : L->q_offsets;
  const int64_t tq = L->q_offsets[L->n_chunks], tk = T ? T->t_text : kv[L->n_chunks];
  const int kb_size = L->dtype == MAGI_DTYPE_BF16 ? kBwdKeysPerItem : 64;
  const int tt_size = B.token_tile;
  B.key_block = kb_size;
  if (T) {
    s = text_key_bounds(L, T, B.key_rows, err);
    if (s != MAGI_OK) return s;
  } else {
    key_bounds(L, B.key_rows);
  }

  // Per key block: the token tiles that see any of its keys, full first.
  const int64_t n_kb = (tk + kb_size - 1) / kb_size;
  const int64_t n_tt_all = (tq + tt_size - 1) / tt_size;
  {
    // int32 list indices on the device: bound the lists as the forward's are
    int64_t bound = 0;
    for (int64_t kb = 0; kb < n_kb; ++kb) {
      int64_t lo = INT64_MAX, hi = 0, glo = INT64_MAX, ghi = 0;
      for (int64_t j = kb * kb_size; j < std::min<int64_t>(tk, (kb + 1) * kb_size); ++j) {
        const KeyBounds& b = B.key_rows[size_t(j)];
        if (b.hi > b.lo) { lo = std::min<int64_t>(lo, b.lo); hi = std::max<int64_t>(hi, b.hi); }
        if (b.ghi > b.glo) { glo = std::min<int64_t>(glo, b.glo); ghi = std::max<int64_t>(ghi, b.ghi); }
      }
      const int64_t a = hi > lo ? (hi + tt_size - 1) / tt_size - lo / tt_size : 0;
      const int64_t c = ghi > glo ? (ghi + tt_size - 1) / tt_size - glo / tt_size : 0;
      bound += kTilePad + std::min<int64_t>(n_tt_all, a + c);
    }
    if (bound > INT32_MAX) {
      err = "the layout's backward tile lists would pass 2^31 entries (" + std::to_string(bound) + ")";
      return MAGI_ERR_UNSUPPORTED;
    }
  }
  std::vector<int32_t> kb_begin(n_kb), kb_n(n_kb), kb_full(n_kb);
  std::vector<int32_t> masked_codes;
  std::vector<KeyBounds> iv;
  std::vector<char> cand;
  B.kv_tiles.clear();
  const int64_t n_tt = (tq + tt_size - 1) / tt_size;
  for (int64_t kb = 0; kb < n_kb; ++kb) {
    const int64_t k0 = kb * kb_size, k1 = std::min<int64_t>(tk, k0 + kb_size);
    iv.clear();
    for (int64_t j = k0; j < k1; ++j) {
      const KeyBounds& b = B.key_rows[j];
      if (iv.empty() || iv.back().lo != b.lo || iv.back().hi != b.hi || iv.back().glo != b.glo || iv.back().ghi != b.ghi)
        iv.push_back(b);
    }
    // candidate token tiles: those touching any key's ranges
    cand.assign(n_tt, 0);
    for (const KeyBounds& b : iv) {
      if (b.hi > b.lo)
        for (int64_t tt = b.lo / tt_size; tt < (int64_t(b.hi) + tt_size - 1) / tt_size; ++tt) cand[tt] = 1;
      if (b.ghi > b.glo)
        for (int64_t tt = b.glo / tt_size; tt < (int64_t(b.ghi) + tt_size - 1) / tt_size; ++tt) cand[tt] = 1;
    }
    kb_begin[kb] = int32_t(B.kv_tiles.size());
    masked_codes.clear();
    for (int64_t tt = 0; tt < n_tt; ++tt) {
      if (!cand[tt]) continue;
      const int cls = classify_key_pair(iv, tt * tt_size, tt * tt_size + tt_size, tq);
      if (cls == 2) B.kv_tiles.push_back(tile_code(tt, 0));
      else if (cls == 1) masked_codes.push_back(tile_code(tt, 1));
    }
    kb_full[kb] = int32_t(B.kv_tiles.size()) - kb_begin[kb];
    B.kv_tiles.insert(B.kv_tiles.end(), masked_codes.begin(), masked_codes.end());
    kb_n[kb] = int32_t(B.kv_tiles.size()) - kb_begin[kb];
    B.kv_tiles.insert(B.kv_tiles.end(), kTilePad, -1);
  }
  // Key blocks that no query sees get no item: their dk and dv are zero.
  B.kv_zero.clear();
  for (int64_t kb = 0; kb < n_kb; ++kb)
    if (kb_n[kb] == 0) {
      B.kv_zero.push_back(int32_t(kb * kb_size));
      B.kv_zero.push_back(0);
    }

  // Items (key block, KV head), longest first, KV head -> XCD as for the
  // forward's items. With too few of them to fill the GPU (bf16: a short
  // text stream, a small video), each list is cut into pieces that write
  // fp32 partial sums to slots, summed in piece order afterwards.
  const int hk = L->n_kv_heads;
  struct Cand { int64_t cost; int32_t kb, kvh, begin, end, full, slot; };
  std::vector<Cand> cands;
  int64_t n_whole = 0, total = 0;
  for (int64_t kb = 0; kb < n_kb; ++kb)
    if (kb_n[kb] > 0) n_whole += hk, total += int64_t(kb_n[kb]) * hk;
  const bool split = L->dtype == MAGI_DTYPE_BF16 && n_whole > 0 && n_whole < kBwdSplitBelowItems;
  const int64_t piece =
      std::max<int64_t>(kBwdMinPieceEntries, (total + kBwdSplitTargetItems - 1) / kBwdSplitTargetItems);
  B.kv_merges.clear();
  B.n_kv_slots = 0;
  for (int kvh = 0; kvh < hk; ++kvh)
    for (int64_t kb = 0; kb < n_kb; ++kb) {
      const int32_t n = kb_n[kb], b0 = kb_begin[kb];
      if (n == 0) continue;
      const int n_pieces =
          split ? int(std::max<int64_t>(1, std::min<int64_t>(kBwdMaxPieces, (n + piece - 1) / piece))) : 1;
      if (n_pieces == 1) {
        cands.push_back(Cand{int64_t(n) * group, int32_t(kb), kvh, b0, b0 + n, kb_full[kb], -1});
        continue;
      }
      B.kv_merges.push_back(KeyMerge{int32_t(kb), kvh, B.n_kv_slots, n_pieces});
      for (int k = 0; k < n_pieces; ++k) {
        const int32_t pb = b0 + int32_t(int64_t(n) * k / n_pieces), pe = b0 + int32_t(int64_t(n) * (k + 1) / n_pieces);
        const int32_t full = std::max(0, std::min(pe - pb, kb_full[kb] - (pb - b0)));
        cands.push_back(Cand{int64_t(pe - pb) * group, int32_t(kb), kvh, pb, pe, full, B.n_kv_slots + k});
      }
      B.n_kv_slots += n_pieces;
    }
  std::stable_sort(cands.begin(), cands.end(), [](const Cand& a, const Cand& b) {
    if (a.cost != b.cost) return a.cost > b.cost;
    if (a.kvh != b.kvh) return a.kvh < b.kvh;
    if (a.kb != b.kb) return a.kb < b.kb;
    return a.begin < b.begin;
  });
  std::vector<std::vector<KeyItem>> queues(kNumXcd);
  std::vector<int64_t> load(kNumXcd, 0);
  const bool by_head = hk % kNumXcd == 0 || kNumXcd % hk == 0;
  const int per_head = hk >= kNumXcd ? 1 : kNumXcd / hk;
  for (const Cand& c : cands) {
    int best = -1;
    if (by_head) {
      for (int j = 0; j < per_head; ++j) {
        const int x = hk >= kNumXcd ? c.kvh % kNumXcd : c.kvh * per_head + j;
        if (best < 0 || load[x] < load[best]) best = x;
      }
    } else {
      best = int(std::min_element(load.begin(), load.end()) - load.begin());
    }
    queues[best].push_back(KeyItem{c.kb, c.kvh, c.begin, c.end, c.full, c.slot, {0, 0}});
    load[best] += c.cost;
  }
  size_t maxlen = 0;
  for (auto& q : queues) maxlen = std::max(maxlen, q.size());
  B.items.clear();
  for (size_t j = 0; j < maxlen; ++j)
    for (int x = 0; x < kNumXcd; ++x)
      B.items.push_back(j < queues[x].size() ? queues[x][j] : KeyItem{0, 0, 0, 0, 0, -1, {0, 0}});
  while (!B.items.empty() && B.items.back().tile_begin == B.items.back().tile_end) B.items.pop_back();
  return MAGI_OK;
}

}  // namespace magi
