// Seeded fuzz of the host planner (plan.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizer.py.
//
// Layouts follow the block-causal problem of the MAGI-1 pages (paperlayer §2
// and Figure 1; paper-notes §2 and Figure 15): packed videos of chunks,
// chunks without queries (a KV cache, paperlayer §2.4.4), a KV-range window,
// a last global block, and chunk-wise text prompts with clean chunks for the
// cross-attention (paperlayer §2.2.3; paper-notes §3.2.6). Every array is
// allocated at exactly the length the layout declares, so that a read past
// it is caught. Valid layouts are planned as the C ABI plans them (self,
// cross and parallel forward plans; training plans) and the plans' lists are
// checked for internal consistency; invalid layouts must be refused. Limit
// cases put offsets at the 2 GiB tensor limits, next to INT32_MAX, and build
// a layout whose tile lists would pass 2^31 entries.
//
// usage: plan_fuzz N_SEEDS [FIRST_SEED]   exit status 0 when every check holds
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <random>
#include <string>
#include <vector>

#include "plan.hpp"

using namespace magi;

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                          \
  do {                                                            \
    if (!(cond)) {                                                \
      std::fprintf(stderr, "check failed: %s: ", #cond);          \
      std::fprintf(stderr, __VA_ARGS__);                          \
      std::fprintf(stderr, "\n");                                 \
      ++g_failures;                                               \
    }                                                             \
  } while (0)

// Heap copies of exactly n elements (ASan sees any read past them).
std::unique_ptr<int32_t[]> exact(const std::vector<int32_t>& v) {
  std::unique_ptr<int32_t[]> p(new int32_t[v.size() ? v.size() : 1]);
  for (size_t i = 0; i < v.size(); ++i) p[i] = v[i];
  return p;
}

struct Case {
  std::vector<int32_t> q, kv, seq, tb, te;
  int32_t hq = 1, hk = 1, d = 128, dtype = MAGI_DTYPE_BF16, kv_range = 0, last_global = 0, t_text = 0;
  bool has_kv = true;
};

struct Owned {
  std::unique_ptr<int32_t[]> q, kv, seq, tb, te;
  magi_attn_layout_t L{};
  magi_attn_text_t T{};
};

Owned own(const Case& c) {
  Owned o;
  o.q = exact(c.q);
  o.kv = exact(c.kv);
  o.seq = exact(c.seq);
  o.tb = exact(c.tb);
  o.te = exact(c.te);
  o.L.n_seqs = int32_t(c.seq.size()) - 1;
  o.L.seq_chunks = o.seq.get();
  o.L.n_chunks = int32_t(c.q.size()) - 1;
  o.L.q_offsets = o.q.get();
  o.L.kv_offsets = c.has_kv ? o.kv.get() : nullptr;
  o.L.n_q_heads = c.hq;
  o.L.n_kv_heads = c.hk;
  o.L.head_dim = c.d;
  o.L.dtype = c.dtype;
  o.L.kv_range = c.kv_range;
  o.L.last_global = c.last_global;
  o.T.t_text = c.t_text;
  o.T.text_begin = o.tb.get();
  o.T.text_end = o.te.get();
  return o;
}

// Consistency of a forward plan's lists.
void check_plan(const HostPlan& P, const char* what) {
  const int bm = P.tiling.tile_q, bn = P.tiling.tile_kv;
  const int64_t n_qt = (P.tq + bm - 1) / bm;
  const int64_t nkt[2] = {(P.tk + bn - 1) / bn, (P.tk_x + bn - 1) / bn};
  CHECK(int64_t(P.qt_tiles.size()) == P.n_phases * n_qt + 1, "%s: qt_tiles size", what);
  CHECK(P.tile_soff.size() == P.tile_codes.size(), "%s: soff size", what);
  int64_t pairs = 0;
  for (int ph = 0; ph < P.n_phases; ++ph) pairs += n_qt * nkt[ph];
  CHECK(P.stats.full_pairs + P.stats.boundary_pairs + P.stats.empty_pairs == pairs,
        "%s: %" PRId64 " + %" PRId64 " + %" PRId64 " != %" PRId64, what, P.stats.full_pairs, P.stats.boundary_pairs,
        P.stats.empty_pairs, pairs);
  for (int ph = 0; ph < P.n_phases; ++ph)
    for (int64_t qt = 0; qt < n_qt; ++qt) {
      const int64_t li = ph * n_qt + qt;
      const int32_t b = P.qt_tiles[li], n = P.qt_ntiles[li], f = P.qt_full[li];
      CHECK(0 <= f && f <= n && b + n + kTilePad == P.qt_tiles[li + 1], "%s: list %" PRId64, what, li);
      for (int32_t t = b; t < b + n; ++t) {
        const int32_t code = P.tile_codes[t];
        CHECK(code >= 0 && (code >> 1) < nkt[ph] && ((code & 1) == (t >= b + f ? 1 : 0)), "%s: code %d", what, code);
      }
      for (int32_t t = b + n; t < b + n + kTilePad; ++t)
        CHECK(P.tile_codes[t] == -1 && P.tile_soff[t] == kNoTileOffset, "%s: padding", what);
    }
  for (const WorkItem& w : P.items) {
    if (w.tile_begin == w.tile_end) continue;
    CHECK(w.phase >= 0 && w.phase < P.n_phases && w.t0 >= 0 && w.t0 < P.tq && w.t0 % bm == 0, "%s: item", what);
    const int64_t li = w.phase * n_qt + w.t0 / bm;
    CHECK(w.tile_begin >= P.qt_tiles[li] && w.tile_end <= P.qt_tiles[li] + P.qt_ntiles[li] && w.n_full >= 0 &&
              w.n_full <= w.tile_end - w.tile_begin && w.slot < P.n_slots,
          "%s: item range", what);
  }
  for (const MergeItem& m : P.merges)
    CHECK(m.n_pieces >= 0 && m.slot0 >= 0 && m.slot0 + m.n_pieces <= P.n_slots, "%s: merge", what);
  // every allowed (row, key) pair lies in a listed tile of its list (small plans)
  if (P.tq * (P.tk + P.tk_x) <= (int64_t(1) << 22)) {
    for (int ph = 0; ph < P.n_phases; ++ph)
      for (int64_t r = 0; r < P.tq; ++r) {
        const RowBounds& rb = P.rows[size_t(ph * P.tq + r)];
        if (rb.hi <= rb.lo) continue;
        const int64_t li = ph * n_qt + r / bm;
        std::vector<char> listed(size_t(nkt[ph]), 0);
        for (int32_t t = P.qt_tiles[li]; t < P.qt_tiles[li] + P.qt_ntiles[li]; ++t) listed[P.tile_codes[t] >> 1] = 1;
        for (int64_t kt = rb.lo / bn; kt <= (rb.hi - 1) / bn; ++kt)
          CHECK(listed[size_t(kt)], "%s: row %" PRId64 " key tile %" PRId64 " not listed", what, r, kt);
      }
  }
}

void check_bwd(const BwdHostPlan& B, int64_t tq, int64_t tk, const char* what) {
  const int64_t n_tt = (tq + B.token_tile - 1) / B.token_tile;
  const int64_t n_kb = (tk + B.key_block - 1) / B.key_block;
  CHECK(int64_t(B.key_rows.size()) == tk, "%s: key_rows", what);
  for (size_t t = 0; t < B.kv_tiles.size(); ++t)
    CHECK(B.kv_tiles[t] == -1 || (B.kv_tiles[t] >= 0 && (B.kv_tiles[t] >> 1) < n_tt), "%s: kv tile code", what);
  for (const KeyItem& k : B.items) {
    if (k.tile_begin == k.tile_end) continue;
    CHECK(k.kb >= 0 && k.kb < n_kb && k.tile_begin >= 0 && k.tile_end <= int32_t(B.kv_tiles.size()) &&
              k.n_full >= 0 && k.n_full <= k.tile_end - k.tile_begin && k.slot < B.n_kv_slots,
          "%s: key item", what);
  }
  for (const KeyMerge& m : B.kv_merges) CHECK(m.slot0 + m.n_pieces <= B.n_kv_slots, "%s: key merge", what);
  check_plan(B.dq, what);
  // Split dq items: every merge entry is either a query block without keys
  // (dq_zero) or a split item (dq_merges, at least 2 pieces); its pieces are
  // the items whose slots are slot0 .. slot0 + n - 1, of the same rows and
  // heads, cutting the block's list into consecutive non-empty ranges in slot
  // order; no other item has a slot.
  const HostPlan& P = B.dq;
  CHECK(B.dq_zero.size() % 2 == 0 && B.dq_zero.size() / 2 + B.dq_merges.size() == P.merges.size(),
        "%s: dq merges %zu + zero blocks %zu != %zu", what, B.dq_merges.size(), B.dq_zero.size() / 2,
        P.merges.size());
  std::vector<const WorkItem*> by_slot(size_t(P.n_slots), nullptr);
  for (const WorkItem& w : P.items) {
    if (w.slot < 0) continue;
    CHECK(w.slot < P.n_slots && !by_slot[size_t(w.slot)], "%s: dq slot %d", what, w.slot);
    if (w.slot < P.n_slots) by_slot[size_t(w.slot)] = &w;
  }
  int32_t slots_seen = 0;
  const int bm = P.tiling.tile_q;
  for (const MergeItem& m : B.dq_merges) {
    CHECK(m.n_pieces >= 2 && m.slot0 == slots_seen, "%s: dq merge pieces %d slot0 %d", what, m.n_pieces, m.slot0);
    slots_seen = m.slot0 + m.n_pieces;
    if (m.n_pieces < 2 || m.slot0 + m.n_pieces > P.n_slots) continue;
    const int64_t li = m.phase * ((P.tq + bm - 1) / bm) + m.t0 / bm;
    int32_t next = P.qt_tiles[li];
    for (int k = 0; k < m.n_pieces; ++k) {
      const WorkItem* w = by_slot[size_t(m.slot0 + k)];
      CHECK(w != nullptr, "%s: dq slot %d has no piece", what, m.slot0 + k);
      if (!w) break;
      CHECK(w->t0 == m.t0 && w->heads == m.heads && w->phase == m.phase && w->tile_begin == next &&
                w->tile_end > w->tile_begin,
            "%s: dq piece %d of block %d", what, k, m.t0);
      next = w->tile_end;
    }
    CHECK(next == P.qt_tiles[li] + P.qt_ntiles[li], "%s: dq pieces of block %d end at %d", what, m.t0, next);
  }
  CHECK(slots_seen == P.n_slots, "%s: dq slots %d of %d in merges", what, slots_seen, P.n_slots);
}

// Plans a case the way the C ABI does; returns the validation status.
magi_status_t run_case(const Case& c, bool expect_valid, const char* tag) {
  Owned o = own(c);
  std::string err;
  magi_status_t s = validate_layout(&o.L, err);
  if (s != MAGI_OK) {
    CHECK(!expect_valid, "%s: valid layout refused: %s", tag, err.c_str());
    return s;
  }
  const Tiling tl = choose_tiling(c.dtype, c.d, c.hq / c.hk);
  HostPlan P;
  s = build_host_plan(kPlanSelf, &o.L, nullptr, tl, P, err);
  if (s == MAGI_OK) {
    check_plan(P, tag);
    BwdHostPlan B;
    const int64_t tq = c.q.back(), tk = c.has_kv ? c.kv.back() : c.q.back();
    if (build_bwd_plan(&o.L, nullptr, B, err) == MAGI_OK) check_bwd(B, tq, tk, tag);
  }
  if (!c.tb.empty()) {
    for (int32_t kind : {int32_t(kPlanCross), int32_t(kPlanParallel)}) {
      std::string e2;
      if (validate_text(&o.L, &o.T, kind, e2) != MAGI_OK) continue;
      HostPlan X;
      if (build_host_plan(kind, &o.L, &o.T, tl, X, e2) == MAGI_OK) check_plan(X, tag);
      if (kind == kPlanCross) {
        BwdHostPlan XB;
        if (build_bwd_plan(&o.L, &o.T, XB, e2) == MAGI_OK) check_bwd(XB, c.q.back(), c.t_text, tag);
      }
    }
  }
  return s;
}

Case random_case(std::mt19937_64& rng) {
  auto U = [&](int a, int b) { return int(std::uniform_int_distribution<int>(a, b)(rng)); };
  Case c;
  const int n_vid = U(1, 4);
  c.q = {0};
  c.kv = {0};
  c.seq = {0};
  for (int v = 0; v < n_vid; ++v) {
    const int n_ch = U(1, 5);
    const int cached = U(0, 2) == 0 ? U(0, n_ch - 1) : 0;   // leading chunks without queries
    for (int k = 0; k < n_ch; ++k) {
      const int len = U(0, 3) == 0 ? U(1, 8) : U(1, 400);
      c.kv.push_back(c.kv.back() + len);
      c.q.push_back(c.q.back() + (k < cached ? 0 : U(0, 4) == 0 ? U(1, len) : len));
    }
    c.seq.push_back(int32_t(c.q.size()) - 1);
  }
  static const int heads[][2] = {{1, 1}, {2, 1}, {6, 2}, {8, 1}, {3, 3}, {24, 8}, {16, 2}, {48, 8}, {12, 4}};
  const auto& h = heads[U(0, 8)];
  c.hq = h[0];
  c.hk = h[1];
  c.dtype = U(0, 3) == 0 ? MAGI_DTYPE_FP32 : MAGI_DTYPE_BF16;
  c.d = c.dtype == MAGI_DTYPE_FP32 && U(0, 1) ? 64 : 128;
  c.kv_range = U(0, 2) == 0 ? U(1, 4) : 0;
  c.last_global = U(0, 3) == 0 ? 1 : 0;
  c.has_kv = !(c.q == c.kv) || U(0, 1);
  if (!c.has_kv) c.kv = c.q;
  // chunk-wise prompts: clean chunks, shared prompts, ragged lengths
  const int n = int(c.q.size()) - 1;
  int t = 0;
  for (int k = 0; k < n; ++k) {
    if (U(0, 3) == 0) { c.tb.push_back(t); c.te.push_back(t); continue; }
    if (k > 0 && U(0, 2) == 0 && c.te.back() > c.tb.back()) { c.tb.push_back(c.tb.back()); c.te.push_back(c.te.back()); continue; }
    const int len = U(1, 300);
    c.tb.push_back(t);
    c.te.push_back(t + len);
    t += len;
  }
  c.t_text = t;
  return c;
}

// A copy of a valid case with one field broken (the planner must refuse it).
Case broken(Case c, int how, std::mt19937_64& rng) {
  const int n = int(c.q.size()) - 1;
  const int k = int(rng() % uint64_t(n)) + 1;
  switch (how % 8) {
    case 0: c.q[k] = c.q[k - 1] - 1; break;                               // decreasing query offsets
    case 1: c.kv[0] = 1; c.has_kv = true; break;                          // not starting at 0
    case 2: c.seq.back() = n - 1 > 0 ? n - 1 : n + 1; break;              // videos do not cover the chunks
    case 3: c.hq = c.hk * 2 + 1; c.hk = 2; break;                         // heads not a multiple
    case 4: c.kv_range = -1; break;
    case 5: c.last_global = 2; break;
    case 6: c.d = 96; break;                                              // unsupported head_dim
    default: c.dtype = 7; break;                                          // unknown dtype
  }
  return c;
}

void limit_cases() {
  // K at the 2 GiB limit: 2^23 - 32 keys of one KV head (bf16, d = 128), a KV
  // cache read by one 100-token chunk: valid; 2^23 keys: refused.
  {
    Case c;
    c.q = {0, 0, 100};
    c.kv = {0, (1 << 23) - 32 - 100, (1 << 23) - 32};
    c.seq = {0, 2};
    run_case(c, true, "kv at 2 GiB - 8 KiB");
    c.kv = {0, (1 << 23) - 100, 1 << 23};
    CHECK(run_case(c, false, "kv at 2 GiB") == MAGI_ERR_UNSUPPORTED, "K of exactly 2 GiB must be refused");
  }
  // Offsets next to INT32_MAX: refused by the tensor limits, without overflow.
  {
    Case c;
    c.q = {0, 64, INT32_MAX};
    c.kv = {0, 64, INT32_MAX};
    c.seq = {0, 2};
    CHECK(run_case(c, false, "offsets at INT32_MAX") != MAGI_OK, "offsets at INT32_MAX must be refused");
    c.q = {0, INT32_MAX - 1, INT32_MAX};
    c.kv = {0, 16, 32};
    c.hq = c.hk = 1;
    CHECK(run_case(c, false, "queries at INT32_MAX") != MAGI_OK, "T_q near INT32_MAX must be refused");
  }
  // One chunk of 8,388,000 tokens with one head: 21,844 query tiles each
  // listing 262,125 key tiles, 5.7e9 entries: refused before any list is built.
  {
    Case c;
    c.q = {0, 8388000};
    c.kv = c.q;
    c.seq = {0, 1};
    Owned o = own(c);
    std::string err;
    CHECK(validate_layout(&o.L, err) == MAGI_OK, "large single chunk validates: %s", err.c_str());
    HostPlan P;
    const magi_status_t s = build_host_plan(kPlanSelf, &o.L, nullptr, choose_tiling(c.dtype, c.d, 1), P, err);
    CHECK(s == MAGI_ERR_UNSUPPORTED && P.tile_codes.empty(), "list of > 2^31 entries must be refused: %d", int(s));
    BwdHostPlan B;
    CHECK(build_bwd_plan(&o.L, nullptr, B, err) == MAGI_ERR_UNSUPPORTED, "backward lists > 2^31 must be refused");
  }
}

// Streaming layouts (a cached prefix of n_cached chunks without queries, then
// n_active chunks with queries) have few dq items with long lists: the
// backward cuts them into pieces. The counts here are the ones the GPU parity
// cases of split dq items rely on (16 x 1100 with 8/1 heads: 35 items of 585
// tiles; 8 pieces would take two rounds of 256 workgroups, 7 take one).
void split_cases() {
  struct S { int n_cached, n_active, chunk, hq, hk, pieces; };
  const S cases[] = {{8, 2, 600, 6, 2, 2}, {8, 2, 600, 8, 1, 2}, {16, 1, 1100, 6, 2, 8}, {16, 1, 1100, 8, 1, 7}};
  for (const S& x : cases) {
    Case c;
    c.q = {0};
    c.kv = {0};
    for (int k = 0; k < x.n_cached + x.n_active; ++k) {
      c.kv.push_back(c.kv.back() + x.chunk);
      c.q.push_back(c.q.back() + (k < x.n_cached ? 0 : x.chunk));
    }
    c.seq = {0, x.n_cached + x.n_active};
    c.hq = x.hq;
    c.hk = x.hk;
    char tag[96];
    std::snprintf(tag, sizeof tag, "split %dx%d+%d %d/%d", x.n_cached, x.chunk, x.n_active, x.hq, x.hk);
    run_case(c, true, tag);
    Owned o = own(c);
    std::string err;
    BwdHostPlan B;
    CHECK(build_bwd_plan(&o.L, nullptr, B, err) == MAGI_OK, "%s: %s", tag, err.c_str());
    CHECK(!B.dq_merges.empty(), "%s: no split dq items", tag);
    for (const MergeItem& m : B.dq_merges)
      CHECK(m.n_pieces == x.pieces, "%s: block %d has %d pieces, want %d", tag, m.t0, m.n_pieces, x.pieces);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 200;
  const uint64_t first = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 0;
  int valid = 0, refused = 0;
  for (int i = 0; i < n; ++i) {
    std::mt19937_64 rng(first + uint64_t(i));
    const Case c = random_case(rng);
    char tag[64];
    std::snprintf(tag, sizeof tag, "seed %d", int(first) + i);
    if (run_case(c, false, tag) == MAGI_OK) ++valid;
    for (int how = 0; how < 8; ++how) {
      std::snprintf(tag, sizeof tag, "seed %d broken %d", int(first) + i, how);
      if (run_case(broken(c, how, rng), false, tag) != MAGI_OK) ++refused;
    }
  }
  limit_cases();
  split_cases();
  std::printf("plan_fuzz: %d seeds, %d valid layouts planned, %d of %d broken layouts refused, %d failed checks\n", n,
              valid, refused, 8 * n, g_failures);
  return g_failures == 0 ? 0 : 1;
}
