// Host-side planning for the block-causal attention forward: layout
// validation, tile classification and the GPU work list.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "magi_attn.h"

namespace magi {

// Kinds of plan. A plan has one or two phases, each an attention of the
// query stream over one key stream: a self plan has the block-causal
// self-attention, a cross plan the text cross-attention, and a parallel plan
// both (phase 0 self, phase 1 cross) in one launch.
enum PlanKind : int32_t { kPlanSelf = 0, kPlanCross = 1, kPlanParallel = 2 };

// One workgroup's work: query tokens [t0, t0 + tile_q) of `heads_per_item`
// consecutive query heads starting at h0, all of KV head kvh, over the key
// tiles of phase `phase` whose codes are tile_codes[tile_begin, tile_end);
// the first n_full of them are full tiles, the rest boundary tiles. Every
// list is followed by kTilePad padding entries (code -1, copy offset
// kNoTileOffset), so a kernel may read that far past tile_end.
struct WorkItem {
  int32_t t0;
  int32_t heads;       // (kvh << 16) | h0
  int32_t tile_begin;
  int32_t tile_end;    // == tile_begin: padding item, the workgroup exits at once
  int32_t n_full;
  int32_t slot;        // -1: writes out / lse; else a piece of a split item: writes partial slot `slot`
  int32_t phase;       // 0 or 1 (parallel plans: 1 = the cross-attention)
  int32_t pad;
};

// A split item: its rows (as in WorkItem) and the partial slots
// [slot0, slot0 + n_pieces) that the merge combines into out / lse of its
// phase. n_pieces == 0: rows that see no key at all (cross-attention rows of
// chunks without text): out = 0 and lse = -inf.
struct MergeItem {
  int32_t t0;
  int32_t heads;
  int32_t slot0;
  int32_t n_pieces;
  int32_t phase;
  int32_t pad[3];
};

// Split-KV policy (bf16): when a layout has fewer than kSplitBelowItems work
// items (too few to keep every compute unit busy to the end), items are cut
// into up to kMaxPieces contiguous ranges of their tile list, at least
// kMinPieceTiles long. The piece length is the mean list cut into the count
// that finishes the phase soonest, counting whole rounds of one item per CU
// and kPieceOverheadTiles per piece (query load, epilogue, merge).
// (Measured: the 4-chunks-on-16-cached streaming window, 384 items, gains;
// the two-video 256x256 layout, 768 short items, loses when split.)
constexpr int kNumCu = 256;
constexpr int kSplitBelowItems = 2 * kNumCu;
constexpr int kMaxPieces = 8;
constexpr int kMinPieceTiles = 64;
constexpr double kPieceOverheadTiles = 16.0;
// The backward's dk/dv items (bf16) split the same way when there are
// fewer (key block, KV head) items than CUs (a short text stream): each
// token-tile list is cut into up to kBwdMaxPieces pieces of at least
// kBwdMinPieceEntries entries, about total / kBwdSplitTargetItems each.
// (With 384 items, video 256x2, the split was 9% slower than none, and
// still 3.5% slower at 2 pieces per item, 768 pieces in three full rounds:
// the fp32 partials and the merge cost more than the tail saves.)
constexpr int kBwdSplitBelowItems = kNumCu;
constexpr int kBwdSplitTargetItems = 4 * kNumCu;
constexpr int kBwdMaxPieces = 64;
constexpr int kBwdMinPieceEntries = 8;
// The backward's dq items (bf16) take the forward's split rule when there are
// fewer than kBwdDqSplitBelowItems of them: the streaming window's 576 items
// ran in three rounds, the last a quarter full. A piece writes its fp32 dq-hat
// sums to a slot; a merge adds them in piece order and finishes the rows.
constexpr int kBwdDqSplitBelowItems = 4 * kNumCu;

constexpr int kTilePad = 16;
constexpr uint32_t kNoTileOffset = 0x80000000u;   // past any tile image buffer (< 2 GiB): reads give zeros

// Key tile code: kt * 2 + masked (masked = 1 for boundary tiles).
inline int32_t tile_code(int64_t kt, int masked) { return int32_t(kt * 2 + masked); }

// Key bounds of one query token: it attends keys [lo, hi).
struct RowBounds {
  int32_t lo;
  int32_t hi;
};

struct Tiling {
  int tile_q;          // query tokens per workgroup
  int tile_kv;         // keys per key tile
  int heads_per_item;  // query heads per workgroup
};

struct HostPlan {
  int32_t kind = kPlanSelf;
  int n_phases = 1;
  int n_chunks = 0, n_seqs = 0;
  int hq = 0, hk = 0, d = 0, dtype = 0;
  int64_t tq = 0;
  int64_t tk = 0;                    // keys of phase 0 (the video keys, or the text of a cross plan)
  int64_t tk_x = 0;                  // keys of phase 1 (parallel plans: the text)
  int64_t n_kt_img = 0;              // key tiles per KV head in the bf16 image arrays (phase 0's, then phase 1's)
  Tiling tiling{};
  std::vector<RowBounds> rows;       // [n_phases * tq]: phase p's bounds of token t at p * tq + t
  std::vector<int32_t> tile_codes;   // per (phase, query tile): full key tiles ascending, then boundary tiles
                                     // ascending, then padding; key tile indices are local to the phase's stream
  std::vector<uint32_t> tile_soff;   // parallel to tile_codes (bf16): byte offset of the key tile's image block,
                                     // (phase's first image tile + kt) * hk * tile_kv * d * 2; kNoTileOffset for padding
  std::vector<int32_t> qt_tiles;     // [n_phases * n_qt + 1] start of each (phase, query tile) list in tile_codes
  std::vector<int32_t> qt_ntiles;    // [n_phases * n_qt] key tiles per list (padding excluded)
  std::vector<int32_t> qt_full;      // [n_phases * n_qt] number of full key tiles per list
  std::vector<WorkItem> items;       // launch order (XCD-interleaved, padded)
  std::vector<MergeItem> merges;     // split items and key-less rows
  int32_t n_slots = 0;               // partial slots (pieces of split items)
  magi_attn_stats_t stats{};
};

// The backward's dk/dv work: keys [kb * key_block, (kb + 1) * key_block) of
// KV head kvh over the token tiles whose codes (tt * 2 + masked) are
// kv_tiles[tile_begin, tile_end), full tiles first; every query head of the
// KV head's group is a step of its own. Lists are followed by kTilePad
// padding codes (-1).
struct KeyItem {
  int32_t kb;
  int32_t kvh;
  int32_t tile_begin;
  int32_t tile_end;    // == tile_begin: padding item
  int32_t n_full;
  int32_t slot;        // -1: the whole list; else a piece, writing partial sums to this slot
  int32_t pad[2];
};

// A split (key block, KV head): pieces slot0 .. slot0 + n_pieces - 1.
struct KeyMerge {
  int32_t kb, kvh, slot0, n_pieces;
};

// Token ranges of the queries that see one key: its own video's [lo, hi),
// and [glo, ghi) for the rows of a last global block (empty otherwise).
struct KeyBounds {
  int32_t lo, hi, glo, ghi;
};

// Backward work lists of a training plan.
struct BwdHostPlan {
  HostPlan dq;                       // query-stationary dq items (never split)
  int32_t key_block = 0;             // keys per dk/dv item
  int32_t token_tile = 32;           // tokens per dk/dv step
  std::vector<KeyBounds> key_rows;   // [tk] token ranges of the queries that see each key
  std::vector<int32_t> kv_tiles;     // per key block: token tile codes, full first, then boundary; padded
  std::vector<KeyItem> items;        // launch order (XCD-interleaved, padded)
  std::vector<int32_t> dq_zero;      // (t0, first head) of the dq blocks whose rows see no key: dq = 0 there
  std::vector<MergeItem> dq_merges;  // split dq items (from dq.merges, those with pieces), merged after the dq kernel
  std::vector<int32_t> kv_zero;      // (first key, 0) of the key blocks no query sees: dk = dv = 0 there
  std::vector<KeyMerge> kv_merges;   // split (key block, KV head) items, summed after the dk/dv kernel
  int32_t n_kv_slots = 0;            // partial slots of their pieces
};

// Whether video s is a last global block (its queries see every key).
inline bool global_video(const magi_attn_layout_t* L, int s) { return L->last_global && s == L->n_seqs - 1; }

// First chunk whose keys chunk c of video s sees: the video's first chunk, or
// with a KV range R, the later of that and c - R + 1 (a global block: every
// chunk's keys, see row_bounds).
inline int first_visible_chunk(const magi_attn_layout_t* L, int s, int c) {
  const int first = L->seq_chunks[s];
  return L->kv_range > 0 && c - L->kv_range + 1 > first ? c - L->kv_range + 1 : first;
}

// Returns MAGI_OK or an error with a message in `err`.
magi_status_t validate_layout(const magi_attn_layout_t* layout, std::string& err);

// Checks the text side of a cross or parallel plan against a valid layout.
magi_status_t validate_text(const magi_attn_layout_t* layout, const magi_attn_text_t* text, int32_t kind,
                            std::string& err);

// Tiling used by the kernels for a dtype / head_dim / GQA group size.
Tiling choose_tiling(int dtype, int head_dim, int group);

// Tiling of the backward's dq items for a dtype / head_dim / GQA group size.
Tiling choose_bwd_tiling(int dtype, int head_dim, int group);

// Builds the full host plan of a kind (layout and text must already be
// valid; text is unused for kPlanSelf). allow_split = false keeps every work
// item whole; split_below is the item count under which a phase is split.
magi_status_t build_host_plan(int32_t kind, const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                              const Tiling& tiling, HostPlan& plan, std::string& err, bool allow_split = true,
                              int split_below = kSplitBelowItems);

// Builds the backward's work lists of a self-attention layout (valid).
// Backward lists of a self plan (text == NULL) or of a cross plan (the text
// keys are the keys).
magi_status_t build_bwd_plan(const magi_attn_layout_t* layout, const magi_attn_text_t* text, BwdHostPlan& plan,
                             std::string& err);

// Per-key token ranges: the queries that see each key.
void key_bounds(const magi_attn_layout_t* layout, std::vector<KeyBounds>& keys);

// Class of the pair (token tile [t0, t1), keys with ranges iv): 2 every
// (token, key) pair allowed, 1 some, 0 none; tokens at or past tq count as
// not allowed.
// The token ranges of the queries that see each text key (chunk c's rows see
// [text_begin[c], text_end[c])): the rows of the chunks whose range holds the
// key, merged where they touch. MAGI_ERR_UNSUPPORTED when some key is seen by
// more than two separate runs of rows.
magi_status_t text_key_bounds(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                              std::vector<KeyBounds>& keys, std::string& err);

int classify_key_pair(const std::vector<KeyBounds>& iv, int64_t t0, int64_t t1, int64_t tq);

// Per-query-token key bounds [lo, hi) of the block-causal self-attention
// (layout must be valid).
void row_bounds(const magi_attn_layout_t* layout, std::vector<RowBounds>& rows);

// Per-query-token text bounds [begin[c], end[c]) of the cross-attention.
void text_row_bounds(const magi_attn_layout_t* layout, const magi_attn_text_t* text, std::vector<RowBounds>& rows);

// Class of the pair (query tile rows [r0, r1), key tile [k0, k1)) given the
// distinct key intervals of those rows: 2 full, 1 boundary, 0 empty.
int classify_pair(const std::vector<RowBounds>& intervals, int64_t k0, int64_t k1, int64_t tk);

// Distinct consecutive key intervals of query rows [r0, r1).
void tile_intervals(const std::vector<RowBounds>& rows, int64_t r0, int64_t r1, std::vector<RowBounds>& out);

constexpr int kNumXcd = 8;

}  // namespace magi
