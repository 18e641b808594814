// Kernel launch interface shared by the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <string>

#include "magi_attn.h"

namespace magi {

// Records `msg` as the calling thread's last error (magi_attn_last_error)
// and returns `s`; for entry points defined outside api.cpp.
magi_status_t set_last_error(magi_status_t s, const std::string& msg);

// (token, head) rows of one bf16 work item: tile_q * heads_per_item.
constexpr int kBf16RowsPerItem = 384;
// Rows of one bf16 dq work item of the backward, and keys of one dk/dv item.
constexpr int kBwdRowsPerItem = 256;
constexpr int kBwdKeysPerItem = 256;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* ws;              // bf16 path: workspace of per-tile K-hat and V^T images (fwd_bf16.hip)
  void* out;
  float* lse;
  const float* q_gain;
  const float* k_gain;
  const int4* items;     // WorkItem[n_items], two int4 each
  const int* tiles;      // key tile codes (kt * 2 + masked); lists padded with code -1
  const unsigned* soffs; // parallel to tiles: byte offset of the tile's image block (bf16 path)
  const int2* rows;      // RowBounds[n_phases * tq]: phase p's bounds of token t at p * tq + t
  const int4* merges;    // MergeItem[n_merges], two int4 each: split items and key-less rows
  float* part_o;         // bf16 path, set by the launcher: partial O of each slot, [slot][384 rows][d] (workspace)
  float* part_ml;        // bf16 path, set by the launcher: partial (m, l) of each slot, [slot][384 rows][2]
  int* item_flag;        // bf16 path, set by the launcher: per (work item, wave) 1 when the static softmax lost a
                         // row's sum and the running-maximum instance must redo the item (workspace)
  float eps;
  float scale;           // softmax temperature on <q_hat, k_hat>
  int tq, tk, hq, hk;
  int tile_q, heads_per_item;
  // Phase 1 of a parallel plan (work items with phase 1): the text
  // cross-attention's queries, keys/values [tkx][hk][d], gains, temperature
  // and outputs. Unused by single-phase plans.
  const void* qx;
  const void* kx;
  const void* vx;
  void* outx;
  float* lsex;
  const float* q_gain_x;
  const float* k_gain_x;
  float scale_x;
  int tkx;
  int n_kt_img;          // bf16 path: key tiles per KV head in the image arrays (phase 0's keys, then phase 1's)
};

// Backward pass (dq, dk, dv and both gain gradients) of the self-attention.
// Work lists come from a training plan: query-stationary items for dq (the
// forward's item layout with `bwd_rows` rows per item) and key-stationary
// items for dk/dv (a block of keys of one KV head over the token tiles that
// see it).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const float* q_gain;
  const float* k_gain;
  void* dq;
  void* dk;
  void* dv;
  float* dq_gain;
  float* dk_gain;
  void* ws;               // workspace (layout: bwd_workspace_layout)
  float eps;
  float scale;
  int tq, tk, hq, hk;
  int tile_q, heads_per_item;        // dq items
  const int4* dq_items;   // WorkItem[n_dq_items]
  const int* dq_tiles;    // key tile codes per dq item list
  const unsigned* dq_soffs;
  const int2* rows;       // per-token key bounds [tq]
  const int4* kv_items;   // KeyItem[n_kv_items]
  const int* kv_tiles;    // token tile codes (tt * 2 + masked) per key block
  const int4* key_rows;   // per-key token ranges [tk]: own video [x, y), last global block [z, w)
                          // (cross plans: the two runs of rows that see a text key)
  const int2* dq_zero;    // (t0, first head) of the dq blocks (tile_q tokens x heads_per_item heads) with no key
  const int2* kv_zero;    // (first key, 0) of the key blocks (key_block keys x all KV heads) no query sees
  const int4* kv_merges;  // (key block, KV head, first slot, pieces) of the split dk/dv items
  const int4* dq_merges;  // MergeItem[n_dq_merges], two int4 each: rows and slots of the split dq items
  int key_block;
  int n_dq_items, n_kv_items, n_dq_zero, n_kv_zero, n_kv_merges, n_kv_slots;
  int n_dq_merges, n_dq_slots;
};

// Byte offsets of the backward workspace's parts.
struct BwdLayout {
  size_t qs, dos, rs, kh, vr, pgq, pgk, pkv, pdq, level, total;
};
// n_dq_rows / n_kv_rows: dq / dk-dv items plus merges (one gain partial
// each); n_kv_slots: partial slots of split dk/dv items (fp32 dV and dK-hat
// sums, 256 KiB each); n_dq_slots: those of split dq items (fp32 dq-hat sums,
// 128 KiB each).
BwdLayout bwd_workspace_layout(long long tq, long long tk, int hq, int hk, int head_dim, int n_dq_rows,
                               int n_kv_rows, int n_kv_slots, int n_dq_slots);
hipError_t launch_bwd_bf16(const BwdParams& p, int head_dim, hipStream_t stream);
hipError_t launch_bwd_fp32(const BwdParams& p, int head_dim, hipStream_t stream);
// Writes zeros where no item writes: dq over the p.dq_zero blocks, dk and dv
// over the p.kv_zero blocks (rows of row_bytes = head_dim * element size).
hipError_t launch_bwd_zero_rows(const BwdParams& p, int row_bytes, hipStream_t stream);
size_t bwd_workspace_bytes_fp32(long long tq, long long tk, int hq, int hk, int head_dim, int n_dq_items,
                                int n_kv_items);

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, int n_items, int n_merges, int n_slots,
                           hipStream_t stream);
size_t workspace_bytes_bf16(long long n_kt_img, int hk, int head_dim, int n_slots, int n_items);
hipError_t launch_fwd_fp32(const FwdParams& p, int head_dim, int n_items, int n_merges, hipStream_t stream);

}  // namespace magi
