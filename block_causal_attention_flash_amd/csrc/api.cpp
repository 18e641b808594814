// C ABI of the block-causal attention library: plans, forward, backward (declared in include/magi_attn.h).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>

#include "kernels.hpp"
#include "magi_attn.h"
#include "plan.hpp"

struct magi_attn_plan {
  magi::HostPlan host;
  bool train = false;            // has the backward's lists
  magi::BwdHostPlan bwd;
  int device = 0;
  void* dmem = nullptr;          // one allocation of every device list below
  const int4* d_items = nullptr;
  const int* d_tiles = nullptr;
  const unsigned* d_soffs = nullptr;
  const int4* d_merges = nullptr;
  const int2* d_rows = nullptr;
  const int4* d_dq_items = nullptr;
  const int* d_dq_tiles = nullptr;
  const unsigned* d_dq_soffs = nullptr;
  const int4* d_kv_items = nullptr;
  const int* d_kv_tiles = nullptr;
  const int4* d_key_rows = nullptr;
  const int2* d_dq_zero = nullptr;
  const int2* d_kv_zero = nullptr;
  const int4* d_kv_merges = nullptr;
  const int4* d_dq_merges = nullptr;
};

namespace {

thread_local std::string g_last_error;

magi_status_t fail(magi_status_t s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

magi_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MAGI_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

magi_status_t validate(int32_t kind, const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                       std::string& err) {
  magi_status_t s = magi::validate_layout(layout, err);
  if (s == MAGI_OK && kind != magi::kPlanSelf) s = magi::validate_text(layout, text, kind, err);
  return s;
}

magi::Tiling tiling_of(const magi_attn_layout_t* L) {
  return magi::choose_tiling(L->dtype, L->head_dim, L->n_q_heads / L->n_kv_heads);
}

magi_status_t plan_stats(int32_t kind, const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                         magi_attn_stats_t* stats) {
  std::string err;
  magi_status_t s = validate(kind, layout, text, err);
  if (s != MAGI_OK) return fail(s, err);
  if (!stats) return fail(MAGI_ERR_INVALID_ARG, "stats is NULL");
  magi::HostPlan hp;
  try {
    s = magi::build_host_plan(kind, layout, text, tiling_of(layout), hp, err);
  } catch (const std::bad_alloc&) {
    return fail(MAGI_ERR_NO_MEMORY, "host allocation failed");
  }
  if (s != MAGI_OK) return fail(s, err);
  *stats = hp.stats;
  return MAGI_OK;
}

// Classes of every (query tile, key tile) pair for per-row key bounds.
void classify_rows(const std::vector<magi::RowBounds>& rows, int64_t tq, int64_t tk, int32_t bm, int32_t bn,
                   int8_t* cls) {
  const int64_t n_qt = (tq + bm - 1) / bm, n_kt = (tk + bn - 1) / bn;
  std::vector<magi::RowBounds> iv;
  for (int64_t qt = 0; qt < n_qt; ++qt) {
    magi::tile_intervals(rows, qt * bm, std::min<int64_t>(tq, qt * bm + bm), iv);
    for (int64_t kt = 0; kt < n_kt; ++kt)
      cls[qt * n_kt + kt] = int8_t(magi::classify_pair(iv, kt * bn, kt * bn + bn, tk));
  }
}

// Host arrays copied into the plan's one device allocation, 256-byte aligned.
struct Upload {
  std::vector<std::pair<const void*, size_t>> parts;
  std::vector<size_t> offsets;
  size_t total = 0;
  size_t add(const void* p, size_t bytes) {
    const size_t o = total;
    parts.emplace_back(p, bytes);
    offsets.push_back(o);
    total += round_up(bytes, 256);
    return o;
  }
};

magi_status_t create_plan(int32_t kind, bool train, const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                          magi_attn_plan_t** out_plan) {
  if (!out_plan) return fail(MAGI_ERR_INVALID_ARG, "plan output pointer is NULL");
  *out_plan = nullptr;
  std::string err;
  magi_status_t s = validate(kind, layout, text, err);
  if (s != MAGI_OK) return fail(s, err);
  if (train && layout->dtype == MAGI_DTYPE_BF16 &&
      (int64_t(layout->q_offsets[layout->n_chunks]) + 31) / 32 * 32 * layout->n_q_heads * 256 >= (int64_t(1) << 31))
    return fail(MAGI_ERR_UNSUPPORTED, "training plans need T_q (rounded up to 32) * n_q_heads * 256 below 2 GiB");
  magi_attn_plan* p = new (std::nothrow) magi_attn_plan();
  if (!p) return fail(MAGI_ERR_NO_MEMORY, "host allocation failed");
  p->train = train;
  try {
    s = magi::build_host_plan(kind, layout, text, tiling_of(layout), p->host, err);
    if (s == MAGI_OK && train) s = magi::build_bwd_plan(layout, kind == magi::kPlanCross ? text : nullptr, p->bwd, err);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(MAGI_ERR_NO_MEMORY, "host allocation failed");
  }
  if (s != MAGI_OK) { delete p; return fail(s, err); }

  const auto& H = p->host;
  const auto& B = p->bwd;
  auto bytes = [](const auto& v) { return v.size() * sizeof(v[0]); };
  Upload up;
  const size_t o_items = up.add(H.items.data(), bytes(H.items));
  const size_t o_tiles = up.add(H.tile_codes.data(), bytes(H.tile_codes));
  const size_t o_soffs = up.add(H.tile_soff.data(), bytes(H.tile_soff));
  const size_t o_rows = up.add(H.rows.data(), bytes(H.rows));
  const size_t o_merges = up.add(H.merges.data(), bytes(H.merges));
  const size_t o_dq_items = up.add(B.dq.items.data(), bytes(B.dq.items));
  const size_t o_dq_tiles = up.add(B.dq.tile_codes.data(), bytes(B.dq.tile_codes));
  const size_t o_dq_soffs = up.add(B.dq.tile_soff.data(), bytes(B.dq.tile_soff));
  const size_t o_kv_items = up.add(B.items.data(), bytes(B.items));
  const size_t o_kv_tiles = up.add(B.kv_tiles.data(), bytes(B.kv_tiles));
  const size_t o_key_rows = up.add(B.key_rows.data(), bytes(B.key_rows));
  const size_t o_dq_zero = up.add(B.dq_zero.data(), bytes(B.dq_zero));
  const size_t o_kv_zero = up.add(B.kv_zero.data(), bytes(B.kv_zero));
  const size_t o_kv_merges = up.add(B.kv_merges.data(), bytes(B.kv_merges));
  const size_t o_dq_merges = up.add(B.dq_merges.data(), bytes(B.dq_merges));
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) { delete p; return hip_fail(e, "hipGetDevice"); }
  e = hipMalloc(&p->dmem, std::max<size_t>(up.total, 256));
  if (e != hipSuccess) {
    delete p;
    return e == hipErrorOutOfMemory ? fail(MAGI_ERR_NO_MEMORY, "hipMalloc of the plan failed") : hip_fail(e, "hipMalloc");
  }
  char* base = static_cast<char*>(p->dmem);
  for (size_t i = 0; i < up.parts.size() && e == hipSuccess; ++i)
    if (up.parts[i].second) e = hipMemcpy(base + up.offsets[i], up.parts[i].first, up.parts[i].second, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(p->dmem);
    delete p;
    return hip_fail(e, "hipMemcpy of the plan");
  }
  p->d_items = reinterpret_cast<const int4*>(base + o_items);
  p->d_tiles = reinterpret_cast<const int*>(base + o_tiles);
  p->d_soffs = reinterpret_cast<const unsigned*>(base + o_soffs);
  p->d_rows = reinterpret_cast<const int2*>(base + o_rows);
  p->d_merges = reinterpret_cast<const int4*>(base + o_merges);
  p->d_dq_items = reinterpret_cast<const int4*>(base + o_dq_items);
  p->d_dq_tiles = reinterpret_cast<const int*>(base + o_dq_tiles);
  p->d_dq_soffs = reinterpret_cast<const unsigned*>(base + o_dq_soffs);
  p->d_kv_items = reinterpret_cast<const int4*>(base + o_kv_items);
  p->d_kv_tiles = reinterpret_cast<const int*>(base + o_kv_tiles);
  p->d_key_rows = reinterpret_cast<const int4*>(base + o_key_rows);
  p->d_dq_zero = reinterpret_cast<const int2*>(base + o_dq_zero);
  p->d_kv_zero = reinterpret_cast<const int2*>(base + o_kv_zero);
  p->d_kv_merges = reinterpret_cast<const int4*>(base + o_kv_merges);
  p->d_dq_merges = reinterpret_cast<const int4*>(base + o_dq_merges);
  *out_plan = p;
  return MAGI_OK;
}

// k and v may be NULL when their key stream is empty (tk == 0).
magi_status_t check_tensors(const void* q, const void* k, const void* v, const float* q_gain, const float* k_gain,
                            float scale, void* out, float* lse, int64_t tk) {
  if (!q || !out || !lse || !q_gain || !k_gain || (tk > 0 && (!k || !v)))
    return fail(MAGI_ERR_INVALID_ARG, "NULL tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(MAGI_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(q_gain, 16) || !aligned(k_gain, 16))
    return fail(MAGI_ERR_INVALID_ARG, "lse must be 4-byte and the gains 16-byte aligned");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(MAGI_ERR_INVALID_ARG, "scale must be finite and > 0");
  return MAGI_OK;
}

magi_status_t check_workspace(const magi_attn_plan_t* plan, void* workspace, size_t workspace_bytes) {
  size_t need = 0;
  magi_attn_workspace_size(plan, &need);
  if (workspace_bytes < need) return fail(MAGI_ERR_INVALID_ARG, "workspace smaller than magi_attn_workspace_size()");
  if (need && (!workspace || !aligned(workspace, 16)))
    return fail(MAGI_ERR_INVALID_ARG, "workspace must be non-NULL and 16-byte aligned");
  return MAGI_OK;
}

// Common launch fields of a plan.
magi::FwdParams plan_params(const magi_attn_plan_t* plan, float rms_eps, void* workspace) {
  const auto& H = plan->host;
  magi::FwdParams prm{};
  prm.ws = workspace;
  prm.items = plan->d_items;
  prm.tiles = plan->d_tiles;
  prm.soffs = plan->d_soffs;
  prm.rows = plan->d_rows;
  prm.merges = plan->d_merges;
  prm.eps = rms_eps;
  prm.tq = int(H.tq);
  prm.tk = int(H.tk);
  prm.tkx = int(H.tk_x);
  prm.n_kt_img = int(H.n_kt_img);
  prm.hq = H.hq;
  prm.hk = H.hk;
  prm.tile_q = H.tiling.tile_q;
  prm.heads_per_item = H.tiling.heads_per_item;
  return prm;
}

magi_status_t launch(const magi_attn_plan_t* plan, const magi::FwdParams& prm, void* stream) {
  const auto& H = plan->host;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int n = int(H.items.size()), nm = int(H.merges.size());
  hipError_t e;
  if (H.dtype == MAGI_DTYPE_BF16) e = magi::launch_fwd_bf16(prm, H.d, n, nm, H.n_slots, st);
  else e = magi::launch_fwd_fp32(prm, H.d, n, nm, st);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return MAGI_OK;
}

}  // namespace

namespace magi {
magi_status_t set_last_error(magi_status_t s, const std::string& msg) { return fail(s, msg); }
}  // namespace magi

extern "C" {

int magi_attn_abi_version(void) { return MAGI_ATTN_ABI_VERSION; }

const char* magi_attn_status_str(magi_status_t s) {
  switch (s) {
    case MAGI_OK: return "ok";
    case MAGI_ERR_INVALID_ARG: return "invalid argument";
    case MAGI_ERR_UNSUPPORTED: return "unsupported";
    case MAGI_ERR_NO_MEMORY: return "out of memory";
    case MAGI_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* magi_attn_last_error(void) { return g_last_error.c_str(); }

magi_status_t magi_attn_classify_host(const magi_attn_layout_t* layout, int32_t bm, int32_t bn, int8_t* cls) {
  std::string err;
  magi_status_t s = magi::validate_layout(layout, err);
  if (s != MAGI_OK) return fail(s, err);
  if (bm < 1 || bn < 1) return fail(MAGI_ERR_INVALID_ARG, "tile sizes must be positive");
  if (!cls) return fail(MAGI_ERR_INVALID_ARG, "cls is NULL");
  std::vector<magi::RowBounds> rows;
  magi::row_bounds(layout, rows);
  const int32_t* kv = layout->kv_offsets ? layout->kv_offsets : layout->q_offsets;
  classify_rows(rows, layout->q_offsets[layout->n_chunks], kv[layout->n_chunks], bm, bn, cls);
  return MAGI_OK;
}

magi_status_t magi_attn_key_classify_host(const magi_attn_layout_t* layout, int32_t bk, int32_t bt, int8_t* cls) {
  std::string err;
  magi_status_t s = magi::validate_layout(layout, err);
  if (s != MAGI_OK) return fail(s, err);
  if (bk < 1 || bt < 1) return fail(MAGI_ERR_INVALID_ARG, "tile sizes must be positive");
  if (!cls) return fail(MAGI_ERR_INVALID_ARG, "cls is NULL");
  std::vector<magi::KeyBounds> keys;
  magi::key_bounds(layout, keys);
  const int32_t* kv = layout->kv_offsets ? layout->kv_offsets : layout->q_offsets;
  const int64_t tk = kv[layout->n_chunks], tq = layout->q_offsets[layout->n_chunks];
  const int64_t n_kb = (tk + bk - 1) / bk, n_tt = (tq + bt - 1) / bt;
  std::vector<magi::KeyBounds> iv;
  for (int64_t kb = 0; kb < n_kb; ++kb) {
    iv.assign(keys.begin() + kb * bk, keys.begin() + std::min<int64_t>(tk, kb * bk + bk));
    for (int64_t tt = 0; tt < n_tt; ++tt)
      cls[kb * n_tt + tt] = int8_t(magi::classify_key_pair(iv, tt * bt, tt * bt + bt, tq));
  }
  return MAGI_OK;
}

magi_status_t magi_attn_cross_classify_host(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                                            int32_t bm, int32_t bn, int8_t* cls) {
  std::string err;
  magi_status_t s = validate(magi::kPlanCross, layout, text, err);
  if (s != MAGI_OK) return fail(s, err);
  if (bm < 1 || bn < 1) return fail(MAGI_ERR_INVALID_ARG, "tile sizes must be positive");
  if (!cls) return fail(MAGI_ERR_INVALID_ARG, "cls is NULL");
  std::vector<magi::RowBounds> rows;
  magi::text_row_bounds(layout, text, rows);
  classify_rows(rows, layout->q_offsets[layout->n_chunks], text->t_text, bm, bn, cls);
  return MAGI_OK;
}

magi_status_t magi_attn_plan_stats(const magi_attn_layout_t* layout, magi_attn_stats_t* stats) {
  return plan_stats(magi::kPlanSelf, layout, nullptr, stats);
}

magi_status_t magi_attn_cross_plan_stats(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                                         int32_t with_self, magi_attn_stats_t* stats) {
  return plan_stats(with_self ? magi::kPlanParallel : magi::kPlanCross, layout, text, stats);
}

magi_status_t magi_attn_plan_create(const magi_attn_layout_t* layout, magi_attn_plan_t** out_plan) {
  return create_plan(magi::kPlanSelf, false, layout, nullptr, out_plan);
}

magi_status_t magi_attn_train_plan_create(const magi_attn_layout_t* layout, magi_attn_plan_t** out_plan) {
  return create_plan(magi::kPlanSelf, true, layout, nullptr, out_plan);
}

magi_status_t magi_attn_cross_train_plan_create(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                                                magi_attn_plan_t** out_plan) {
  return create_plan(magi::kPlanCross, true, layout, text, out_plan);
}

magi_status_t magi_attn_cross_plan_create(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                                          magi_attn_plan_t** out_plan) {
  return create_plan(magi::kPlanCross, false, layout, text, out_plan);
}

magi_status_t magi_attn_parallel_plan_create(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                                             magi_attn_plan_t** out_plan) {
  return create_plan(magi::kPlanParallel, false, layout, text, out_plan);
}

magi_status_t magi_attn_plan_destroy(magi_attn_plan_t* plan) {
  if (!plan) return MAGI_OK;
  magi_status_t s = MAGI_OK;
  if (plan->dmem) {
    hipError_t e = hipFree(plan->dmem);
    if (e != hipSuccess) s = hip_fail(e, "hipFree of the plan");
  }
  delete plan;
  return s;
}

magi_status_t magi_attn_workspace_size(const magi_attn_plan_t* plan, size_t* bytes) {
  if (!plan || !bytes) return fail(MAGI_ERR_INVALID_ARG, "plan or bytes is NULL");
  const auto& H = plan->host;
  *bytes = H.dtype == MAGI_DTYPE_BF16 ? magi::workspace_bytes_bf16(H.n_kt_img, H.hk, H.d, H.n_slots, int(H.items.size()))
                                      : 0;
  return MAGI_OK;
}

magi_status_t magi_attn_fwd(const magi_attn_plan_t* plan, const void* q, const void* k, const void* v,
                            const float* q_gain, const float* k_gain, float rms_eps, float scale, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MAGI_ERR_INVALID_ARG, "plan is NULL");
  const auto& H = plan->host;
  if (H.kind == magi::kPlanParallel)
    return fail(MAGI_ERR_INVALID_ARG, "a parallel plan runs with magi_attn_fwd_parallel");
  if (H.items.empty() && H.merges.empty()) return MAGI_OK;    // no query token: nothing to do
  magi_status_t s = check_workspace(plan, workspace, workspace_bytes);
  if (s != MAGI_OK) return s;
  s = check_tensors(q, k, v, q_gain, k_gain, scale, out, lse, H.tk);
  if (s != MAGI_OK) return s;
  if (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps)) return fail(MAGI_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");

  magi::FwdParams prm = plan_params(plan, rms_eps, workspace);
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.out = out;
  prm.lse = lse;
  prm.q_gain = q_gain;
  prm.k_gain = k_gain;
  prm.scale = scale;
  return launch(plan, prm, stream);
}

magi_status_t magi_attn_fwd_parallel(const magi_attn_plan_t* plan, const magi_attn_parallel_io_t* io, float rms_eps,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MAGI_ERR_INVALID_ARG, "plan is NULL");
  if (!io) return fail(MAGI_ERR_INVALID_ARG, "io is NULL");
  const auto& H = plan->host;
  if (H.kind != magi::kPlanParallel)
    return fail(MAGI_ERR_INVALID_ARG, "magi_attn_fwd_parallel needs a plan from magi_attn_parallel_plan_create");
  if (H.items.empty() && H.merges.empty()) return MAGI_OK;    // no query token: nothing to do
  magi_status_t s = check_workspace(plan, workspace, workspace_bytes);
  if (s != MAGI_OK) return s;
  s = check_tensors(io->q, io->k, io->v, io->q_gain, io->k_gain, io->scale, io->out, io->lse, H.tk);
  if (s != MAGI_OK) return s;
  s = check_tensors(io->q_x, io->k_x, io->v_x, io->q_gain_x, io->k_gain_x, io->scale_x, io->out_x, io->lse_x,
                    H.tk_x);
  if (s != MAGI_OK) return s;
  if (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps)) return fail(MAGI_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");

  magi::FwdParams prm = plan_params(plan, rms_eps, workspace);
  prm.q = io->q;
  prm.k = io->k;
  prm.v = io->v;
  prm.out = io->out;
  prm.lse = io->lse;
  prm.q_gain = io->q_gain;
  prm.k_gain = io->k_gain;
  prm.scale = io->scale;
  prm.qx = io->q_x;
  prm.kx = io->k_x;
  prm.vx = io->v_x;
  prm.outx = io->out_x;
  prm.lsex = io->lse_x;
  prm.q_gain_x = io->q_gain_x;
  prm.k_gain_x = io->k_gain_x;
  prm.scale_x = io->scale_x;
  return launch(plan, prm, stream);
}

magi_status_t magi_attn_bwd_workspace_size(const magi_attn_plan_t* plan, size_t* bytes) {
  if (!plan || !bytes) return fail(MAGI_ERR_INVALID_ARG, "plan or bytes is NULL");
  if (!plan->train) return fail(MAGI_ERR_INVALID_ARG, "not a training plan (magi_attn_train_plan_create)");
  const auto& H = plan->host;
  const int nq = int(plan->bwd.dq.items.size()), nk = int(plan->bwd.items.size());
  const auto& B = plan->bwd;
  *bytes = H.dtype == MAGI_DTYPE_BF16
               ? magi::bwd_workspace_layout(H.tq, H.tk, H.hq, H.hk, H.d, nq + int(B.dq_merges.size()),
                                            nk + int(B.kv_merges.size()), B.n_kv_slots, B.dq.n_slots).total
                                      : magi::bwd_workspace_bytes_fp32(H.tq, H.tk, H.hq, H.hk, H.d, nq, nk);
  return MAGI_OK;
}

magi_status_t magi_attn_bwd(const magi_attn_plan_t* plan, const magi_attn_bwd_io_t* io, float rms_eps, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MAGI_ERR_INVALID_ARG, "plan is NULL");
  if (!io) return fail(MAGI_ERR_INVALID_ARG, "io is NULL");
  if (!plan->train)
    return fail(MAGI_ERR_INVALID_ARG,
                "magi_attn_bwd needs a plan from magi_attn_train_plan_create or magi_attn_cross_train_plan_create");
  const auto& H = plan->host;
  size_t need = 0;
  magi_attn_bwd_workspace_size(plan, &need);
  if (workspace_bytes < need) return fail(MAGI_ERR_INVALID_ARG, "workspace smaller than magi_attn_bwd_workspace_size()");
  if (need && (!workspace || !aligned(workspace, 16)))
    return fail(MAGI_ERR_INVALID_ARG, "workspace must be non-NULL and 16-byte aligned");
  const void* tens[] = {io->q, io->out, io->dout, io->dq};
  for (const void* t : tens)
    if (!t || !aligned(t, 16)) return fail(MAGI_ERR_INVALID_ARG, "q, out, dout, dq must be non-NULL and 16-byte aligned");
  const void* ktens[] = {io->k, io->v, io->dk, io->dv};                 // may be NULL when there are no keys
  for (const void* t : ktens)
    if ((H.tk > 0 && !t) || !aligned(t, 16))
      return fail(MAGI_ERR_INVALID_ARG, "k, v, dk, dv must be non-NULL (unless T_k == 0) and 16-byte aligned");
  if (!io->lse || !aligned(io->lse, 4) || !io->q_gain || !io->k_gain || !aligned(io->q_gain, 16) ||
      !aligned(io->k_gain, 16) || !io->dq_gain || !io->dk_gain || !aligned(io->dq_gain, 4) || !aligned(io->dk_gain, 4))
    return fail(MAGI_ERR_INVALID_ARG, "lse, the gains and the gain gradients must be non-NULL and aligned");
  if (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps)) return fail(MAGI_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(MAGI_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (H.tq == 0) return MAGI_OK;

  magi::BwdParams b{};
  b.q = io->q;
  b.k = io->k;
  b.v = io->v;
  b.out = io->out;
  b.dout = io->dout;
  b.lse = io->lse;
  b.q_gain = io->q_gain;
  b.k_gain = io->k_gain;
  b.dq = io->dq;
  b.dk = io->dk;
  b.dv = io->dv;
  b.dq_gain = io->dq_gain;
  b.dk_gain = io->dk_gain;
  b.ws = workspace;
  b.eps = rms_eps;
  b.scale = scale;
  b.tq = int(H.tq);
  b.tk = int(H.tk);
  b.hq = H.hq;
  b.hk = H.hk;
  b.tile_q = plan->bwd.dq.tiling.tile_q;
  b.heads_per_item = plan->bwd.dq.tiling.heads_per_item;
  b.dq_items = plan->d_dq_items;
  b.dq_tiles = plan->d_dq_tiles;
  b.dq_soffs = plan->d_dq_soffs;
  b.rows = plan->d_rows;
  b.kv_items = plan->d_kv_items;
  b.kv_tiles = plan->d_kv_tiles;
  b.key_rows = plan->d_key_rows;
  b.dq_zero = plan->d_dq_zero;
  b.n_dq_zero = int(plan->bwd.dq_zero.size() / 2);
  b.kv_zero = plan->d_kv_zero;
  b.n_kv_zero = int(plan->bwd.kv_zero.size() / 2);
  b.key_block = plan->bwd.key_block;
  b.kv_merges = plan->d_kv_merges;
  b.n_kv_merges = int(plan->bwd.kv_merges.size());
  b.n_kv_slots = plan->bwd.n_kv_slots;
  b.dq_merges = plan->d_dq_merges;
  b.n_dq_merges = int(plan->bwd.dq_merges.size());
  b.n_dq_slots = plan->bwd.dq.n_slots;
  b.n_dq_items = int(plan->bwd.dq.items.size());
  b.n_kv_items = int(plan->bwd.items.size());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = H.dtype == MAGI_DTYPE_BF16 ? magi::launch_bwd_bf16(b, H.d, st) : magi::launch_bwd_fp32(b, H.d, st);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return MAGI_OK;
}

magi_status_t magi_attn_fwd_simple(const void* q, const void* k, const void* v, void* out, float* lse,
                                   const int32_t* chunk_offsets, int32_t n_chunks, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, int32_t dtype, const float* q_gain,
                                   const float* k_gain, float rms_eps, float scale, void* stream) {
  if (!chunk_offsets) return fail(MAGI_ERR_INVALID_ARG, "chunk_offsets is NULL");
  const int32_t seq[2] = {0, n_chunks};
  magi_attn_layout_t L{};
  L.n_seqs = 1;
  L.seq_chunks = seq;
  L.n_chunks = n_chunks;
  L.q_offsets = chunk_offsets;
  L.kv_offsets = chunk_offsets;
  L.n_q_heads = n_q_heads;
  L.n_kv_heads = n_kv_heads;
  L.head_dim = head_dim;
  L.dtype = dtype;
  magi_attn_plan_t* plan = nullptr;
  magi_status_t s = magi_attn_plan_create(&L, &plan);
  if (s != MAGI_OK) return s;
  size_t ws_bytes = 0;
  magi_attn_workspace_size(plan, &ws_bytes);
  void* ws = nullptr;
  if (ws_bytes) {
    hipError_t e = hipMalloc(&ws, ws_bytes);
    if (e != hipSuccess) {
      magi_attn_plan_destroy(plan);
      return e == hipErrorOutOfMemory ? fail(MAGI_ERR_NO_MEMORY, "hipMalloc of the workspace failed")
                                      : hip_fail(e, "hipMalloc");
    }
  }
  s = magi_attn_fwd(plan, q, k, v, q_gain, k_gain, rms_eps, scale, out, lse, ws, ws_bytes, stream);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (s == MAGI_OK && e != hipSuccess) s = hip_fail(e, "hipStreamSynchronize");
  const std::string keep = g_last_error;
  if (ws) (void)hipFree(ws);
  magi_status_t d = magi_attn_plan_destroy(plan);
  if (s != MAGI_OK) { g_last_error = keep; return s; }
  return d;
}

}  // extern "C"
