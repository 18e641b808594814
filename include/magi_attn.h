/*
 * magi_attn.h -- C ABI of an MI355X (gfx950) block-causal attention forward.
 *
 * The operation (MAGI-1 pages): the self-attention of a chunk-wise
 * autoregressive video diffusion transformer over packed video-chunk tokens.
 *   - paperlayer summary §2 and Figure 1; paper-notes §2 and its Figure 1:
 *     attention is bidirectional among the tokens of one chunk and causal
 *     across chunks (a chunk sees itself and all earlier chunks of its video);
 *   - paper-notes Figure 15 ("varlen block-causal"): several videos packed in
 *     one token stream never attend to each other;
 *   - paperlayer §2.2.2, paper-notes §3.2.2 (architecture list and the DiT block
 *     pseudocode): queries and keys are normalised per head right before the
 *     attention ("QK-Norm"), and query heads share key/value heads (GQA);
 *   - paperlayer §2.4.4: keys/values of clean chunks come from a KV cache, so
 *     the key stream may be longer than the query stream.
 * The backward of the self-attention (dq, dk, dv and the gradients of both
 * QK-norm gains) runs from the forward's saved log-sum-exp: see
 * magi_attn_bwd. Beside it, the same library runs the block's text cross-attention
 * (paperlayer §2.2.2 and §2.2.3; paper-notes §3.2.2 and §3.2.6), alone or
 * together with the self-attention in one launch: see magi_attn_text_t.
 *
 * Per query token i of chunk c (video s) and query head h, with KV head
 * g = h / (n_q_heads / n_kv_heads):
 *   q_hat = q * q_gain / sqrt(mean_d(q^2) + eps),  k_hat likewise with k_gain,
 *   s_ij  = scale * <q_hat_ih, k_hat_jg> for keys j in
 *           [kv_offsets[f], kv_offsets[c + 1]), f = seq_chunks[s] (with a KV
 *           range R >= 1: max(seq_chunks[s], c - R + 1)); all of [0, T_k)
 *           for the queries of a last global block,
 *   out_ih = sum_j softmax_j(s_ij) v_jg,   lse_hi = ln sum_j exp(s_ij).
 *
 * Conventions shared by every entry point:
 *   - Every function returns a magi_status_t; nothing aborts or throws across
 *     the ABI. magi_attn_last_error() returns a per-thread detail message.
 *   - Device tensors are caller-owned, contiguous, 16-byte aligned:
 *       q, out : [T_q][n_q_heads][head_dim]    (T_q = q_offsets[n_chunks])
 *       k, v   : [T_k][n_kv_heads][head_dim]   (T_k = kv_offsets[n_chunks])
 *       lse    : [n_q_heads][T_q] float32 (natural log)
 *       q_gain, k_gain : [head_dim] float32
 *     q, k, v and out share the element type of the layout (bf16 or fp32).
 *     out and lse must not alias any input. The library keeps no tensor
 *     pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 */
#ifndef MAGI_ATTN_H
#define MAGI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MAGI_API __attribute__((visibility("default")))
#else
#define MAGI_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define MAGI_ATTN_ABI_VERSION 7

typedef enum magi_status {
  MAGI_OK = 0,
  MAGI_ERR_INVALID_ARG = 1,   /* bad layout, NULL or misaligned pointer, bad size */
  MAGI_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement    */
  MAGI_ERR_NO_MEMORY = 3,     /* host or device allocation failed                 */
  MAGI_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed       */
} magi_status_t;

typedef enum magi_dtype {
  MAGI_DTYPE_BF16 = 0,
  MAGI_DTYPE_FP32 = 1
} magi_dtype_t;

/*
 * Chunk layout of the packed query and key streams (host arrays, read during
 * the call only):
 *   seq_chunks[n_seqs+1]  : video s owns chunks [seq_chunks[s], seq_chunks[s+1]);
 *                           seq_chunks[0] == 0, seq_chunks[n_seqs] == n_chunks,
 *                           strictly increasing (no empty video).
 *   q_offsets[n_chunks+1] : chunk c owns queries [q_offsets[c], q_offsets[c+1]);
 *                           non-decreasing from 0 (a chunk may own no queries,
 *                           as the clean chunks of a KV cache do).
 *   kv_offsets[n_chunks+1]: chunk c owns keys/values [kv_offsets[c], kv_offsets[c+1]);
 *                           non-decreasing from 0; NULL means kv_offsets == q_offsets.
 * kv_range             : 0: a chunk sees every earlier chunk of its video and
 *                        itself (block-causal); R >= 1: chunk c sees only
 *                        chunks max(first chunk of its video, c - R + 1) .. c
 *                        (the pages' "KV range" of streaming inference:
 *                        paperlayer §2.4.4, paper-notes §3.4.4 and Figure 12).
 * last_global          : 1: the last video is a global block (the pages'
 *                        "varlen block-causal with a (last) global block":
 *                        paper-notes Figure 15(g), paperlayer Figure 23):
 *                        its queries see every key of the stream, [0, T_k);
 *                        no other video sees its keys. 0: off.
 * A chunk that owns queries must see at least one key.
 * head_dim: 64 or 128. n_q_heads % n_kv_heads == 0.
 */
typedef struct magi_attn_layout {
  int32_t n_seqs;
  const int32_t* seq_chunks;
  int32_t n_chunks;
  const int32_t* q_offsets;
  const int32_t* kv_offsets;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;              /* magi_dtype_t */
  int32_t kv_range;           /* 0: block-causal; R >= 1: the last R chunks of the video */
  int32_t last_global;        /* 1: the last video's queries see every key of the stream */
} magi_attn_layout_t;

/*
 * Text side of the cross-attention (host arrays, read during the call only).
 * In every transformer block of MAGI-1 the video tokens also attend to the
 * text condition, beside the self-attention and from the same query
 * projection, with QK-Norm and GQA (paperlayer §2.2.2; paper-notes §3.2.2:
 * architecture list, spec table, block pseudocode). Prompts are given per
 * chunk (paperlayer §2.2.3) and chunks that are already clean carry no text
 * (paper-notes §3.2.6). For query token i of chunk c and query head h:
 *   s_ij   = scale_x * <q_hat_ih, k_hat_jg>  for text keys j in [text_begin[c], text_end[c]),
 *   out_ih = sum_j softmax_j(s_ij) v_jg,     lse_hi = ln sum_j exp(s_ij),
 * with q_hat, k_hat RMS-normalised as above (with the cross-attention's own
 * gains) and the values not normalised. A chunk with text_begin[c] ==
 * text_end[c] has no text: its rows get out = 0 and lse = -inf.
 *   t_text           : tokens of the packed text stream, >= 0
 *   text_begin[n_chunks], text_end[n_chunks] : 0 <= begin <= end <= t_text
 * Text keys/values are [t_text][n_kv_heads][head_dim] (same heads, head_dim
 * and dtype as the layout); with t_text == 0 their pointers may be NULL.
 * Several chunks may share one prompt's range.
 */
typedef struct magi_attn_text {
  int32_t t_text;
  const int32_t* text_begin;
  const int32_t* text_end;
} magi_attn_text_t;

typedef struct magi_attn_plan magi_attn_plan_t;   /* opaque */

/*
 * Validates a layout, classifies every (query tile, key tile) pair as full,
 * boundary or empty, orders the non-empty work for the GPU and uploads the
 * work list to device memory of the current HIP device (one allocation, owned
 * by the plan). Host arrays are copied; the caller may free them afterwards.
 * A plan is immutable after creation and may be used by concurrent calls on
 * several streams of the device it was created on.
 * Errors: MAGI_ERR_INVALID_ARG (layout rules above), MAGI_ERR_UNSUPPORTED
 * (head_dim/dtype combination; K or V of 2 GiB or more, for bf16 with T_k
 * rounded up to a multiple of 32; T_q * n_q_heads of 2^31 or more),
 * MAGI_ERR_NO_MEMORY, MAGI_ERR_HIP. On error
 * *plan is set to NULL. Validation runs before any HIP call.
 */
MAGI_API magi_status_t magi_attn_plan_create(const magi_attn_layout_t* layout, magi_attn_plan_t** plan);

/*
 * Plan of the text cross-attention alone, run with magi_attn_fwd, passing
 * the text keys/values as k and v and the cross-attention's gains and
 * temperature. The layout is validated as above (its q_offsets, chunks,
 * heads, head_dim and dtype are used; its kv_offsets and kv_range are not);
 * the text must satisfy the rules of magi_attn_text_t. Errors as for
 * magi_attn_plan_create, with the text's K/V under the same 2 GiB limit.
 */
MAGI_API magi_status_t magi_attn_cross_plan_create(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                                                   magi_attn_plan_t** plan);

/*
 * Plan of the parallel attention block's two attentions (paperlayer §2.2.2:
 * self- and cross-attention side by side from one query projection): the
 * block-causal self-attention of `layout` and the cross-attention of `text`,
 * run together by magi_attn_fwd_parallel as one pass (one pre-pass over both
 * key streams, one main-kernel launch holding both attentions' work items).
 * Errors as for the two plans above; for bf16 the re-laid-out video and text
 * keys together must stay under 2 GiB.
 */
MAGI_API magi_status_t magi_attn_parallel_plan_create(const magi_attn_layout_t* layout,
                                                      const magi_attn_text_t* text, magi_attn_plan_t** plan);

/*
 * Plan for training: the self-attention plan of magi_attn_plan_create (it
 * runs the forward with magi_attn_fwd) plus the work lists of the backward
 * (magi_attn_bwd): query-stationary lists for dq and, for dk/dv, the token
 * tiles that see each block of keys. Same rules and errors as
 * magi_attn_plan_create; in addition, for bf16, T_q rounded up to a multiple
 * of 32 times n_q_heads times 256 bytes must stay under 2 GiB (the
 * backward's per-row images).
 */
MAGI_API magi_status_t magi_attn_train_plan_create(const magi_attn_layout_t* layout, magi_attn_plan_t** plan);

/*
 * Plan for training the text cross-attention (magi_attn_text_t): the cross
 * plan of magi_attn_cross_plan_create (forward with magi_attn_fwd, the text
 * keys/values as k and v) plus the backward's lists, with the text keys as
 * the keys (the training of the pages' cross-attention branch, paperlayer
 * §2.2.2 with §4.1.2). Same rules and errors as magi_attn_cross_plan_create
 * and magi_attn_train_plan_create; in addition MAGI_ERR_UNSUPPORTED when a
 * text token is seen by more than two separate runs of query rows (chunks
 * that share a prompt and are adjacent count as one run).
 */
MAGI_API magi_status_t magi_attn_cross_train_plan_create(const magi_attn_layout_t* layout,
                                                         const magi_attn_text_t* text, magi_attn_plan_t** plan);

/* Frees the plan and its device memory (synchronous with respect to the host;
 * the caller must not destroy a plan that queued work still uses). NULL is OK. */
MAGI_API magi_status_t magi_attn_plan_destroy(magi_attn_plan_t* plan);

/*
 * Device workspace bytes that magi_attn_fwd (or magi_attn_fwd_parallel)
 * needs for this plan. bf16: the RMS-normalised keys and the values
 * re-laid out in 32-key tiles, 2 * n_tiles * 32 * n_kv_heads * head_dim * 2
 * bytes with n_tiles = ceil(T_k / 32) (parallel plans: plus ceil(t_text / 32)),
 * plus, when the
 * plan splits work items along the key axis (layouts with too few items to
 * fill the GPU), the pieces' partial results, pieces * 384 * (head_dim + 2)
 * * 4 bytes, plus 32 bytes per work item (the flags by which the static
 * softmax hands items to the running-maximum instance). fp32: 0.
 */
MAGI_API magi_status_t magi_attn_workspace_size(const magi_attn_plan_t* plan, size_t* bytes);

/*
 * Enqueues the forward pass of a self or cross plan on `stream`: out and lse
 * as defined at the top (cross plans: as defined at magi_attn_text_t, with
 * k, v the text keys/values [t_text][n_kv_heads][head_dim]).
 * rms_eps >= 0 is added to mean(x^2) inside the square root; scale > 0 is the
 * softmax temperature applied to <q_hat, k_hat> (1/sqrt(head_dim) usually).
 * `workspace` is caller-owned device memory of at least
 * magi_attn_workspace_size() bytes, 16-byte aligned (may be NULL when that
 * size is 0); the call overwrites it, so concurrent calls need distinct
 * workspaces. Allocates nothing and never synchronises, so it can be
 * captured in a HIP graph. Errors: MAGI_ERR_INVALID_ARG (NULL/misaligned
 * pointer, workspace too small, bad eps or scale, a parallel plan),
 * MAGI_ERR_HIP (launch failure). Device faults surface at the caller's next
 * synchronisation.
 */
MAGI_API magi_status_t magi_attn_fwd(const magi_attn_plan_t* plan,
                            const void* q, const void* k, const void* v,
                            const float* q_gain, const float* k_gain,
                            float rms_eps, float scale,
                            void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch array behind magi_attn_fwd_noalloc. */
#define MAGI_ATTN_NOALLOC_SCRATCH_BYTES 268435456u

/*
 * magi_attn_fwd without any allocation, for callers that cannot allocate
 * device memory or pass a workspace: code being captured into a HIP graph,
 * tight serving loops, harnesses that forbid allocation. Same arguments,
 * results and errors as magi_attn_fwd, minus the workspace: the library uses
 * a static device array of MAGI_ATTN_NOALLOC_SCRATCH_BYTES (256 MiB) bytes
 * that every GPU it runs on holds until the process ends. Plans whose
 * magi_attn_workspace_size() exceeds that are refused with
 * MAGI_ERR_UNSUPPORTED (for example the 480x832 video: 613 MB of tile images;
 * the 256x256 two-video batch fits). Allocates nothing and never
 * synchronises. All calls on one GPU share its array, which keeps the last
 * call's contents: calls that overlap in time on one GPU (two streams, two
 * host threads) race and must be serialised by the caller. The device current
 * at the call must be the device of the plan and of `stream`.
 */
MAGI_API magi_status_t magi_attn_fwd_noalloc(const magi_attn_plan_t* plan,
                                             const void* q, const void* k, const void* v,
                                             const float* q_gain, const float* k_gain,
                                             float rms_eps, float scale,
                                             void* out, float* lse, void* stream);

/*
 * Tensors of one call of the parallel attention block. The self-attention
 * takes q, k, v, its gains and scale and writes out, lse, as defined at the
 * top. The cross-attention takes q_x (the same query projection; the pages
 * apply RoPE to the self-attention branch only, so q_x may differ from q, or
 * be the same pointer), the text keys/values k_x, v_x
 * [t_text][n_kv_heads][head_dim], its own gains and scale_x, and writes
 * out_x [T_q][n_q_heads][head_dim] and lse_x [n_q_heads][T_q]. Alignment and
 * ownership as for magi_attn_fwd; no output may alias an input or another
 * output.
 */
typedef struct magi_attn_parallel_io {
  const void* q;
  const void* k;
  const void* v;
  const float* q_gain;
  const float* k_gain;
  float scale;
  void* out;
  float* lse;
  const void* q_x;
  const void* k_x;
  const void* v_x;
  const float* q_gain_x;
  const float* k_gain_x;
  float scale_x;
  void* out_x;
  float* lse_x;
} magi_attn_parallel_io_t;

/*
 * Enqueues both attentions of a parallel plan on `stream` as one pass (the
 * short cross-attention work items fill the tail of the self-attention
 * launch). rms_eps applies to both normalisations. Workspace, allocation and
 * synchronisation rules as for magi_attn_fwd. Errors: those of magi_attn_fwd,
 * and MAGI_ERR_INVALID_ARG for a plan that is not a parallel plan or a NULL io.
 */
MAGI_API magi_status_t magi_attn_fwd_parallel(const magi_attn_plan_t* plan, const magi_attn_parallel_io_t* io,
                                              float rms_eps, void* workspace, size_t workspace_bytes,
                                              void* stream);

/* Device workspace bytes of magi_attn_bwd for a training plan (bf16: the
 * re-laid-out normalised queries, upstream gradients, keys and values, about
 * 2 * |q| + 2 * |k| bytes, plus 256 KiB of fp32 partial sums per piece when
 * the plan splits its dk/dv work because it has fewer key blocks times KV
 * heads than the GPU has CUs (a short text stream: about 1024 pieces), and
 * 128 KiB per piece when it splits its dq work because it has fewer than
 * 1024 dq items (a streaming window with a long cached prefix: up to 8
 * pieces per item);
 * fp32: the normalised queries, 2 * |q|; plus per-workgroup gain partials). */
MAGI_API magi_status_t magi_attn_bwd_workspace_size(const magi_attn_plan_t* plan, size_t* bytes);

/*
 * Tensors of one backward call. Inputs: q, k, v, q_gain, k_gain as given to
 * the forward; out and lse that the forward returned for them; dout, the
 * gradient of the loss with respect to out ([T_q][n_q_heads][head_dim], the
 * element type of the layout). Outputs (caller-owned, written in full):
 * dq [T_q][n_q_heads][head_dim], dk and dv [T_k][n_kv_heads][head_dim] (the
 * element type of the layout), dq_gain and dk_gain [head_dim] float32. For a
 * cross training plan, k and v are the text keys/values, dk and dv
 * [t_text][n_kv_heads][head_dim] their gradients, and the gains the
 * cross-attention's; with t_text == 0, k, v, dk and dv may be NULL. Rows
 * that see no key (a chunk without text) get dq = 0.
 */
typedef struct magi_attn_bwd_io {
  const void* q;
  const void* k;
  const void* v;
  const float* q_gain;
  const float* k_gain;
  const void* out;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dq_gain;
  float* dk_gain;
} magi_attn_bwd_io_t;

/*
 * Enqueues the backward pass of a training plan's attention on `stream`: the
 * gradients of a loss with respect to q, k, v and both gains, given its
 * gradient dout with respect to out (the chain rule of the forward defined
 * at the top; the attention's backward from saved softmax statistics,
 * paperlayer §4.1.2 and §B.1). rms_eps and scale must be the forward's. The
 * softmax is recomputed from lse, so lse must be the one the forward wrote
 * for these inputs. Workspace, allocation and synchronisation rules as for
 * magi_attn_fwd. Errors: MAGI_ERR_INVALID_ARG (not a training plan, NULL or
 * misaligned pointer, workspace too small, bad eps or scale), MAGI_ERR_HIP.
 */
MAGI_API magi_status_t magi_attn_bwd(const magi_attn_plan_t* plan, const magi_attn_bwd_io_t* io, float rms_eps,
                                     float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One-shot form for a single video of self-attention (q and kv offsets both
 * = chunk_offsets[n_chunks+1], host array): builds a plan, allocates the
 * workspace, enqueues the forward on `stream`, waits for the stream, and
 * frees both. Not capturable (it allocates and synchronises). Same errors as
 * above, plus MAGI_ERR_NO_MEMORY.
 */
MAGI_API magi_status_t magi_attn_fwd_simple(const void* q, const void* k, const void* v,
                                   void* out, float* lse,
                                   const int32_t* chunk_offsets, int32_t n_chunks,
                                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                   int32_t dtype, const float* q_gain, const float* k_gain,
                                   float rms_eps, float scale, void* stream);

/*
 * Host-only tile classifier (no HIP call): for query tiles of `bm` tokens and
 * key tiles of `bn` tokens, writes cls[qt * n_kt + kt] = 2 (every pair allowed),
 * 1 (some allowed, some not) or 0 (none allowed), n_qt = ceil(T_q/bm),
 * n_kt = ceil(T_k/bn); keys at or beyond T_k count as not allowed. `cls`
 * must hold n_qt * n_kt bytes. Same layout validation as plan creation.
 */
MAGI_API magi_status_t magi_attn_classify_host(const magi_attn_layout_t* layout, int32_t bm, int32_t bn,
                                      int8_t* cls);

/* Host-only summary of what a plan for `layout` would launch. */
typedef struct magi_attn_stats {
  int64_t unmasked_pairs;     /* allowed (query, key) pairs per query head          */
  int64_t full_pairs;         /* (query tile, key tile) pairs classified full        */
  int64_t boundary_pairs;     /* ... boundary (masked on the GPU)                    */
  int64_t empty_pairs;        /* ... empty (never launched)                          */
  int64_t executed_pairs;     /* (query, key) pairs per query head the kernel computes */
  int32_t tile_q;             /* query tokens per workgroup                          */
  int32_t tile_kv;            /* keys per key tile                                   */
  int32_t heads_per_item;     /* query heads per workgroup                           */
  int32_t n_items;            /* workgroups launched (including XCD padding)         */
} magi_attn_stats_t;

MAGI_API magi_status_t magi_attn_plan_stats(const magi_attn_layout_t* layout, magi_attn_stats_t* stats);

/* Host-only: the classes of the backward's (key block, token tile) pairs:
 * cls[kb * n_tt + tt] for blocks of `bk` keys and tiles of `bt` query
 * tokens (n_kb = ceil(T_k/bk), n_tt = ceil(T_q/bt)), with the values and
 * validation of magi_attn_classify_host. */
MAGI_API magi_status_t magi_attn_key_classify_host(const magi_attn_layout_t* layout, int32_t bk, int32_t bt,
                                                   int8_t* cls);

/* Host-only: the tile classes of the cross-attention's text mask (as
 * magi_attn_classify_host, with n_kt = ceil(t_text / bn)). */
MAGI_API magi_status_t magi_attn_cross_classify_host(const magi_attn_layout_t* layout,
                                                     const magi_attn_text_t* text, int32_t bm, int32_t bn,
                                                     int8_t* cls);

/* Host-only summary of a cross plan (with_self == 0) or a parallel plan
 * (with_self != 0; pair counts are the sums over both attentions). */
MAGI_API magi_status_t magi_attn_cross_plan_stats(const magi_attn_layout_t* layout, const magi_attn_text_t* text,
                                                  int32_t with_self, magi_attn_stats_t* stats);

MAGI_API const char* magi_attn_status_str(magi_status_t status);
MAGI_API const char* magi_attn_last_error(void);
MAGI_API int magi_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAGI_ATTN_H */
