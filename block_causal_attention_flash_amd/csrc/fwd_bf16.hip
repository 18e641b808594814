// Block-causal QK-RMSNorm GQA attention forward, bf16, head_dim 64 or 128, gfx950.
//
// What is computed follows the MAGI-1 pages (paperlayer §2 / Figure 1 and
// §2.2.2; paper-notes §3.2.2 block pseudocode and Figure 15): per query row,
// softmax over its allowed keys of scale * <rms(q) * g_q, rms(k) * g_k>,
// times V, plus the natural-log log-sum-exp. The forward's cost is the two
// matrix products over the mask area (paperlayer §B.2.1), so both run on the
// bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Workgroup = one work item: 384 (token, head) rows, i.e. tile_q tokens of
// `heads_per_item` query heads that share one KV head; 8 waves, two per SIMD,
// 48 rows each (three 16-row MFMA blocks). Per 32-key tile:
//   * a pre-pass kernel has RMS-normalised every key once (k_hat = k / rms(k),
//     bf16) and written K-hat and V^T as per-tile LDS images into a
//     workspace; g_k is folded into the normalised queries, so
//     s_ij = <q'_i, k_hat_j>;
//   * the K-hat and V^T images are copied from global memory straight into
//     LDS rings (buffer_load ... lds, zero fill past the last tile) six tiles
//     ahead and serve all 384 rows: K/V leave L2 once per workgroup, not once
//     per query head;
//   * S^T = K Q'^T: every K fragment read from LDS feeds the three row blocks
//     of the wave (24 MFMAs per tile);
//   * O^T += V^T P^T: every V^T fragment feeds the three row blocks (24 MFMAs);
//     P stays in registers.
// Software pipeline of step i: the MFMAs of S(i) and of P(i-1) V(i-1), with
// the softmax of S(i-1) into P(i-1) on the vector ALUs between them, and the
// LDS reads kept ahead of the MFMAs. A workgroup barrier every second tile
// recycles the LDS rings.
//
// Queries are normalised in the prologue (RMS over head_dim, times
// g_q * g_k * scale * log2 e) and held in registers as bf16 MFMA operands.
//
// Softmax. QK-normalisation bounds every logit: s_ij = <q'_i, k_hat_j> <=
// |q'_i| |k_hat_j| <= |q'_i| sqrt(d) (a normalised key has norm at most
// sqrt(d)). Each wave takes B = the largest such bound of its 48 rows (log2
// units, with 1% for the bf16 rounding of k_hat and fp32 sums) and computes
// P = exp2(s - b) with the fixed shift b = max(0, B - 64), which the S products
// start from (their accumulators begin at -b): no running maximum, no
// rescaling and no VALU work for it. Softmax is invariant to the shift; P <=
// 2^64, and with fewer than 2^23 keys (the 2 GiB limit on K) the row sum
// stays below 2^87, so O = sum P v cannot overflow fp32 for |v| < 2^40. When
// B is far above the actual logits (gains much larger than the data's
// alignment uses, or keys pointing away from the query) a row's sum can fall
// out of [2^-100, 2^100); its wave then flags the work item, and a second
// instance of the kernel, launched after the first, redoes flagged items with
// a running row maximum, rescaling its accumulator only when the maximum has
// grown by more than 2^8. Unflagged items leave that instance at once. (One
// kernel holding both loops paid for the online loop's registers with spills
// in the static one.)
//
// The same kernel runs the block's text cross-attention (paperlayer §2.2.2,
// §2.2.3; paper-notes §3.2.2, §3.2.6): only the key stream and the per-row key
// bounds differ. A work item of phase 1 (parallel plans) takes the second set
// of queries, gains, temperature and outputs, and key tiles whose images
// follow the video keys' in the workspace. A row that sees no key (a chunk
// without text) gets out = 0 and lse = -inf.
//
// head_dim D is a template parameter (64 or 128): a tile image holds 32 x D
// bf16 values, so at D = 128 every thread copies 16 bytes of the K image and
// 16 of the V image per tile, and at D = 64 waves 0-3 copy the K image and
// waves 4-7 the V image. The S product takes D / 32 K fragments of two 16-key
// halves, the P V product D / 16 dim blocks.
//
// MFMA lane layouts (v_mfma_f32_16x16x32_bf16, lane l, g = l / 16):
//   A: A[l % 16][8g + j], B: B[8g + j][l % 16] (j = 0..7), D: D[4g + i][l % 16]
//   (i = 0..3).
#include "cdna4.hpp"
#include "kernels.hpp"

namespace magi {
namespace {

constexpr int BN = 32;                                // keys per tile
constexpr int NWAVE = 8;                              // two waves per SIMD
constexpr int NRB = 3;                                // 16-row MFMA blocks per wave
constexpr int ROWS = NWAVE * NRB * 16;                // 384 rows per workgroup
constexpr int NTHR = NWAVE * 64;
constexpr int NSTAGE = 8;                             // LDS ring depth (K and V each)
constexpr int NPRE = 2;                               // K fragments of the next tile read before the barrier
static_assert(ROWS == kBf16RowsPerItem, "rows per work item");

// Sizes that depend on head_dim D.
template <int D>
struct Geo {
  static_assert(D == 64 || D == 128, "head_dim");
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;   // 8 KiB (D = 128) or 4 KiB (D = 64)
  static constexpr int NKS = D / 32;                  // 32-dim steps of the S product
  static constexpr int NKF = 2 * NKS;                 // K fragments per tile (two 16-key halves per step)
  static constexpr int NDB = D / 16;                  // 16-dim blocks of O
  static constexpr int COPY_THREADS = TILE_BYTES / 16;  // threads copying one image (16 bytes each)
  static constexpr bool SPLIT_COPY = COPY_THREADS < NTHR;  // waves 0-3 copy K, waves 4-7 copy V
  static_assert(COPY_THREADS == NTHR || 2 * COPY_THREADS == NTHR, "copy units");
  // The workgroup barrier runs on even steps only. After the barrier of even
  // step i, copies start for K(i+6), V(i+5), K(i+7), V(i+6), in that order,
  // into stages that every wave left before this barrier. Before the barrier
  // of step i, K(i), K(i+1), K(i+2), V(i-1), V(i) must have landed (steps i and
  // i+1 read them; step i+1 reads K(i+2) ahead): everything issued at step
  // i-6 or earlier, plus K(i+2), the first copy issued at step i-4. A wave
  // waits for its own copies, the barrier publishes everyone's. When every
  // wave copies both images (D = 128), up to 7 copies younger than K(i+2) may
  // still fly. When a wave copies only K (D = 64), 3 may (K(i+3), K(i+4),
  // K(i+5)); a V wave needs V(i), issued at step i-6, with 4 younger, and
  // waits for 3 (one copy more than it needs).
  static constexpr int WAIT_YOUNGER = SPLIT_COPY ? 3 : 7;
  // Copies of the prologue (even steps -6, -4, -2) per wave, and how many of
  // them may fly once the wave's first copy (K(0) for a K wave) has landed.
  static constexpr int PROLOGUE_YOUNGER = SPLIT_COPY ? 5 : 11;
};
constexpr float kStaticBound = 64.0f;                // largest exponent of P on the static path
constexpr float kBoundSlack = 1.01f;                  // bf16 rounding of k_hat (2^-8), fp32 sums
constexpr float kMinRowSum = 0x1p-100f;               // static-path row sums outside [2^-100, 2^100):
constexpr float kMaxRowSum = 0x1p100f;                //   the item goes to the running-maximum instance
constexpr float kRescaleSlack = 8.0f;
constexpr float kNegInf = -__builtin_inff();

template <int D>
struct Smem {
  unsigned char k[NSTAGE][Geo<D>::TILE_BYTES];
  unsigned char v[NSTAGE][Geo<D>::TILE_BYTES];
  float gqk[D];
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Maximum over the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float sumsq8(bf16x8 a, float acc) {
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    bf16x2 p = {a[j], a[j + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

// Tile images. The pre-pass writes every (32-key tile, KV head) of K-hat and
// of V as a block of 64 D bytes that is copied byte for byte into an LDS ring
// stage. Both are chunk-major, so that a 16-lane phase of a ds_read_b128
// reads 256 contiguous bytes (no bank conflicts) and every fragment address is
// a per-lane base plus an instruction immediate:
//   K-hat: [D / 8 chunks][32 keys][16 bytes]: chunk c of key j (dims
//          8c..8c+7) at byte 512 c + 16 j;
//   V^T:   [4 chunks][D dims][16 bytes]: chunk c of dim row r holds keys
//          4c + {0..3} and 16 + 4c + {0..3} (the key order of a lane's P
//          fragment, see softmax_tile) at byte 16 D c + 16 r.
// Images are stored [tile][KV head], so copy thread t copies bytes
// [16t, 16t + 16) of one image.
struct LaneOffsets {
  unsigned dma;      // buffer offset of this thread's copy unit (the tile part goes in the scalar offset)
  unsigned kq;       // K ring, stage 0: fragment (ks, kb) at kq + 2048 ks + 256 kb
  unsigned vq;       // V ring, stage 0: fragment db at vq + 256 db
  // kq and vq are opaque to the compiler, so that stage and fragment offsets
  // stay instruction immediates wherever the rings lie in LDS.
};

template <int D>
__device__ __forceinline__ LaneOffsets lane_offsets(int tid, int kvh, unsigned k_ring, unsigned v_ring) {
  LaneOffsets o;
  const int lane = tid & 63;
  o.dma = unsigned(kvh) * Geo<D>::TILE_BYTES + unsigned(tid % Geo<D>::COPY_THREADS) * 16;
  o.kq = k_ring + unsigned((lane >> 4) * 512 + (lane & 15) * 16);
  o.vq = v_ring + unsigned((lane >> 4) * 16 * D + (lane & 15) * 16);
  asm("" : "+v"(o.kq));
  asm("" : "+v"(o.vq));
  return o;
}

template <int D>
struct WaveState {
  bf16x8 qf[NRB][Geo<D>::NKS];  // B operands of S^T: row (l & 15) of block rb, dims 32 ks + 8 (l >> 4) ..
  f32x4 o[NRB][Geo<D>::NDB];    // O^T accumulators: row (l & 15), dims 16 db + 4 (l >> 4) + i
  bf16x8 p[NRB];         // P of the previous tile (B operands of P V)
  bf16x8 kpre[NPRE];     // first K fragments of the current tile, read before the barrier
  f32x4 s0;              // initial S accumulator: -b, the wave's softmax shift (0 on the online path)
  float lsum[NRB];       // partial row sums over this lane's keys
  float m[NRB];          // online path: reference maximum (log2 units)
  int lo[NRB], hi[NRB];  // key bounds of the lane's rows
};

// K fragment f = 2 ks + kb of the tile in K stage kstage: keys 16 kb + (l & 15),
// dims 32 ks + 8 (l >> 4) ..
template <int D>
__device__ __forceinline__ bf16x8 k_frag(const LaneOffsets& lo, int kstage, int f) {
  return *(lds_bf16x8*)(size_t)(lo.kq + unsigned(kstage * Geo<D>::TILE_BYTES + (f >> 1) * 2048 + (f & 1) * 256));
}

// Phase 1: S^T(tile in K stage kstage); its first NPRE K fragments are in st.kpre.
template <int D>
__device__ __forceinline__ void qk_tile(int kstage, const LaneOffsets& lo, const WaveState<D>& st,
                                        f32x4 (&s)[NRB][2]) {
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) s[rb][0] = s[rb][1] = st.s0;
#pragma unroll
  for (int f = 0; f < Geo<D>::NKF; ++f) {
    const int ks = f >> 1, kb = f & 1;
    const bf16x8 a = f < NPRE ? st.kpre[f < NPRE ? f : 0] : k_frag<D>(lo, kstage, f);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, st.qf[rb][ks], s[rb][kb], 0, 0, 0);
  }
}

// Phase 2 (MFMA part): O^T += V^T P^T for one tile. The A operand of dim
// block db is one 16-byte chunk of the V^T image: dims 16 db + (l & 15), the
// 8 keys of chunk (l >> 4), in the order of the lane's P fragment.
template <int D>
__device__ __forceinline__ bf16x8 v_frag(const LaneOffsets& lo, int vstage, int db) {
  return *(lds_bf16x8*)(size_t)(lo.vq + unsigned(vstage * Geo<D>::TILE_BYTES + db * 256));
}

template <int D>
__device__ __forceinline__ void pv_tile(int vstage, const LaneOffsets& lo, const bf16x8 (&p)[NRB], WaveState<D>& st,
                                        const bf16x8* vpre = nullptr) {
#pragma unroll
  for (int db = 0; db < Geo<D>::NDB; ++db) {
    const bf16x8 a = (vpre && db < 2) ? vpre[db < 2 ? db : 0] : v_frag<D>(lo, vstage, db);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      st.o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p[rb], st.o[rb][db], 0, 0, 0);
  }
}

// Vector part: S -> P for one tile. Lane l holds, for row (l & 15) of each
// row block, keys 16 kb + 4 g + i (g = l >> 4; kb = 0, 1; i = 0..3); P element
// j of the B operand is key 16 (j / 4) + 4 g + (j % 4).
template <bool MASKED, bool STATIC, int D>
__device__ __forceinline__ void softmax_tile(f32x4 (&s)[NRB][2], int kt, WaveState<D>& st, bf16x8 (&p)[NRB],
                                             float (&alpha)[NRB], int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    if (MASKED) {
      // key allowed  <=>  (key - lo) < (hi - lo) as unsigned
      const unsigned base = unsigned(kt * BN + g * 4 - st.lo[rb]);
      const unsigned len = unsigned(st.hi[rb] - st.lo[rb]);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned rel = base + unsigned(kb * 16 + i);
          s[rb][kb][i] = rel < len ? s[rb][kb][i] : kNegInf;
        }
    }
    alpha[rb] = 1.0f;
    if (!STATIC) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[rb][kb][i]);
      mx = max_groups(mx);
      // keep the reference maximum unless the tile exceeds it by > 2^8
      const float m_new = (mx > st.m[rb] + kRescaleSlack) ? mx : st.m[rb];
      alpha[rb] = (m_new == st.m[rb]) ? 1.0f : __builtin_amdgcn_exp2f(st.m[rb] - m_new);
      st.m[rb] = m_new;
      const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[rb][kb][i] -= m_use;
    }
    // Row sums in fp32 of the unrounded exponentials (v_dot2 of the bf16 P
    // shares the matrix cores' issue and cost more alongside the products).
    // (the sum starts at the first pair rather than at 0: the same value, since
    // a sum of exponentials is never -0, without the add of 0 that strict fp
    // semantics would keep)
    float ls;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float e0 = __builtin_amdgcn_exp2f(s[rb][kb][i]);
        const float e1 = __builtin_amdgcn_exp2f(s[rb][kb][i + 1]);
        const bf16x2 pp = {(__bf16)e0, (__bf16)e1};
        p[rb][kb * 4 + i] = pp[0];
        p[rb][kb * 4 + i + 1] = pp[1];
        ls = (kb == 0 && i == 0) ? e0 + e1 : ls + (e0 + e1);
      }
    st.lsum[rb] = st.lsum[rb] * alpha[rb] + ls;
  }
}

// Per-workgroup constants of the tile loop.
struct LoopCtx {
  i32x4 rsk, rsv;             // buffer resources of the K-hat and V^T images
  unsigned k_base, v_base;    // LDS byte addresses of the K and V rings (plus this wave's 1 KiB block)
  const int* tiles;           // this item's key tile codes (for the boundary mask)
  const unsigned* soffs;      // this item's tile copy offsets; kNoTile in the padding after the list
  int n_tiles;
  // split copies (D = 64): whether this wave copies the K image (else the V
  // image), and that image's buffer resource and LDS ring base
  bool kwave;
  i32x4 rs_own;
  unsigned own_base;
};

// Starts the copies of the K tile image at scalar offset sk into stage js and
// of the V image at sv into stage jvs (kNoTile: zeros). With split copies a
// wave issues only its own image's copy.
template <int D>
__device__ __forceinline__ void issue_copies(const LoopCtx& c, const LaneOffsets& lo, unsigned sk, int js, unsigned sv,
                                             int jvs) {
  constexpr int TB = Geo<D>::TILE_BYTES;
  if constexpr (Geo<D>::SPLIT_COPY) {
    // wave-uniform selects, no branch: the unrolled steps stay one block
    dma16(c.rs_own, lo.dma, c.kwave ? sk : sv, c.own_base + unsigned(c.kwave ? js : jvs) * TB);
  } else {
    dma16(c.rsk, lo.dma, sk, c.k_base + js * TB);
    dma16(c.rsv, lo.dma, sv, c.v_base + jvs * TB);
  }
}

// Reads the first NPRE K fragments of the tile in K stage kstage into
// st.kpre; their latency is spent before the next barrier, where the wave
// waits anyway.
template <int D>
__device__ __forceinline__ void prefetch_k(int kstage, const LaneOffsets& lo, WaveState<D>& st) {
#pragma unroll
  for (int f = 0; f < NPRE; ++f) st.kpre[f] = k_frag<D>(lo, kstage, f);
}

// One step i. The stage of tile j is j % NSTAGE; callers that know i % NSTAGE
// at compile time pass it as si so every LDS offset folds into an immediate.
// On even steps (sync): wait for the copies listed at WAIT_YOUNGER, barrier,
// start the next four copies. Then S(i) on the matrix cores (its first K
// fragments were read at the end of the previous step), P(i-1) V(i-1) with
// the softmax of S(i) between its MFMAs, and the first K fragments of tile
// i+1 (published at this or the previous barrier).
// so4: copy offsets of K(i+6), K(i+7), V(i+5), V(i+6); used on even steps.
template <bool MASKED, bool STATIC, int D>
__device__ __forceinline__ void tile_step(const LoopCtx& c, const LaneOffsets& lo, WaveState<D>& st, int i, int si,
                                          bool sync, const unsigned (&so4)[4], int lane) {
  constexpr int NKF = Geo<D>::NKF, NDB = Geo<D>::NDB;
  if (sync) {
    wait_vmcnt<Geo<D>::WAIT_YOUNGER>();
    lds_barrier();
    issue_copies<D>(c, lo, so4[0], (si + 6) % NSTAGE, so4[2], (si + 5) % NSTAGE);
    issue_copies<D>(c, lo, so4[1], (si + 7) % NSTAGE, so4[3], (si + 6) % NSTAGE);
  }
  const int vst = (si + NSTAGE - 1) % NSTAGE;
  f32x4 s[NRB][2];
  qk_tile<D>(si, lo, st, s);
  bf16x8 vpre[2];
  vpre[0] = v_frag<D>(lo, vst, 0);
  vpre[1] = v_frag<D>(lo, vst, 1);
  if (STATIC && !MASKED) {
    // region 1: K reads two ahead of the S MFMAs, then the first V reads
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int f = 0; f < NKF; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, NRB, 0);
      if (f < NKF - NPRE) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  pv_tile<D>(vst, lo, st.p, st, vpre);
  bf16x8 p[NRB];
  float alpha[NRB];
  softmax_tile<MASKED, STATIC, D>(s, MASKED ? (c.tiles[i] >> 1) : 0, st, p, alpha, lane);
  if (!STATIC) {
    bool any = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) any |= alpha[rb] != 1.0f;
    if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) st.o[rb][db] *= alpha[rb];
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) st.p[rb] = p[rb];
  prefetch_k<D>((si + 1) % NSTAGE, lo, st);
  if (STATIC && !MASKED) {
    // region 2: P V MFMAs with the next V read and the softmax of S(i) between
    // them (the softmax's vector work per tile does not depend on D)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      __builtin_amdgcn_sched_group_barrier(0x008, NRB, 0);
      if (db < NDB - 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, 2 * NRB * (8 / NDB), 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, NPRE, 0);
  }
}

// Copy offsets used by even step i: K(i+6), K(i+7), V(i+5), V(i+6).
__device__ __forceinline__ void step_offsets(const unsigned* soffs, int i, unsigned (&so4)[4]) {
  so4[0] = soffs[i + 6];
  so4[1] = soffs[i + 7];
  so4[2] = soffs[i + 5];
  so4[3] = soffs[i + 6];
}

// so[u] is the copy offset of tile i0 + 5 + u.
template <bool STATIC, int U, int D>
__device__ __forceinline__ void unrolled_steps(const LoopCtx& c, const LaneOffsets& lo, WaveState<D>& st, int i0,
                                               const unsigned (&so)[NSTAGE + 1], int lane) {
  const unsigned so4[4] = {so[U + 1], so[U + 2], so[U], so[U + 1]};
  tile_step<false, STATIC, D>(c, lo, st, i0 + U, U, (U & 1) == 0, so4, lane);
  if constexpr (U + 1 < NSTAGE) unrolled_steps<STATIC, U + 1, D>(c, lo, st, i0, so, lane);
}

// Whether keys [lo, hi) meet any tile of the item's list (used only for rows
// whose static-path sum is out of range in items without full tiles: a full
// tile is seen by every row of the query tile).
__device__ __forceinline__ bool row_sees_a_tile(const LoopCtx& c, int lo, int hi) {
  for (int i = 0; i < c.n_tiles; ++i) {
    const int k0 = (c.tiles[i] >> 1) * BN;
    if (k0 < hi && k0 + BN > lo) return true;
  }
  return false;
}

// Full tiles first, then boundary tiles. Full tiles run NSTAGE at a time
// (NSTAGE is even, so groups start on even steps) with compile-time stages and
// their copy offsets loaded once per group; the rest one by one. Copy offsets
// are read up to 7 entries past the list, which the list's padding covers.
// The last tile's P V runs after the loop, behind one more barrier when the
// last step had none (V(n-1) was then not yet published).
template <bool STATIC, int D>
__device__ __forceinline__ void run_tiles(const LoopCtx& c, const LaneOffsets& lo, int n_full, WaveState<D>& st,
                                          int lane) {
  const int n = c.n_tiles;
  int i = 0;
  for (; i + NSTAGE <= n_full; i += NSTAGE) {
    unsigned so[NSTAGE + 1];
#pragma unroll
    for (int u = 0; u <= NSTAGE; ++u) so[u] = c.soffs[i + 5 + u];
    unrolled_steps<STATIC, 0, D>(c, lo, st, i, so, lane);
  }
  for (; i < n_full; ++i) {
    unsigned so4[4];
    step_offsets(c.soffs, i, so4);
    tile_step<false, STATIC, D>(c, lo, st, i, i % NSTAGE, (i & 1) == 0, so4, lane);
  }
  for (; i < n; ++i) {
    unsigned so4[4];
    step_offsets(c.soffs, i, so4);
    tile_step<true, STATIC, D>(c, lo, st, i, i % NSTAGE, (i & 1) == 0, so4, lane);
  }
  if ((n & 1) == 0) {
    wait_vmcnt<0>();
    lds_barrier();
  }
  pv_tile<D>((n + NSTAGE - 1) % NSTAGE, lo, st.p, st);
}

template <bool STATIC, int D>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_kernel(FwdParams prm, const int4* __restrict__ items, const int* __restrict__ tiles,
                const unsigned* __restrict__ soffs, const int2* __restrict__ rows) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(1024))) Smem<D> sm;
  const int4 item = items[2 * blockIdx.x];
  if (item.z == item.w) return;                       // padding item
  const int4 item2 = items[2 * blockIdx.x + 1];
  const int n_full = item2.x;
  const int slot = item2.y;                            // >= 0: a piece of a split item
  const bool px = item2.z != 0;                        // phase 1: the cross-attention of a parallel plan
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4;

  // ---- the running-maximum instance takes only the items that the static
  // instance (launched first, on the same stream) flagged
  if (!STATIC) {
    const int4* fl = reinterpret_cast<const int4*>(prm.item_flag + size_t(blockIdx.x) * NWAVE);
    const int4 f0 = fl[0], f1 = fl[1];
    if ((f0.x | f0.y | f0.z | f0.w | f1.x | f1.y | f1.z | f1.w) == 0) return;
  }
  const int kvh = item.y >> 16, h0 = item.y & 0xffff;
  const int tb = item.z, n_tiles = item.w - item.z;

  // Row r of the item (0..383) is token t0 + r % tile_q of head h0 + r / tile_q.
  WaveState<D> st;
  int tok[NRB], head[NRB];
  bool valid[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = (wave * NRB + rb) * 16 + (lane & 15);
    head[rb] = h0 + r / prm.tile_q;
    tok[rb] = item.x + r % prm.tile_q;
    valid[rb] = tok[rb] < prm.tq;
  }
  // ---- every load of the prologue first, older than every K/V copy, so that
  // they share one round trip: the gains, the query rows (unconditionally: a
  // row past the stream's end reads the last row, and its norm factor is 0)
  // and the rows' key bounds
  float gq = 0.0f, gk = 0.0f;
  if (tid < D) {
    gq = px ? prm.q_gain_x[tid] : prm.q_gain[tid];
    gk = px ? prm.k_gain_x[tid] : prm.k_gain[tid];
  }
  bf16x8 qr[NRB][G::NKS];
  int2 bnd[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int t = min(tok[rb], prm.tq - 1);
    const __bf16* qrow = reinterpret_cast<const __bf16*>(px ? prm.qx : prm.q) + (size_t(t) * prm.hq + head[rb]) * D;
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks) qr[rb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + g * 8);
    bnd[rb] = rows[(px ? prm.tq : 0) + t];
  }

  // ---- K/V copies ahead of the first step
  const unsigned img_bytes = unsigned(prm.n_kt_img) * unsigned(prm.hk) * unsigned(G::TILE_BYTES);
  const LaneOffsets lo = lane_offsets<D>(tid, kvh, lds_addr(&sm.k[0][0]), lds_addr(&sm.v[0][0]));
  // copy wave w writes its 1 KiB block of every image (w % 4 with split copies)
  const int cwave = G::SPLIT_COPY ? (wave & 3) : wave;
  LoopCtx ctx;
  ctx.rsk = make_rsrc(prm.ws, img_bytes);
  ctx.rsv = make_rsrc(static_cast<const unsigned char*>(prm.ws) + img_bytes, img_bytes);
  ctx.k_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm.k[0][0])) + cwave * 1024;
  ctx.v_base = __builtin_amdgcn_readfirstlane(lds_addr(&sm.v[0][0])) + cwave * 1024;
  ctx.tiles = tiles + tb;
  ctx.soffs = soffs + tb;
  ctx.n_tiles = n_tiles;
  ctx.kwave = __builtin_amdgcn_readfirstlane(wave < 4 ? 1 : 0) != 0;
  ctx.rs_own = ctx.kwave ? ctx.rsk : ctx.rsv;
  ctx.own_base = ctx.kwave ? ctx.k_base : ctx.v_base;
  // the copies of even steps -6, -4, -2 (V(-1) is a zero tile)
#pragma unroll
  for (int j = -6; j < 0; j += 2) {
    issue_copies<D>(ctx, lo, ctx.soffs[j + 6], (j + 6 + NSTAGE) % NSTAGE, j + 5 >= 0 ? ctx.soffs[j + 5] : kNoTile,
                    (j + 5 + NSTAGE) % NSTAGE);
    issue_copies<D>(ctx, lo, ctx.soffs[j + 7], (j + 7 + NSTAGE) % NSTAGE, ctx.soffs[j + 6],
                    (j + 6 + NSTAGE) % NSTAGE);
  }

  if (tid < D) sm.gqk[tid] = gq * gk * ((px ? prm.scale_x : prm.scale) * kLog2e);
  wait_vmcnt<G::PROLOGUE_YOUNGER>();                  // the wave's oldest copy (K(0) on a K-copying wave) landed
  __syncthreads();                                     // gqk and K(0) visible
  prefetch_k<D>(0, lo, st);

  // ---- query prologue: RMS-normalise, fold gains/temperature, to bf16
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks) ss = sumsq8(qr[rb][ks], ss);
    ss = sum_groups(ss);
    const float rq = valid[rb] ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + prm.eps) : 0.0f;
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks) {
      const int d0 = ks * 32 + g * 8;
      const f32x4 g0 = *LDS_PTR(const f32x4, &sm.gqk[d0]);
      const f32x4 g1 = *LDS_PTR(const f32x4, &sm.gqk[d0 + 4]);
#pragma unroll
      for (int j = 0; j < 8; ++j) st.qf[rb][ks][j] = (__bf16)(float(qr[rb][ks][j]) * rq * (j < 4 ? g0[j] : g1[j - 4]));
    }
    const int2 b = valid[rb] ? bnd[rb] : int2{0, 0};
    st.lo[rb] = b.x;
    st.hi[rb] = b.y;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) st.o[rb][db] = f32x4{};
    st.p[rb] = bf16x8{};                                      // tile -1: P = 0
    st.lsum[rb] = 0.0f;
    st.m[rb] = kNegInf;
  }
  // ---- the wave's softmax shift b = max(0, B - 64), B = max over its rows of
  // |q'| sqrt(d) (1 + slack), from the rounded operands the products use
  float shift = 0.0f;
  if (STATIC) {
    float qq = 0.0f;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float ss = 0.0f;
#pragma unroll
      for (int ks = 0; ks < G::NKS; ++ks) ss = sumsq8(st.qf[rb][ks], ss);
      qq = fmaxf(qq, sum_groups(ss));
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) qq = fmaxf(qq, __shfl_xor(qq, o, 64));
    const float bound = __builtin_sqrtf(qq * float(D)) * kBoundSlack;
    shift = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                          __builtin_bit_cast(int, fmaxf(0.0f, bound - kStaticBound))));
  }
  st.s0 = f32x4{-shift, -shift, -shift, -shift};
  run_tiles<STATIC, D>(ctx, lo, n_full, st, lane);

  // ---- epilogue: lane l holds dims 16 db + 4 g + i of row (l & 15) per block
  // (row coordinates recomputed rather than kept live through the loop)
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = (wave * NRB + rb) * 16 + (lane & 15);
    head[rb] = h0 + r / prm.tile_q;
    tok[rb] = item.x + r % prm.tile_q;
    valid[rb] = tok[rb] < prm.tq;
  }
  float lsr[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) lsr[rb] = sum_groups(st.lsum[rb]);
  if (STATIC) {
    // a row with keys whose sum left [2^-100, 2^100) flags the item for the
    // running-maximum instance (every wave writes its flag on every call)
    bool bad = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
      if (valid[rb] && !(lsr[rb] >= kMinRowSum && lsr[rb] < kMaxRowSum))
        bad |= n_full > 0 || row_sees_a_tile(ctx, st.lo[rb], st.hi[rb]);
    const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) prm.item_flag[size_t(blockIdx.x) * NWAVE + wave] = any_bad ? 1 : 0;
  }
  if (slot >= 0) {
    // piece of a split item: unnormalised O, reference maximum (the shift on
    // the static path: P = exp2(s - b)) and row sum, for the merge kernel
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float lsum = lsr[rb];
      const size_t r = size_t(slot) * ROWS + size_t((wave * NRB + rb) * 16 + (lane & 15));
#pragma unroll
      for (int db = 0; db < G::NDB; ++db)
        *reinterpret_cast<f32x4*>(prm.part_o + r * D + db * 16 + g * 4) = st.o[rb][db];
      if (g == 0) *reinterpret_cast<float2*>(prm.part_ml + r * 2) = float2{STATIC ? shift : st.m[rb], lsum};
    }
    return;
  }
  __bf16* const obase = reinterpret_cast<__bf16*>(px ? prm.outx : prm.out);
  float* const lbase = px ? prm.lsex : prm.lse;
  // The output leaves through LDS so that every store writes whole rows (a
  // lane's accumulators hold 4 dims of each of 16 rows: stored directly, each
  // store instruction would write 32 bytes in 16 rows). The wave's 48 rows go
  // to its own block of the rings, free once every wave has read its last V
  // tile, in row order with 16-byte chunks XOR-swizzled by the row (no bank
  // conflicts), and come back 16 bytes per lane, D / 8 lanes per row.
  constexpr int CPR = D / 8;                          // 16-byte chunks per row
  constexpr int WROWS = NRB * 16;                     // rows per wave
  constexpr int RPI = 64 / CPR;                       // rows per store instruction
  const auto swz = [](int row, int c) { return D == 128 ? (c ^ (row & 15)) : (c ^ ((row >> 1) & 7)); };
  __syncthreads();
  const unsigned ob = lds_addr(&sm.k[0][0]) + unsigned(wave * WROWS * G::ROW_BYTES);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float lsum = lsr[rb];
    const bool any = lsum > 0.0f;                       // false only for a row that sees no key
    const float inv = any ? 1.0f / lsum : 0.0f;
    const int row = rb * 16 + (lane & 15);
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (__bf16)(st.o[rb][db][i] * inv);
      const int c = 2 * db + (g >> 1);
      *LDS_PTR(bf16x4, size_t(ob + unsigned(row * G::ROW_BYTES + swz(row, c) * 16 + (g & 1) * 8))) = w;
    }
    if (valid[rb] && g == 0) {
      const float l2 = __builtin_amdgcn_logf(lsum);     // log2
      const float lse = !any ? kNegInf : ((STATIC ? shift : st.m[rb]) + l2) * kLn2;
      lbase[size_t(head[rb]) * prm.tq + tok[rb]] = lse;
    }
  }
  const int c = lane % CPR;
#pragma unroll
  for (int k = 0; k < WROWS / RPI; ++k) {
    const int row = k * RPI + lane / CPR;
    const bf16x8 x = *(lds_bf16x8*)(size_t)(ob + unsigned(row * G::ROW_BYTES + swz(row, c) * 16));
    const int r = wave * WROWS + row;                   // row of the item
    const int t = item.x + r % prm.tile_q;
    if (t < prm.tq)
      *reinterpret_cast<bf16x8*>(obase + (size_t(t) * prm.hq + h0 + r / prm.tile_q) * D + c * 8) = x;
  }
}

// Pre-pass: one workgroup per (32-key tile, KV head) writes that tile's two
// images (layouts above). Keys are RMS-normalised here, once per key:
// k_hat = k / sqrt(mean_d k^2 + eps) in bf16 (g_k is folded into the
// queries). Keys past the stream's end are written as zeros in both images.
// Workgroups [0, n0) cover the first key stream (k, v, tk); a parallel
// plan's text keys (kx, vx, tkx) follow, so image block b is workgroup b.
constexpr int PP_THREADS = 256;
template <int D>
__global__ void __launch_bounds__(PP_THREADS) kv_prepare_kernel(const __bf16* __restrict__ k0,
                                                                const __bf16* __restrict__ v0,
                                                                const __bf16* __restrict__ k1,
                                                                const __bf16* __restrict__ v1,
                                                                unsigned char* __restrict__ kimg,
                                                                unsigned char* __restrict__ vimg, int tk0, int tk1,
                                                                int n0, int hk, float eps) {
  constexpr int ROW_BYTES = Geo<D>::ROW_BYTES, CHUNKS = D / 8;   // 16-byte chunks per key row
  constexpr int ROUNDS = BN * CHUNKS / PP_THREADS;                // 2 (D = 128) or 1 (D = 64)
  __shared__ __attribute__((aligned(16))) unsigned char vs[Geo<D>::TILE_BYTES];
  const bool second = int(blockIdx.x) >= n0;
  const int b = second ? int(blockIdx.x) - n0 : int(blockIdx.x);
  const __bf16* const k = second ? k1 : k0;
  const __bf16* const v = second ? v1 : v0;
  const int tk = second ? tk1 : tk0;
  const int kt = b / hk, kvh = b % hk;
  const size_t img = size_t(blockIdx.x) * Geo<D>::TILE_BYTES;
  const int tid = threadIdx.x;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int u = tid + r * PP_THREADS;        // key u / CHUNKS, 16-byte chunk u % CHUNKS; CHUNKS lanes per key
    const int key = u / CHUNKS, c = u % CHUNKS;
    const int tok = kt * BN + key;
    bf16x8 x = {}, y = {};
    if (tok < tk) {
      const size_t src = (size_t(tok) * hk + kvh) * D + c * 8;
      x = *reinterpret_cast<const bf16x8*>(k + src);
      y = *reinterpret_cast<const bf16x8*>(v + src);
    }
    float ss = sumsq8(x, 0.0f);
    ss += dpp<0xB1>(ss);                  // quad_perm [1,0,3,2]
    ss += dpp<0x4E>(ss);                  // quad_perm [2,3,0,1]
    ss += dpp<0x141>(ss);                 // row_half_mirror: the other quad of 8 lanes
    if constexpr (CHUNKS == 16) ss += dpp<0x140>(ss);   // row_mirror: the other half of the 16 lanes
    const float rk = tok < tk ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps) : 0.0f;
    bf16x8 xn;
#pragma unroll
    for (int j = 0; j < 8; ++j) xn[j] = (__bf16)(float(x[j]) * rk);
    *reinterpret_cast<bf16x8*>(kimg + img + c * 512 + key * 16) = xn;
    *LDS_PTR(bf16x8, vs + key * ROW_BYTES + c * 16) = y;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int u = tid + r * PP_THREADS;        // V^T unit: chunk u / D, dim row u % D
    const int c = u / D, d = u % D;
    bf16x8 w;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = 16 * (j >> 2) + 4 * c + (j & 3);
      w[j] = *LDS_PTR(const __bf16, vs + key * ROW_BYTES + d * 2);
    }
    *reinterpret_cast<bf16x8*>(vimg + img + u * 16) = w;
  }
}

// Merge of a split item's pieces (one workgroup per merge entry): with the
// pieces' reference maxima m_s, row sums l_s and unnormalised outputs O_s,
// M = max m_s, w_s = 2^(m_s - M): out = sum w_s O_s / sum w_s l_s and
// lse = (M + log2 sum w_s l_s) ln 2. A thread handles 16 dims of one row. An
// entry without pieces (rows that see no key) writes out = 0, lse = -inf, as
// does a row whose pieces saw no key.
constexpr int MG_THREADS = 256;
template <int D>
__global__ void __launch_bounds__(MG_THREADS) merge_kernel(FwdParams prm) {
  constexpr int CPR = D / 16;                          // threads per row
  const int4 mi = prm.merges[2 * blockIdx.x];
  const bool px = prm.merges[2 * blockIdx.x + 1].x != 0;
  __bf16* const obase = reinterpret_cast<__bf16*>(px ? prm.outx : prm.out);
  float* const lbase = px ? prm.lsex : prm.lse;
  const int h0 = mi.y & 0xffff;
  for (int u = threadIdx.x; u < ROWS * CPR; u += MG_THREADS) {
    const int r = u / CPR, c = u % CPR;
    const int head = h0 + r / prm.tile_q, tok = mi.x + r % prm.tile_q;
    if (tok >= prm.tq) continue;
    float mmax = kNegInf;
    for (int sp = 0; sp < mi.w; ++sp) mmax = fmaxf(mmax, prm.part_ml[(size_t(mi.z + sp) * ROWS + r) * 2]);
    float l = 0.0f;
    f32x4 acc[4] = {};
    for (int sp = 0; sp < mi.w; ++sp) {
      const size_t rr = size_t(mi.z + sp) * ROWS + r;
      const float2 ml = *reinterpret_cast<const float2*>(prm.part_ml + rr * 2);
      const float w = ml.x == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(ml.x - mmax);
      l += w * ml.y;
      const f32x4* po = reinterpret_cast<const f32x4*>(prm.part_o + rr * D + c * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += w * po[q];
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    __bf16* orow = obase + (size_t(tok) * prm.hq + head) * D + c * 16;
    bf16x8 w0, w1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0[j] = (__bf16)(acc[0][j] * inv);
      w0[j + 4] = (__bf16)(acc[1][j] * inv);
      w1[j] = (__bf16)(acc[2][j] * inv);
      w1[j + 4] = (__bf16)(acc[3][j] * inv);
    }
    reinterpret_cast<bf16x8*>(orow)[0] = w0;
    reinterpret_cast<bf16x8*>(orow)[1] = w1;
    if (c == 0) lbase[size_t(head) * prm.tq + tok] = l > 0.0f ? (mmax + __builtin_amdgcn_logf(l)) * kLn2 : kNegInf;
  }
}

size_t image_bytes_bf16(long long n_kt_img, int hk, int d) { return size_t(n_kt_img) * size_t(hk) * BN * d * 2; }

template <int D>
hipError_t launch_fwd_bf16_d(const FwdParams& prm, int n_items, int n_merges, int n_slots, hipStream_t stream) {
  FwdParams p = prm;
  const size_t img = image_bytes_bf16(p.n_kt_img, p.hk, D);
  p.part_o = reinterpret_cast<float*>(static_cast<unsigned char*>(p.ws) + 2 * img);
  p.part_ml = p.part_o + size_t(n_slots) * ROWS * D;
  p.item_flag = reinterpret_cast<int*>(p.part_ml + size_t(n_slots) * ROWS * 2);
  if (n_items > 0) {
    if (p.n_kt_img > 0) {
      unsigned char* kimg = static_cast<unsigned char*>(p.ws);
      const int n0 = (p.tk + BN - 1) / BN * p.hk;
      hipLaunchKernelGGL(kv_prepare_kernel<D>, dim3(unsigned(p.n_kt_img) * unsigned(p.hk)), dim3(PP_THREADS), 0, stream,
                         static_cast<const __bf16*>(p.k), static_cast<const __bf16*>(p.v),
                         static_cast<const __bf16*>(p.kx), static_cast<const __bf16*>(p.vx), kimg, kimg + img, p.tk,
                         p.tkx, n0, p.hk, p.eps);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    // The static instance runs every item and flags the ones whose row sums
    // it lost; the running-maximum instance redoes only those.
    hipLaunchKernelGGL((fwd_bf16_kernel<true, D>), dim3(n_items), dim3(NTHR), 0, stream, p, p.items, p.tiles,
                       p.soffs, p.rows);
    hipLaunchKernelGGL((fwd_bf16_kernel<false, D>), dim3(n_items), dim3(NTHR), 0, stream, p, p.items, p.tiles,
                       p.soffs, p.rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_merges == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel<D>, dim3(n_merges), dim3(MG_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t workspace_bytes_bf16(long long n_kt_img, int hk, int head_dim, int n_slots, int n_items) {
  // K-hat images, V^T images, partial O, partial (m, l), per-wave item flags
  return 2 * image_bytes_bf16(n_kt_img, hk, head_dim) + size_t(n_slots) * ROWS * (head_dim + 2) * sizeof(float) +
         size_t(n_items) * NWAVE * sizeof(int);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, int n_items, int n_merges, int n_slots,
                           hipStream_t stream) {
  if (head_dim == 128) return launch_fwd_bf16_d<128>(p, n_items, n_merges, n_slots, stream);
  if (head_dim == 64) return launch_fwd_bf16_d<64>(p, n_items, n_merges, n_slots, stream);
  return hipErrorInvalidValue;
}

}  // namespace magi
