// Backward of the block-causal QK-RMSNorm GQA attention, bf16, head_dim 64 or 128, gfx950.
//
// Training needs the gradients of the attention of the MAGI-1 pages
// (paperlayer §2 / Figure 1, §2.2.2; paper-notes §3.2.2 and Figure 15), and
// the pages' attention kernel runs its backward from the forward's saved
// softmax statistics (paperlayer §4.1.2, §B.1). With q_hat = rms(q) g_q,
// k' = rms(k) g_k scale log2(e) (both rounded to bf16 once), the natural
// log-sum-exp lse of each row and the upstream gradient dO:
//   P_ij  = 2^(<q_hat_i, k'_j> - lse_i log2 e)        (recomputed, no max pass)
//   dP_ij = <dO_i, v_j>,  D_i = <dO_i, O_i>,  dS_ij = P_ij (dP_ij - D_i)
//   dq_hat_i = sum_j dS_ij k'_j / log2 e              (dq kernel; = scale sum_j dS_ij k_hat_j)
//   dk_hat_j = scale sum_i dS_ij q_hat_i              (dk/dv kernel, over all query heads of j's group)
//   dv_j     = sum_i P_ij dO_i                        (dk/dv kernel)
//   dx = (g dx_hat - u mean_d(u g dx_hat)) / r,  u = x / r   (RMSNorm, in the epilogues)
//   dg = sum over rows of u dx_hat                    (per-workgroup partials, then one reduction)
//
// Kernels, in stream order:
//   prep_q  per (32-token tile, query head): the tile images of q_hat and of
//           dO, and the row statistics negated (-lse log2 e, -D: the
//           starting values of the S and dP accumulators);
//   prep_k  per (32-key tile, KV head): the images of k' and of V;
//   dq      query-stationary (the forward's order): 8 waves x 32 rows, per
//           key tile S^T and dP^T on the matrix cores, dS on the vector ALUs,
//           then (dq_hat)^T += k'^T dS^T;
//   dkdv    key-stationary: 8 waves x 32 keys of one KV head, per
//           (32-token tile, query head) S and dP, then dV^T += dO^T P and
//           dK^T += q_hat^T dS; when a plan has fewer key blocks x KV heads
//           than CUs, each list is cut into pieces that write fp32 sums;
//   merge   adds a split list's pieces in order and finishes like dkdv (and,
//           for the split dq items of small layouts, like dq);
//   zero    dq of rows no item covers (they see no key) and dk, dv of key
//           blocks no row sees;
//   reduce  the gain gradients from the per-workgroup partials.
// On boundary tiles a branch that unmasked steps skip sets S to -inf outside
// each row's (dq) or each key's (dk/dv) allowed range before the
// exponentials. A cross-attention plan runs the same kernels: its keys are
// the text's, a row's range is its chunk's text, a text key's rows are the
// chunks whose prompt holds it.
// Every image is [D / 8 chunks][32 row slots][16 B] (head_dim D = 64 or 128,
// a template parameter): chunk c of row r (dims 8c..8c+7) sits at byte
// 512 c + 16 (r XOR 12 (c mod 2)). The XOR keeps each
// 16-row block of a chunk in its own 256 bytes, so row reads stay contiguous,
// and puts the odd chunk's rows of a transposed read (rows 4 g .. 4 g + 3 of
// chunks 2 b and 2 b + 1 for the 16 lanes of group g) on the other banks: a
// quarter wave covers 32 distinct banks and a half wave 64. A lane reads
// an MFMA operand fragment in row order with one ds_read_b128 (row l % 16,
// dims 32 ks + 8 (l / 16) ..), or transposed with two LDS transpose loads
// (ds_read_b64_tr_b16: within 16 lanes, lane i's element j comes from the
// 8-byte address of lane 4j + i / 4, element i % 4) that give lane l dim
// 16 db + l % 16 of rows 4 (l / 16) + {0..3} and 16 + 4 (l / 16) + {0..3}:
// the row order of a lane's fragment of a 16x16 result pair. Copies into LDS
// rings use LDS-direct buffer loads four steps ahead; on even steps a wave
// waits for its copies of the step pair and the workgroup barrier publishes
// both stages (and frees the two stages the next pair of copies fills). An
// image is 64 D bytes: at D = 128 every thread copies 16 bytes of each of a
// step's two images, at D = 64 waves 0-3 copy the first and waves 4-7 the
// second.
#include "cdna4.hpp"
#include "kernels.hpp"

namespace magi {
namespace {

constexpr int TT = 32;                       // tokens per image (and per dk/dv step), keys per dq tile
constexpr int NTHR = 512;
constexpr int RING = 8;                      // LDS ring stages: copies four steps ahead, a barrier every second step
static_assert(kBwdRowsPerItem == 8 * 32 && kBwdKeysPerItem == 8 * 32, "8 waves per workgroup");

// Sizes that depend on head_dim D.
template <int D>
struct BGeo {
  static_assert(D == 64 || D == 128, "head_dim");
  static constexpr int IMG = TT * D * 2;     // 8 KiB (D = 128) or 4 KiB (D = 64)
  static constexpr int NKS = D / 32;         // 32-dim steps of a product over d
  static constexpr int NDB = D / 16;         // 16-dim blocks of a result over d
  static constexpr int COPY_THREADS = IMG / 16;
  static constexpr bool SPLIT_COPY = COPY_THREADS < NTHR;  // one image per half workgroup
  static_assert(COPY_THREADS == NTHR || 2 * COPY_THREADS == NTHR, "copy units");
};

// Sums over the 16 lanes of a group / over 8 lanes.
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 8, 64);
  return x;
}
__device__ __forceinline__ float sum8(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 4, 64);
  return x;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Byte offset of (chunk c, row r) in an image.
__device__ __forceinline__ constexpr unsigned img_off(int c, int r) {
  return unsigned(512 * c + 16 * (r ^ (12 * (c & 1))));
}

// Per-lane byte offset of the transposed fragment reads: lane l = 16 g + 4 j + q
// points at row 4 g + j, dims 4 q .. 4 q + 3 of dim block 0 of an image (rows
// 16 .. 31 lie 256 bytes further: the XOR does not touch bit 4 of the row).
__device__ __forceinline__ unsigned tr_lane_offset(int lane) {
  const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
  return img_off(q >> 1, 4 * g + j) + unsigned(8 * (q & 1));
}

// A operand of 16 dims (block db) x 32 rows, rows in the order of a lane's
// fragment of a 16x16 result pair, read transposed from a row image at
// `addr` = image base + tr_lane_offset(lane).
__device__ __forceinline__ bf16x8 tr_frag(unsigned addr, int db) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(size_t)(addr + 1024 * db));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(size_t)(addr + 1024 * db + 256));
  const i16x4 w[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, w);
}

// ------------------------------------------------------------------ pre-passes

// One workgroup per (32-token tile tt, query head h), image b = tt * hq + h;
// thread t: token row j = t / 8, dims [D / 8 (t % 8), +D / 8) (PC = D / 64
// chunks of 8 dims).
constexpr int PREP_THREADS = 256;
template <int D>
__global__ void __launch_bounds__(PREP_THREADS) bwd_prep_q_kernel(BwdParams p, BwdLayout L) {
  constexpr int PC = D / 64, IMG = BGeo<D>::IMG;
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int b = blockIdx.x, tt = b / p.hq, h = b % p.hq;
  const int t = threadIdx.x, j = t >> 3, part = t & 7;
  const int tok = tt * TT + j;
  const bool valid = tok < p.tq;
  const size_t row = (size_t(tok) * p.hq + h) * D + part * 8 * PC;
  bf16x8 q[PC] = {}, dd[PC] = {}, oo[PC] = {};
  if (valid) {
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      q[c] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.q) + row + 8 * c);
      dd[c] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.dout) + row + 8 * c);
      oo[c] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.out) + row + 8 * c);
    }
  }
  float ss = 0.0f, dsum = 0.0f;
#pragma unroll
  for (int c = 0; c < PC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ss += float(q[c][e]) * float(q[c][e]);
      dsum += float(dd[c][e]) * float(oo[c][e]);
    }
  ss = sum8(ss);
  dsum = sum8(dsum);
  const float rq = valid ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps) : 0.0f;
#pragma unroll
  for (int c = 0; c < PC; ++c) {
    bf16x8 qh;
#pragma unroll
    for (int e = 0; e < 8; ++e) qh[e] = (__bf16)(float(q[c][e]) * rq * p.q_gain[part * 8 * PC + 8 * c + e]);
    const size_t at = size_t(b) * IMG + img_off(PC * part + c, j);
    *reinterpret_cast<bf16x8*>(ws + L.qs + at) = qh;
    *reinterpret_cast<bf16x8*>(ws + L.dos + at) = dd[c];
  }
  if (part == 0) {
    float* rs = reinterpret_cast<float*>(ws + L.rs) + size_t(b) * 64;
    rs[j] = valid ? -p.lse[size_t(h) * p.tq + tok] * kLog2e : 0.0f;
    rs[32 + j] = valid ? -dsum : 0.0f;
  }
}

// One workgroup per (32-key tile kt, KV head), image b = kt * hk + kvh.
template <int D>
__global__ void __launch_bounds__(PREP_THREADS) bwd_prep_k_kernel(BwdParams p, BwdLayout L) {
  constexpr int PC = D / 64, IMG = BGeo<D>::IMG;
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int b = blockIdx.x, kt = b / p.hk, kvh = b % p.hk;
  const int t = threadIdx.x, j = t >> 3, part = t & 7;
  const int key = kt * TT + j;
  const bool valid = key < p.tk;
  const size_t row = (size_t(key) * p.hk + kvh) * D + part * 8 * PC;
  bf16x8 k[PC] = {}, v[PC] = {};
  if (valid) {
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      k[c] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.k) + row + 8 * c);
      v[c] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.v) + row + 8 * c);
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < PC; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += float(k[c][e]) * float(k[c][e]);
  ss = sum8(ss);
  const float rk = valid ? __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps) : 0.0f;
  const float fold = p.scale * kLog2e;
#pragma unroll
  for (int c = 0; c < PC; ++c) {
    bf16x8 kf;
#pragma unroll
    for (int e = 0; e < 8; ++e) kf[e] = (__bf16)(float(k[c][e]) * rk * p.k_gain[part * 8 * PC + 8 * c + e] * fold);
    const size_t at = size_t(b) * IMG + img_off(PC * part + c, j);
    *reinterpret_cast<bf16x8*>(ws + L.kh + at) = kf;
    *reinterpret_cast<bf16x8*>(ws + L.vr + at) = v[c];
  }
}

// Writes the wave-summed gain partial of every lane's D / 4 dims
// (16 db + 4 g + i) through LDS and the workgroup's sum to part[0 .. D - 1].
template <int D>
__device__ __forceinline__ void store_gain_partial(float (&gp)[D / 16][4], float (*red)[D], float* part, int wave,
                                                   int lane, int tid) {
  const int g = lane >> 4;
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = sum16(gp[db][i]);
      if ((lane & 15) == 0) red[wave][16 * db + 4 * g + i] = x;
    }
  __syncthreads();
  if (tid < D) {
    float x = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) x += red[w][tid];
    part[tid] = x;
  }
}

// RMSNorm backward of one row held as D / 4 dims per lane (dims
// 16 db + 4 g + i, four lanes per row): x the input row, dxh the gradient of
// x_hat = rms(x) g. Writes dx (bf16) when `store`, and adds u * dxh to gp.
template <int D>
__device__ __forceinline__ void rms_backward_row(const __bf16* xrow, __bf16* dxrow, const float (&dxh)[D / 16][4],
                                                 const float* gain, float eps, bool store, float (&gp)[D / 16][4],
                                                 int g) {
  constexpr int NDB = D / 16;
  bf16x4 xv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    xv[db] = store ? *reinterpret_cast<const bf16x4*>(xrow + 16 * db + 4 * g) : bf16x4{};
  float ss = 0.0f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) ss += float(xv[db][i]) * float(xv[db][i]);
  ss = sum_groups(ss);
  const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
  float m = 0.0f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) m += float(xv[db][i]) * r * gain[16 * db + 4 * g + i] * dxh[db][i];
  m = sum_groups(m) * (1.0f / D);
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    bf16x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = float(xv[db][i]) * r;
      w[i] = (__bf16)((gain[16 * db + 4 * g + i] * dxh[db][i] - u * m) * r);
      gp[db][i] += store ? u * dxh[db][i] : 0.0f;
    }
    if (store) *reinterpret_cast<bf16x4*>(dxrow + 16 * db + 4 * g) = w;
  }
}

// ------------------------------------------------------------------ dq

template <int D>
struct DqLds {
  unsigned char kh[RING][BGeo<D>::IMG];
  unsigned char vr[RING][BGeo<D>::IMG];
  float gq[D];
  float red[8][D];
};

template <int D>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_kernel(BwdParams p, BwdLayout L, const int4* __restrict__ items, const int* __restrict__ tiles,
              const unsigned* __restrict__ soffs_all) {
  using G = BGeo<D>;
  constexpr int IMG = G::IMG, NKS = G::NKS, NDB = G::NDB;
  __shared__ __attribute__((aligned(1024))) DqLds<D> sm;
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  float* part = reinterpret_cast<float*>(ws + L.pgq) + size_t(blockIdx.x) * D;
  const int4 item = items[2 * blockIdx.x];
  if (item.z == item.w) {                              // padding item: an empty partial
    if (tid < D) part[tid] = 0.0f;
    return;
  }
  const int n_full = items[2 * blockIdx.x + 1].x;
  const int kvh = item.y >> 16, h0 = item.y & 0xffff;
  const int n = item.w - item.z;
  // The wave's 32 rows are one (token tile, head) image.
  const int r0 = wave * 32;
  const int head = h0 + r0 / p.tile_q;
  const int tok0 = item.x + r0 % p.tile_q;
  const int img = (tok0 / TT) * p.hq + head;
  // A wave whose rows all lie past T_q (the last query tile) has no image:
  // it computes with zeros (P = 1, dP = 0, dS = 0) and stores nothing.
  const bool live = tok0 < p.tq;

  bf16x8 qs[2][NKS], dov[2][NKS];
  {
    const size_t base = size_t(live ? img : 0) * IMG + img_off(g, r16);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        qs[rb][ks] = live ? *reinterpret_cast<const bf16x8*>(ws + L.qs + base + 2048 * ks + 256 * rb) : bf16x8{};
        dov[rb][ks] = live ? *reinterpret_cast<const bf16x8*>(ws + L.dos + base + 2048 * ks + 256 * rb) : bf16x8{};
      }
  }
  float nl2[2], nd[2];                               // -lse log2 e and -D of the lane's rows
  int lo[2], hi[2];
  {
    const float* rs = reinterpret_cast<const float*>(ws + L.rs) + size_t(live ? img : 0) * 64;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      nl2[rb] = live ? rs[16 * rb + r16] : 0.0f;
      nd[rb] = live ? rs[32 + 16 * rb + r16] : 0.0f;
      const int tok = tok0 + 16 * rb + r16;
      const int2 bnd = tok < p.tq ? p.rows[tok] : int2{0, 0};
      lo[rb] = bnd.x;
      hi[rb] = bnd.y;
    }
  }
  if (tid < D) sm.gq[tid] = p.q_gain[tid];

  const unsigned n_kt = unsigned(p.tk + TT - 1) / TT;
  const unsigned kbytes = n_kt * unsigned(p.hk) * IMG;
  const i32x4 rkh = make_rsrc(ws + L.kh, kbytes), rvr = make_rsrc(ws + L.vr, kbytes);
  const unsigned voff = unsigned(kvh) * IMG + unsigned(tid % G::COPY_THREADS) * 16;
  const unsigned kh0 = lds_addr(sm.kh[0]), vr0 = lds_addr(sm.vr[0]);
  // this wave's part of every image copy (split copies: waves 0-3 copy k', 4-7 V)
  const unsigned wpart = unsigned(G::SPLIT_COPY ? (wave & 3) : wave) * 1024;
  const bool kwave = wave < 4;
  const i32x4 rown = kwave ? rkh : rvr;
  const unsigned own0 = kwave ? kh0 : vr0;
  const int* codes = tiles + item.z;
  const unsigned* soffs = soffs_all + item.z;    // padded past the list with kNoTile
  auto issue_at = [&](int i, unsigned so) {
    const unsigned st = unsigned(i % RING) * IMG + wpart;
    if constexpr (G::SPLIT_COPY) {
      dma16(rown, voff, so, own0 + st);
    } else {
      dma16(rkh, voff, so, kh0 + st);
      dma16(rvr, voff, so, vr0 + st);
    }
  };
  for (int i = 0; i < 4; ++i) issue_at(i, __builtin_amdgcn_readfirstlane(soffs[i]));

  f32x4 acc[2][NDB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x4{};
  const unsigned rowq = img_off(g, r16), trq = tr_lane_offset(lane);  // chunk g + 4 ks has g's parity
  // copies per tile and wave: 2, or 1 when split; tiles i, i + 1 must have
  // landed, the copies of i + 2, i + 3 may still fly
  constexpr int kYounger = G::SPLIT_COPY ? 2 : 4;
  for (int i = 0; i < n; ++i) {
    if ((i & 1) == 0) {
      wait_vmcnt<kYounger>();
      lds_barrier();                                  // and every wave left the stages of tiles i - 4, i - 3
      // both offsets read before either copy, so that they come in one scalar load
      const unsigned so4 = __builtin_amdgcn_readfirstlane(soffs[i + 4]);
      const unsigned so5 = __builtin_amdgcn_readfirstlane(soffs[i + 5]);
      issue_at(i + 4, so4);
      issue_at(i + 5, so5);
    }
    const unsigned st = unsigned(i % RING) * IMG;
    // The S^T and dP^T chains start from -lse log2 e and -D (the lane's row
    // is the same for its four elements), so they end as S - lse log2 e and
    // dP - D.
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      s[rb][0] = s[rb][1] = f32x4{nl2[rb], nl2[rb], nl2[rb], nl2[rb]};
      dp[rb][0] = dp[rb][1] = f32x4{nd[rb], nd[rb], nd[rb], nd[rb]};
    }
#pragma unroll
    for (int f = 0; f < 2 * NKS; ++f) {
      const int ks = f >> 1, kb = f & 1;
      const bf16x8 a = *(lds_bf16x8*)(size_t)(kh0 + st + rowq + 2048 * ks + 256 * kb);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) s[rb][kb] = mfma(a, qs[rb][ks], s[rb][kb]);
    }
    // lane: row r16 of block rb, keys 16 kb + 4 g + i of the tile
    const bool masked = i >= n_full;
    const int kt = masked ? (codes[i] >> 1) : 0;
    if (masked) {                                     // keys outside the row's range: S = -inf, P = 0
      asm volatile("" ::: "memory");                  // a branch, not selects on every step
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const unsigned base = unsigned(kt * TT + 4 * g - lo[rb]), len = unsigned(hi[rb] - lo[rb]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[rb][kb][e] = base + unsigned(16 * kb + e) < len ? s[rb][kb][e] : -__builtin_inff();
      }
    }
    // dP on the matrix cores with P = 2^S (in place of S) on the vector ALUs
    // between its MFMAs: the exponentials do not wait for dP
#pragma unroll
    for (int f = 0; f < 2 * NKS; ++f) {
      const int ks = f >> 1, kb = f & 1;
      const bf16x8 a = *(lds_bf16x8*)(size_t)(vr0 + st + rowq + 2048 * ks + 256 * kb);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) dp[rb][kb] = mfma(a, dov[rb][ks], dp[rb][kb]);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[rb][kb][e] = __builtin_amdgcn_exp2f(s[rb][kb][e]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int f = 0; f < 2 * NKS; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (f < 2 * NKS - 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 ds[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[rb][4 * kb + e] = (__bf16)(s[rb][kb][e] * dp[rb][kb][e]);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16x8 a = tr_frag(kh0 + st + trq, db);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) acc[rb][db] = mfma(a, ds[rb], acc[rb][db]);
    }
  }
  wait_vmcnt<0>();                                    // the padding copies of the last two steps

  // A piece of a split item writes its fp32 dq-hat^T sums (times log2 e) to
  // its slot, [256 item rows][D dims], and an empty gain partial; the dq
  // merge adds the pieces and finishes the rows.
  const int slot = __builtin_amdgcn_readfirstlane(items[2 * blockIdx.x + 1].y);
  if (slot >= 0) {
    float* pd = reinterpret_cast<float*>(ws + L.pdq) + size_t(slot) * kBwdRowsPerItem * D;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(pd + size_t(r0 + 16 * rb + r16) * D + 16 * db + 4 * g) = acc[rb][db];
    if (tid < D) part[tid] = 0.0f;
    return;
  }

  // Epilogue: lane holds dims 16 db + 4 g + i of row r16 of block rb.
  float gp[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) gp[db][e] = 0.0f;
  __syncthreads();                                    // gains in LDS (and the loop's last reads) done
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int tok = tok0 + 16 * rb + r16;
    const bool valid = tok < p.tq;
    float dxh[NDB][4];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) dxh[db][e] = acc[rb][db][e] * (1.0f / kLog2e);
    const size_t off = (size_t(valid ? tok : 0) * p.hq + head) * D;
    rms_backward_row<D>(static_cast<const __bf16*>(p.q) + off, static_cast<__bf16*>(p.dq) + off, dxh, sm.gq, p.eps,
                        valid, gp, g);
  }
  store_gain_partial<D>(gp, sm.red, part, wave, lane, tid);
}

// ------------------------------------------------------------------ dk / dv

template <int D>
struct KvLds {
  unsigned char qs[RING][BGeo<D>::IMG];
  unsigned char dos[RING][BGeo<D>::IMG];
  float rs[RING][8][64];  // per stage and wave: -lse log2 e [32], -D [32] of the step's rows
  float gk[D];
  float red[8][D];
};

// 8 waves x 32 keys: wave w holds keys 32 w + 16 j + (0..15), j = 0, 1, of
// the item's 256, which are rows 16 j + (0..15) of one 32-key image. Every
// LDS fragment of a step feeds the MFMAs of both 16-key halves.
template <int D>
__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dkdv_kernel(BwdParams p, BwdLayout L, const int4* __restrict__ items, const int* __restrict__ tiles) {
  using G = BGeo<D>;
  constexpr int IMG = G::IMG, NKS = G::NKS, NDB = G::NDB;
  __shared__ __attribute__((aligned(1024))) KvLds<D> sm;
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  float* part = reinterpret_cast<float*>(ws + L.pgk) + size_t(blockIdx.x) * D;
  const int4 item = items[2 * blockIdx.x];
  if (item.z == item.w) {
    if (tid < D) part[tid] = 0.0f;
    return;
  }
  const int n_full = items[2 * blockIdx.x + 1].x;
  const int kb = item.x, kvh = item.y;
  const int grp = p.hq / p.hk;
  const int n_entries = item.w - item.z;
  const int n_steps = n_entries * grp;
  // The lane's keys (B operand columns, output rows), one per half.
  const int kt = kb * (kBwdKeysPerItem / TT) + wave;
  const int key0 = kt * TT + r16;
  const unsigned n_kt = unsigned(p.tk + TT - 1) / TT;
  bf16x8 ku[2][NKS], vv[2][NKS];
  {
    const bool have = unsigned(kt) < n_kt;
    const size_t base = (size_t(have ? kt : 0) * p.hk + kvh) * IMG;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const size_t at = base + img_off(g, 16 * j + r16) + 2048 * ks;
        ku[j][ks] = have ? *reinterpret_cast<const bf16x8*>(ws + L.kh + at) : bf16x8{};
        vv[j][ks] = have ? *reinterpret_cast<const bf16x8*>(ws + L.vr + at) : bf16x8{};
      }
  }
  int4 kbnd[2];                                       // token ranges that see each key
#pragma unroll
  for (int j = 0; j < 2; ++j) kbnd[j] = key0 + 16 * j < p.tk ? p.key_rows[key0 + 16 * j] : int4{0, 0, 0, 0};
  if (tid < D) sm.gk[tid] = p.k_gain[tid];

  const unsigned n_tt = unsigned(p.tq + TT - 1) / TT;
  const unsigned qbytes = n_tt * unsigned(p.hq) * IMG;
  const i32x4 rqs = make_rsrc(ws + L.qs, qbytes), rdo = make_rsrc(ws + L.dos, qbytes),
              rrs = make_rsrc(ws + L.rs, n_tt * unsigned(p.hq) * 256u);
  const unsigned qs0 = lds_addr(sm.qs[0]), do0 = lds_addr(sm.dos[0]), rs0 = lds_addr(&sm.rs[0][wave][0]);
  const int* codes = tiles + item.z;
  const int hbase = kvh * grp;
  // Step s = (entry s / grp, head hbase + s % grp); its image (token tile, head).
  int ie = 0, ih = 0;                                 // entry and head of the next step to issue
  // this wave's part of every image copy (split copies: waves 0-3 copy q_hat, 4-7 dO)
  const unsigned wpart = unsigned(G::SPLIT_COPY ? (wave & 3) : wave) * 1024;
  const bool qwave = wave < 4;
  const i32x4 rown = qwave ? rqs : rdo;
  const unsigned own0 = qwave ? qs0 : do0;
  const unsigned voff = unsigned(tid % G::COPY_THREADS) * 16;
  int icode = __builtin_amdgcn_readfirstlane(codes[0]);   // code of entry ie, read once per entry
  auto issue = [&]() {
    const bool live = ie < n_entries;
    const unsigned imgi = __builtin_amdgcn_readfirstlane(live ? unsigned((icode >> 1) * p.hq + hbase + ih) : 0u);
    const unsigned so = live ? imgi * IMG : kNoTile;
    const unsigned st = unsigned(((ie * grp + ih) % RING)) * IMG + wpart;
    if constexpr (G::SPLIT_COPY) {
      dma16(rown, voff, so, own0 + st);
    } else {
      dma16(rqs, voff, so, qs0 + st);
      dma16(rdo, voff, so, do0 + st);
    }
    if (lane < 16)
      dma16(rrs, unsigned(lane) * 16, live ? imgi * 256u : kNoTile,
            rs0 + unsigned((ie * grp + ih) % RING) * 8 * 256);
    if (++ih == grp) {
      ih = 0;
      ++ie;
      icode = __builtin_amdgcn_readfirstlane(codes[ie]);   // the list is padded past its end
    }
  };
  for (int i = 0; i < 4; ++i) issue();

  f32x4 accv[2][NDB], acck[2][NDB];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int db = 0; db < NDB; ++db) accv[j][db] = acck[j][db] = f32x4{};
  const unsigned rowq = img_off(g, r16), trq = tr_lane_offset(lane);  // chunk g + 4 ks has g's parity
  // copies per step and wave: q_hat, dO and the row statistics (3), or one
  // image and the statistics (2) when split; steps s, s + 1 must have landed,
  // the copies of s + 2, s + 3 may still fly
  constexpr int kYounger = G::SPLIT_COPY ? 4 : 6;
  int ce = 0, ch = 0;                                 // entry and head of the current step
  for (int s = 0; s < n_steps; ++s) {
    if ((s & 1) == 0) {
      wait_vmcnt<kYounger>();
      lds_barrier();
      issue();
      issue();
    }
    const unsigned st = unsigned(s % RING) * IMG;
    const unsigned rsa = rs0 + unsigned(s % RING) * 8 * 256;
    const bool masked = ce >= n_full;
    // S (lane: key r16 of half j, rows 16 rb + 4 g + e of the step's token
    // tile), started from the rows' -lse log2 e so that it ends as S - lse log2 e
    f32x4 sc[2][2], dp[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      sc[0][rb] = sc[1][rb] = *(lds_f32x4*)(size_t)(rsa + 4 * (16 * rb + 4 * g));
      dp[0][rb] = dp[1][rb] = *(lds_f32x4*)(size_t)(rsa + 128 + 4 * (16 * rb + 4 * g));
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 a = *(lds_bf16x8*)(size_t)(qs0 + st + rowq + 2048 * ks + 256 * rb);
        sc[0][rb] = mfma(a, ku[0][ks], sc[0][rb]);
        sc[1][rb] = mfma(a, ku[1][ks], sc[1][rb]);
      }
    if (masked) {                                     // rows that do not see the key: S = -inf, P = 0
      asm volatile("" ::: "memory");                  // a branch, not selects on every step
      const int tt = codes[ce] >> 1;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = tt * TT + 16 * rb + 4 * g + e;
            if (unsigned(tok - kbnd[j].x) >= unsigned(kbnd[j].y - kbnd[j].x) &&
                unsigned(tok - kbnd[j].z) >= unsigned(kbnd[j].w - kbnd[j].z))
              sc[j][rb][e] = -__builtin_inff();
          }
    }
    // dP, started from -D so that it ends as dP - D, on the matrix cores with
    // P = 2^S (in place of S) on the vector ALUs between its MFMAs
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 a = *(lds_bf16x8*)(size_t)(do0 + st + rowq + 2048 * ks + 256 * rb);
        dp[0][rb] = mfma(a, vv[0][ks], dp[0][rb]);
        dp[1][rb] = mfma(a, vv[1][ks], dp[1][rb]);
      }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[j][rb][e] = __builtin_amdgcn_exp2f(sc[j][rb][e]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int f = 0; f < 2 * NKS; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (f < 2 * NKS - 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // P and dS = P (dP - D) in bf16, then dV^T += dO^T P and dK^T += q_hat^T dS,
    // one transposed fragment of each image per dim block
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = sc[j][rb][e];
          pb[j][4 * rb + e] = (__bf16)pv;
          dsb[j][4 * rb + e] = (__bf16)(pv * dp[j][rb][e]);
        }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16x8 a = tr_frag(do0 + st + trq, db);
      const bf16x8 b = tr_frag(qs0 + st + trq, db);
      accv[0][db] = mfma(a, pb[0], accv[0][db]);
      accv[1][db] = mfma(a, pb[1], accv[1][db]);
      acck[0][db] = mfma(b, dsb[0], acck[0][db]);
      acck[1][db] = mfma(b, dsb[1], acck[1][db]);
    }
    // transposed reads (two per fragment) one dim block ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      if (db < NDB - 1) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    if (++ch == grp) { ch = 0; ++ce; }
  }
  wait_vmcnt<0>();

  // Epilogue: lane holds dims 16 db + 4 g + e of key key0 + 16 j. A piece of
  // a split list (slot >= 0) writes its fp32 sums of dV and of dK-hat / scale
  // to the slot ([2][256 keys][D dims]) and a zero gain partial; the merge
  // adds the pieces and finishes.
  const int slot = __builtin_amdgcn_readfirstlane(items[2 * blockIdx.x + 1].y);
  float* pk = reinterpret_cast<float*>(ws + L.pkv) + size_t(slot < 0 ? 0 : slot) * 2 * kBwdKeysPerItem * D;
  float gp[NDB][4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) gp[db][e] = 0.0f;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (slot >= 0) {
      const int kl = 32 * wave + 16 * j + r16;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        *reinterpret_cast<f32x4*>(pk + size_t(kl) * D + 16 * db + 4 * g) = accv[j][db];
        *reinterpret_cast<f32x4*>(pk + size_t(kBwdKeysPerItem + kl) * D + 16 * db + 4 * g) = acck[j][db];
      }
      continue;
    }
    const int key = key0 + 16 * j;
    const bool valid = key < p.tk;
    const size_t off = (size_t(valid ? key : 0) * p.hk + kvh) * D;
    if (valid) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)accv[j][db][e];
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.dv) + off + 16 * db + 4 * g) = w;
      }
    }
    float dxh[NDB][4];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) dxh[db][e] = p.scale * acck[j][db][e];
    rms_backward_row<D>(static_cast<const __bf16*>(p.k) + off, static_cast<__bf16*>(p.dk) + off, dxh, sm.gk, p.eps,
                        valid, gp, g);
  }
  store_gain_partial<D>(gp, sm.red, part, wave, lane, tid);
}

// Sums the per-workgroup gain partials in a fixed order, in two levels:
// workgroup b of REDUCE_SLICES (for dq, then as many for dk) sums the
// partial rows [n b / S, n (b + 1) / S) into level[b]; the final pass sums
// the S level rows. Threads: 256 / D lanes of each of the D dims, whose
// strided sums add up in lane order.
constexpr int REDUCE_SLICES = 256;
template <int D>
__global__ void __launch_bounds__(256) bwd_gain_slices_kernel(const float* pgq, int nq, const float* pgk, int nk,
                                                             float* level) {
  constexpr int H = 256 / D;
  const bool kside = blockIdx.x >= REDUCE_SLICES;
  const int b = kside ? blockIdx.x - REDUCE_SLICES : blockIdx.x;
  const float* src = kside ? pgk : pgq;
  const int n = kside ? nk : nq;
  const int i0 = int(int64_t(n) * b / REDUCE_SLICES), i1 = int(int64_t(n) * (b + 1) / REDUCE_SLICES);
  __shared__ float lanes[H][D];
  const int t = threadIdx.x, d = t % D, h = t / D;
  float x = 0.0f;
  for (int i = i0 + h; i < i1; i += H) x += src[size_t(i) * D + d];
  if (h > 0) lanes[h][d] = x;
  __syncthreads();
  if (h == 0) {
#pragma unroll
    for (int k = 1; k < H; ++k) x += lanes[k][d];
    level[size_t(blockIdx.x) * D + d] = x;
  }
}

template <int D>
__global__ void __launch_bounds__(256) bwd_gain_final_kernel(const float* level, float* dq_gain, float* dk_gain) {
  const int t = threadIdx.x, d = t % D, side = t / D;
  if (side > 1) return;
  float x = 0.0f;
  for (int b = 0; b < REDUCE_SLICES; ++b) x += level[size_t(side * REDUCE_SLICES + b) * D + d];
  (side ? dk_gain : dq_gain)[d] = x;
}

// Finishes a split dk/dv item: sums its pieces' slots in piece order, writes
// dV, applies the RMSNorm backward to dK-hat = scale * sum and writes dK and
// the workgroup's gain partial (row n_kv_items + merge index). Thread t
// handles dims [D / 4 (t % 4), +D / 4) of keys t / 4 + 64 i, i = 0..3.
constexpr int MERGE_THREADS = 256;
template <int D>
__global__ void __launch_bounds__(MERGE_THREADS) bwd_kv_merge_kernel(BwdParams p, BwdLayout L,
                                                                     const int4* __restrict__ merges) {
  constexpr int DPT = D / 4;                          // dims per thread
  __shared__ float gk[D];
  __shared__ float red[64][D + 1];
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int4 m = merges[blockIdx.x];                  // key block, KV head, first slot, pieces
  const int t = threadIdx.x, quarter = t & 3, kq = t >> 2;
  if (t < D) gk[t] = p.k_gain[t];
  __syncthreads();
  float gp[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) gp[i] = 0.0f;
  const float* slots = reinterpret_cast<const float*>(ws + L.pkv);
  for (int pass = 0; pass < kBwdKeysPerItem / 64; ++pass) {
    const int kl = 64 * pass + kq;
    const int key = m.x * kBwdKeysPerItem + kl;
    const bool valid = key < p.tk;
    float sv[DPT], sk[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) sv[i] = sk[i] = 0.0f;
    for (int k = 0; k < m.w; ++k) {
      const float* s = slots + size_t(m.z + k) * 2 * kBwdKeysPerItem * D + size_t(kl) * D + DPT * quarter;
#pragma unroll
      for (int c = 0; c < DPT / 4; ++c) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(s + 4 * c);
        const f32x4 b = *reinterpret_cast<const f32x4*>(s + size_t(kBwdKeysPerItem) * D + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[4 * c + e] += a[e];
          sk[4 * c + e] += b[e];
        }
      }
    }
    const size_t off = (size_t(valid ? key : 0) * p.hk + m.y) * D + DPT * quarter;
    float x[DPT];
#pragma unroll
    for (int c = 0; c < DPT / 8; ++c) {
      const bf16x8 xv = valid ? *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.k) + off + 8 * c)
                              : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * c + e] = float(xv[e]);
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < DPT; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    const float r = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
    float mm = 0.0f;
#pragma unroll
    for (int i = 0; i < DPT; ++i) mm += x[i] * r * gk[DPT * quarter + i] * (p.scale * sk[i]);
    mm += __shfl_xor(mm, 1, 64);
    mm += __shfl_xor(mm, 2, 64);
    mm *= 1.0f / D;
    if (valid) {
#pragma unroll
      for (int c = 0; c < DPT / 8; ++c) {
        bf16x8 wv, wk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * c + e;
          const float dxh = p.scale * sk[i], u = x[i] * r;
          wv[e] = (__bf16)sv[i];
          wk[e] = (__bf16)((gk[DPT * quarter + i] * dxh - u * mm) * r);
          gp[i] += u * dxh;
        }
        *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.dv) + off + 8 * c) = wv;
        *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.dk) + off + 8 * c) = wk;
      }
    }
  }
  // gain partial: sum over the 64 keys of each quarter
#pragma unroll
  for (int i = 0; i < DPT; ++i) red[kq][DPT * quarter + i] = gp[i];
  __syncthreads();
  if (t < D) {
    float s = 0.0f;
    for (int k = 0; k < 64; ++k) s += red[k][t];
    reinterpret_cast<float*>(ws + L.pgk)[size_t(p.n_kv_items + blockIdx.x) * D + t] = s;
  }
}

// Finishes a split dq item: sums its pieces' slots in piece order
// (dq-hat = sum / log2 e), applies the RMSNorm backward, writes dq and the
// workgroup's gain partial (row n_dq_items + merge index). Item row r is token
// t0 + r % tile_q of head h0 + r / tile_q. Thread t handles dims
// [D / 4 (t % 4), +D / 4) of rows t / 4 + 64 i, i = 0..3.
template <int D>
__global__ void __launch_bounds__(MERGE_THREADS) bwd_dq_merge_kernel(BwdParams p, BwdLayout L,
                                                                     const int4* __restrict__ merges) {
  constexpr int DPT = D / 4;                          // dims per thread
  __shared__ float gq[D];
  __shared__ float red[64][D + 1];
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int4 m = merges[2 * blockIdx.x];              // t0, (kvh << 16) | h0, first slot, pieces
  const int h0 = m.y & 0xffff;
  const int t = threadIdx.x, quarter = t & 3, rq = t >> 2;
  if (t < D) gq[t] = p.q_gain[t];
  __syncthreads();
  float gp[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) gp[i] = 0.0f;
  const float* slots = reinterpret_cast<const float*>(ws + L.pdq);
  for (int pass = 0; pass < kBwdRowsPerItem / 64; ++pass) {
    const int r = 64 * pass + rq;
    const int tok = m.x + r % p.tile_q, head = h0 + r / p.tile_q;
    const bool valid = tok < p.tq;
    float sq[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) sq[i] = 0.0f;
    for (int k = 0; k < m.w; ++k) {
      const float* s = slots + (size_t(m.z + k) * kBwdRowsPerItem + r) * D + DPT * quarter;
#pragma unroll
      for (int c = 0; c < DPT / 4; ++c) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(s + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) sq[4 * c + e] += a[e];
      }
    }
    const size_t off = (size_t(valid ? tok : 0) * p.hq + head) * D + DPT * quarter;
    float x[DPT];
#pragma unroll
    for (int c = 0; c < DPT / 8; ++c) {
      const bf16x8 xv = valid ? *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.q) + off + 8 * c)
                              : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * c + e] = float(xv[e]);
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < DPT; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    const float rr = __builtin_amdgcn_rsqf(ss * (1.0f / D) + p.eps);
    float mm = 0.0f;
#pragma unroll
    for (int i = 0; i < DPT; ++i) mm += x[i] * rr * gq[DPT * quarter + i] * (sq[i] * (1.0f / kLog2e));
    mm += __shfl_xor(mm, 1, 64);
    mm += __shfl_xor(mm, 2, 64);
    mm *= 1.0f / D;
    if (valid) {
#pragma unroll
      for (int c = 0; c < DPT / 8; ++c) {
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * c + e;
          const float dxh = sq[i] * (1.0f / kLog2e), u = x[i] * rr;
          w[e] = (__bf16)((gq[DPT * quarter + i] * dxh - u * mm) * rr);
          gp[i] += u * dxh;
        }
        *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.dq) + off + 8 * c) = w;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < DPT; ++i) red[rq][DPT * quarter + i] = gp[i];
  __syncthreads();
  if (t < D) {
    float s = 0.0f;
    for (int k = 0; k < 64; ++k) s += red[k][t];
    reinterpret_cast<float*>(ws + L.pgq)[size_t(p.n_dq_items + blockIdx.x) * D + t] = s;
  }
}

// dq = 0 over the blocks whose rows see no key (no dq item covers them): one
// workgroup per block of `rows` tokens x `heads` heads, 16-byte stores.
__global__ void __launch_bounds__(256) bwd_zero_rows_kernel(unsigned char* dq, const int2* __restrict__ blocks,
                                                           int rows, int heads, int tq, int hq, int row_bytes) {
  const int2 blk = blocks[blockIdx.x];
  const int chunks = row_bytes / 16;
  const int n = rows * heads * chunks;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int c = i % chunks, hh = (i / chunks) % heads, r = i / (chunks * heads);
    const int tok = blk.x + r;
    if (tok < tq) *reinterpret_cast<int4*>(dq + (size_t(tok) * hq + blk.y + hh) * row_bytes + 16 * c) = int4{0, 0, 0, 0};
  }
}

}  // namespace

hipError_t launch_bwd_zero_rows(const BwdParams& p, int row_bytes, hipStream_t stream) {
  if (p.n_dq_zero > 0)
    hipLaunchKernelGGL(bwd_zero_rows_kernel, dim3(p.n_dq_zero), dim3(256), 0, stream, static_cast<unsigned char*>(p.dq),
                       p.dq_zero, p.tile_q, p.heads_per_item, p.tq, p.hq, row_bytes);
  if (p.n_kv_zero > 0) {
    hipLaunchKernelGGL(bwd_zero_rows_kernel, dim3(p.n_kv_zero), dim3(256), 0, stream, static_cast<unsigned char*>(p.dk),
                       p.kv_zero, p.key_block, p.hk, p.tk, p.hk, row_bytes);
    hipLaunchKernelGGL(bwd_zero_rows_kernel, dim3(p.n_kv_zero), dim3(256), 0, stream, static_cast<unsigned char*>(p.dv),
                       p.kv_zero, p.key_block, p.hk, p.tk, p.hk, row_bytes);
  }
  return hipGetLastError();
}

BwdLayout bwd_workspace_layout(long long tq, long long tk, int hq, int hk, int D, int n_dq_rows, int n_kv_rows,
                               int n_kv_slots, int n_dq_slots) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t IMG = size_t(TT) * D * 2;
  const size_t qimg = size_t((tq + TT - 1) / TT) * size_t(hq) * IMG;
  const size_t kimg = size_t((tk + TT - 1) / TT) * size_t(hk) * IMG;
  BwdLayout L{};
  L.qs = 0;
  L.dos = L.qs + up(qimg);
  L.rs = L.dos + up(qimg);
  L.kh = L.rs + up(qimg / IMG * 256);
  L.vr = L.kh + up(kimg);
  L.pgq = L.vr + up(kimg);
  L.pgk = L.pgq + up(size_t(n_dq_rows) * D * sizeof(float));
  L.pkv = L.pgk + up(size_t(n_kv_rows) * D * sizeof(float));
  L.pdq = L.pkv + up(size_t(n_kv_slots) * 2 * kBwdKeysPerItem * D * sizeof(float));
  L.level = L.pdq + up(size_t(n_dq_slots) * kBwdRowsPerItem * D * sizeof(float));
  L.total = L.level + up(size_t(2 * REDUCE_SLICES) * D * sizeof(float));
  return L;
}

namespace {

template <int D>
hipError_t launch_bwd_bf16_d(const BwdParams& p, hipStream_t stream) {
  const BwdLayout L = bwd_workspace_layout(p.tq, p.tk, p.hq, p.hk, D, p.n_dq_items + p.n_dq_merges,
                                           p.n_kv_items + p.n_kv_merges, p.n_kv_slots, p.n_dq_slots);
  const unsigned n_tt = unsigned((p.tq + TT - 1) / TT), n_kt = unsigned((p.tk + TT - 1) / TT);
  hipLaunchKernelGGL(bwd_prep_q_kernel<D>, dim3(n_tt * unsigned(p.hq)), dim3(PREP_THREADS), 0, stream, p, L);
  if (n_kt > 0)
    hipLaunchKernelGGL(bwd_prep_k_kernel<D>, dim3(n_kt * unsigned(p.hk)), dim3(PREP_THREADS), 0, stream, p, L);
  const hipError_t ez = launch_bwd_zero_rows(p, D * 2, stream);
  if (ez != hipSuccess) return ez;
  if (p.n_dq_items > 0)
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(p.n_dq_items), dim3(NTHR), 0, stream, p, L, p.dq_items, p.dq_tiles,
                       p.dq_soffs);
  if (p.n_kv_items > 0)
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(p.n_kv_items), dim3(NTHR), 0, stream, p, L, p.kv_items, p.kv_tiles);
  if (p.n_kv_merges > 0)
    hipLaunchKernelGGL(bwd_kv_merge_kernel<D>, dim3(p.n_kv_merges), dim3(MERGE_THREADS), 0, stream, p, L,
                       p.kv_merges);
  if (p.n_dq_merges > 0)
    hipLaunchKernelGGL(bwd_dq_merge_kernel<D>, dim3(p.n_dq_merges), dim3(MERGE_THREADS), 0, stream, p, L,
                       p.dq_merges);
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  float* level = reinterpret_cast<float*>(ws + L.level);
  hipLaunchKernelGGL(bwd_gain_slices_kernel<D>, dim3(2 * REDUCE_SLICES), dim3(256), 0, stream,
                     reinterpret_cast<const float*>(ws + L.pgq), p.n_dq_items + p.n_dq_merges,
                     reinterpret_cast<const float*>(ws + L.pgk), p.n_kv_items + p.n_kv_merges, level);
  hipLaunchKernelGGL(bwd_gain_final_kernel<D>, dim3(1), dim3(256), 0, stream, level, p.dq_gain, p.dk_gain);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_bwd_bf16_d<128>(p, stream);
  if (head_dim == 64) return launch_bwd_bf16_d<64>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace magi
