// Block-causal QK-RMSNorm GQA attention forward, bf16, head_dim 128, gfx950.
//
// What is computed follows the MAGI-1 pages (paperlayer §2 / Figure 1 and
// §2.2.2; paper-notes §3.2.2 block pseudocode and Figure 15): per query row,
// softmax over its allowed keys of scale * <rms(q) * g_q, rms(k) * g_k>,
// times V, plus the natural-log log-sum-exp. The forward's cost is the two
// matrix products over the mask area (paperlayer §B.2.1), so both run on the
// bf16 matrix cores.
//
// Workgroup = one work item: 256 (token, head) rows = 8 waves x 32 rows of
// `heads_per_item` query heads that share one KV head. Per key tile (64 keys):
//   * the K and V tiles are copied from global memory straight into LDS with
//     buffer_load ... lds (zero fill past T_k), three stages deep, and serve
//     all 256 rows: K/V are read from L2 once per workgroup, not per head;
//   * the K RMS factor r_j = 1/sqrt(mean(k_j^2) + eps) is computed once per
//     key by the workgroup; g_k is folded into the normalised queries, so the
//     raw bf16 keys feed the matrix cores and s_ij = r_j * <q'_i, k_j>;
//   * S^T = K Q'^T on v_mfma_f32_32x32x16_bf16 (lane = query row), softmax in
//     fp32 registers, P rounded to bf16, O^T += V^T P^T with V read through
//     ds_read_b64_tr_b16 from the row-major LDS tile.
// Queries are normalised in the prologue (RMS over head_dim, times g_q * g_k
// * scale * log2 e) and kept in registers as bf16 MFMA operands.
//
// Softmax. QK-normalisation bounds every logit: |s_ij| <= |q'_i| |k_hat_j|
// <= |q'_i| sqrt(d). When that bound is at most 40 (log2 units) for all rows
// of a wave, the wave uses exp2(s) directly (no running maximum, no rescale):
// softmax is invariant to the shift and 2^+-40 is far inside fp32/bf16 range.
// Otherwise the wave runs the online softmax with a running row maximum.
#include "kernels.hpp"

namespace magi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int D = 128;
constexpr int BN = 64;
constexpr int NWAVE = 8;
constexpr int NTHR = NWAVE * 64;
constexpr int NSTAGE = 3;
constexpr int ROW_BYTES = D * 2;                       // 256
constexpr int TILE_BYTES = BN * ROW_BYTES;             // 16 KiB
constexpr int UNITS_PER_THREAD = TILE_BYTES / (NTHR * 16);  // 2
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kStaticBound = 40.0f;
constexpr float kNegInf = -__builtin_inff();

struct Smem {
  unsigned char k[NSTAGE][TILE_BYTES];
  unsigned char v[NSTAGE][TILE_BYTES];
  float rk[2][BN];
  float gqk[D];
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float sumsq8(bf16x8 a, float acc) {
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    bf16x2 p = {a[j], a[j + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
  }
  return acc;
}

// Walks the key tiles of a work item's segment list, one tile per step.
struct TileCursor {
  const int4* segs;
  int seg, seg_end;
  int kt, kt_end, masked;
  __device__ void init(const int4* s, int b, int e) {
    segs = s; seg = b; seg_end = e;
    load();
  }
  __device__ void load() {
    if (seg < seg_end) {
      const int4 g = segs[seg];
      kt = g.x; kt_end = g.y; masked = g.z;
    }
  }
  __device__ void next() {
    if (++kt == kt_end) { ++seg; load(); }
  }
};

// Copies key tile kt of KV head kvh into LDS stage buffers. LDS images:
//   K: row-major [key][128], 16-byte chunk c of key j stored at chunk c ^ (j & 15)
//   V: row-major [key][128], 64-byte segment g of key j stored at g ^ (j & 3)
// Each wave instruction writes 1 KiB of LDS (lane i -> +16 i); the lane's
// global source is chosen so the image comes out swizzled.
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, Smem& sm, int stage,
                                           int kt, int kvh, int hk, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < UNITS_PER_THREAD; ++i) {
    const int blk = i * NWAVE + wave;                  // 1 KiB block of the image
    const int u = blk * 64 + lane;                     // 16-byte unit
    const int key = u >> 4, pc = u & 15;
    const unsigned row = unsigned((kt * BN + key) * hk + kvh) * ROW_BYTES;
    const int ck = pc ^ (key & 15);
    const int cv = ((((pc >> 2) ^ (key & 3)) << 2) | (pc & 3));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, LDS_PTR(void, sm.k[stage] + blk * 1024), 16, row + ck * 16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, LDS_PTR(void, sm.v[stage] + blk * 1024), 16, row + cv * 16, 0, 0, 0);
  }
}

// r_j = 1 / sqrt(mean_d k_j^2 + eps) for the 64 keys of a staged K tile.
__device__ __forceinline__ void key_rms(Smem& sm, int stage, int rs, float eps) {
  const int tid = threadIdx.x;
  const int key = tid >> 3, part = tid & 7;
  const unsigned char* row = sm.k[stage] + key * ROW_BYTES;
  const bf16x8 a0 = *LDS_PTR(const bf16x8, row + (((2 * part) ^ (key & 15)) * 16));
  const bf16x8 a1 = *LDS_PTR(const bf16x8, row + (((2 * part + 1) ^ (key & 15)) * 16));
  float ss = sumsq8(a1, sumsq8(a0, 0.0f));
  ss += dpp<0xB1>(ss);    // quad_perm [1,0,3,2]
  ss += dpp<0x4E>(ss);    // quad_perm [2,3,0,1]
  ss += dpp<0x141>(ss);   // row_half_mirror: the other quad of 8 lanes
  if (part == 0) sm.rk[rs][key] = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
}

struct WaveState {
  bf16x8 qf[8];          // B operand of S^T: lane row (l & 31), dims (2ks + (l>>5)) * 8 ..
  f32x16 o[4];           // O^T accumulator: lane row (l & 31), 4 dim blocks of 32
  float lsum;            // partial row sum over this lane's half of the keys
  float m;               // running max (online path), log2 units
  int lo, hi;            // key bounds of the lane's row
  bool stat;             // wave-uniform: static-bound softmax
};

__device__ __forceinline__ void compute_tile(const Smem& sm, int stage, int rs, int kt, bool masked, WaveState& st,
                                             int lane) {
  const int l31 = lane & 31, hi5 = lane >> 5;
  const unsigned char* kb_base = sm.k[stage];
  // ---- S^T[key][row] for two 32-key blocks
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 acc = {};
    const unsigned char* row = kb_base + (kb * 32 + l31) * ROW_BYTES;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = (2 * ks + hi5) ^ (lane & 15);
      const bf16x8 a = *LDS_PTR(const bf16x8, row + c * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.qf[ks], acc, 0, 0, 0);
    }
    s[kb] = acc;
  }
  // ---- scale by the key RMS factors, mask, exponentiate
  // lane holds keys kb*32 + (i/4)*8 + hi5*4 + (i%4), i = 0..15
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 r = *LDS_PTR(const f32x4, &sm.rk[rs][kb * 32 + u * 8 + hi5 * 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = s[kb][u * 4 + e] * r[e];
        if (masked) {
          const int key = kt * BN + kb * 32 + u * 8 + hi5 * 4 + e;
          x = (key >= st.lo && key < st.hi) ? x : kNegInf;
        }
        s[kb][u * 4 + e] = x;
      }
    }
  }
  if (!st.stat) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(st.m, mx);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);
    st.m = m_new;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] -= m_use;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
      st.lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) st.o[db] *= alpha;
    }
  }
  bf16x8 p[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) p[kb][t][j] = (__bf16)__builtin_amdgcn_exp2f(s[kb][t * 8 + j]);
  // row sum of the rounded probabilities (what P V actually weights)
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 pp = {p[kb][t][j], p[kb][t][j + 1]};
        st.lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, st.lsum, false);
      }
  // ---- O^T[dim][row] += V^T P^T
  // k-step (kb, t) covers keys kb*32 + t*16 + {s*8 + hi5*4 + r}: the P layout.
  // ds_read_b64_tr_b16: lane 16b+n receives, for r = 0..3, element n%4 of what
  // lane 16b + 4r + n/4 read; lane 16b+i therefore reads 4 dims of key
  // (.. + (b>>1)*4 + i/4) at dim (b&1)*16 + (i%4)*4 of the 32-dim block.
  const unsigned char* vb = sm.v[stage];
  const int b = lane >> 4, n = lane & 15;
  const int key_in = (b >> 1) * 4 + (n >> 2);
  const int dim_in = (b & 1) * 16 + (n & 3) * 4;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        i16x4 h[2];
#pragma unroll
        for (int sidx = 0; sidx < 2; ++sidx) {
          const int key = kb * 32 + t * 16 + sidx * 8 + key_in;
          const int off = key * ROW_BYTES + ((db ^ (key & 3)) * 64) + dim_in * 2;
          h[sidx] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vb + off));
        }
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, p[kb][t], st.o[db], 0, 0, 0);
      }
  }
}

__global__ void __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_bf16_d128_kernel(FwdParams prm) {
  __shared__ __attribute__((aligned(1024))) Smem sm;
  const int4 item = prm.items[blockIdx.x];
  if (item.z == item.w) return;                       // padding item
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int kvh = item.y >> 16, h0 = item.y & 0xffff;
  const int rb_per_head = prm.tile_q >> 5;
  const int head = h0 + wave / rb_per_head;
  const int t = item.x + (wave % rb_per_head) * 32 + (lane & 31);
  const bool valid = t < prm.tq;

  // gains product, folded with the temperature and log2 e
  if (tid < D) sm.gqk[tid] = prm.q_gain[tid] * prm.k_gain[tid] * (prm.scale * kLog2e);

  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(prm.k), (short)0, int(unsigned(prm.tk) * unsigned(prm.hk) * unsigned(ROW_BYTES)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(prm.v), (short)0, int(unsigned(prm.tk) * unsigned(prm.hk) * unsigned(ROW_BYTES)), 0x00020000);

  // tiles of this item
  int n_tiles = 0;
  for (int sg = item.z; sg < item.w; ++sg) { const int4 g = prm.segs[sg]; n_tiles += g.y - g.x; }
  TileCursor cur_load, cur_comp;
  cur_load.init(prm.segs, item.z, item.w);
  cur_comp = cur_load;
  // prefetch tiles 0 and 1
  issue_tile(rk, rv, sm, 0, cur_load.kt, kvh, prm.hk, wave, lane);
  cur_load.next();
  if (n_tiles > 1) { issue_tile(rk, rv, sm, 1, cur_load.kt, kvh, prm.hk, wave, lane); cur_load.next(); }

  // ---- query prologue: load, RMS-normalise, fold gains/temperature, to bf16
  WaveState st;
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(prm.q) + (size_t(t) * prm.hq + head) * D;
    bf16x8 qr[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (valid) qr[ks] = *reinterpret_cast<const bf16x8*>(qrow + (2 * ks + (lane >> 5)) * 8);
      else qr[ks] = bf16x8{};
    }
    float ss = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) ss = sumsq8(qr[ks], ss);
    ss += xor32(ss);
    const float rq = __builtin_amdgcn_rsqf(ss * (1.0f / D) + prm.eps);
    __syncthreads();                                   // gqk visible
    float nq = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int d0 = (2 * ks + (lane >> 5)) * 8;
      const f32x4 g0 = *LDS_PTR(const f32x4, &sm.gqk[d0]);
      const f32x4 g1 = *LDS_PTR(const f32x4, &sm.gqk[d0 + 4]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float g = j < 4 ? g0[j] : g1[j - 4];
        const float x = valid ? float(qr[ks][j]) * rq * g : 0.0f;
        st.qf[ks][j] = (__bf16)x;
      }
      nq = sumsq8(st.qf[ks], nq);
    }
    nq += xor32(nq);
    const float bound = __builtin_sqrtf(nq) * __builtin_sqrtf(float(D)) * 1.02f;
    st.stat = __builtin_amdgcn_ballot_w64(!(bound <= kStaticBound)) == 0;
    const int2 rb = valid ? prm.rows[t] : int2{0, 0};
    st.lo = rb.x;
    st.hi = rb.y;
#pragma unroll
    for (int db = 0; db < 4; ++db) st.o[db] = f32x16{};
    st.lsum = 0.0f;
    st.m = kNegInf;
  }

  // tile 0's K factors
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  key_rms(sm, 0, 0, prm.eps);

  for (int i = 0; i < n_tiles; ++i) {
    // tile i+1 landed (own loads), everyone done with tile i-1, r(i) published
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (i + 2 < n_tiles) {
      issue_tile(rk, rv, sm, (i + 2) % NSTAGE, cur_load.kt, kvh, prm.hk, wave, lane);
      cur_load.next();
    }
    if (i + 1 < n_tiles) key_rms(sm, (i + 1) % NSTAGE, (i + 1) & 1, prm.eps);
    compute_tile(sm, i % NSTAGE, i & 1, cur_comp.kt, cur_comp.masked != 0, st, lane);
    cur_comp.next();
  }

  // ---- epilogue
  const float lsum = st.lsum + xor32(st.lsum);
  if (valid) {
    const float inv = 1.0f / lsum;
    __bf16* orow = reinterpret_cast<__bf16*>(prm.out) + (size_t(t) * prm.hq + head) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(st.o[db][u * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + u * 8 + (lane >> 5) * 4) = w;
      }
    if (lane < 32) {
      const float l2 = __builtin_amdgcn_logf(lsum);   // log2
      const float lse = st.stat ? l2 * kLn2 : (st.m + l2) * kLn2;
      prm.lse[size_t(head) * prm.tq + t] = lse;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16_d128(const FwdParams& p, int n_items, hipStream_t stream) {
  hipLaunchKernelGGL(fwd_bf16_d128_kernel, dim3(n_items), dim3(NTHR), 0, stream, p);
  return hipGetLastError();
}

}  // namespace magi
