// Block-causal QK-RMSNorm GQA attention forward, fp32 (head_dim 64 or 128).
//
// Same operation as the bf16 kernel (MAGI-1 pages: paperlayer §2 / Figure 1,
// §2.2.2; paper-notes §3.2.2 and Figure 15), computed entirely in fp32 on the
// vector ALUs for callers that need fp32 accuracy. One wave per work item:
// 64 query tokens of one query head, one thread per query row. Key tiles of
// 32 keys are staged in LDS (shared by the 64 rows), normalised there once,
// and read back as broadcasts. Online softmax in exp2 units with a per-tile
// rescale. Work items of phase 1 (parallel plans) run the text
// cross-attention with the second set of tensors (paperlayer §2.2.2;
// paper-notes §3.2.2); rows that see no key get out = 0 and lse = -inf.
#include "kernels.hpp"

namespace magi {
namespace {

constexpr int BN = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

template <int D>
__global__ void __launch_bounds__(64) fwd_fp32_kernel(FwdParams prm) {
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  __shared__ float gk[D];
  const int4 item = prm.items[2 * blockIdx.x];
  if (item.z == item.w) return;
  const bool px = prm.items[2 * blockIdx.x + 1].z != 0;   // phase 1: the cross-attention of a parallel plan
  const int lane = threadIdx.x;
  const int kvh = item.y >> 16, head = item.y & 0xffff;
  const int t = item.x + lane;
  const bool valid = t < prm.tq;
  const float* qg = px ? prm.q_gain_x : prm.q_gain;
  const float* kgain = px ? prm.k_gain_x : prm.k_gain;
  const int tk = px ? prm.tkx : prm.tk;
  for (int d = lane; d < D; d += 64) gk[d] = kgain[d];

  float q[D];
  float o[D];
  {
    const float* qrow = reinterpret_cast<const float*>(px ? prm.qx : prm.q) + (size_t(t) * prm.hq + head) * D;
    float ss = 0.0f;
    for (int d = 0; d < D; ++d) {
      q[d] = valid ? qrow[d] : 0.0f;
      ss += q[d] * q[d];
    }
    const float rq = 1.0f / __builtin_sqrtf(ss / D + prm.eps);
    const float c = (px ? prm.scale_x : prm.scale) * kLog2e;
    for (int d = 0; d < D; ++d) {
      q[d] = valid ? q[d] * rq * qg[d] * c : 0.0f;
      o[d] = 0.0f;
    }
  }
  const int2 rb = valid ? prm.rows[(px ? prm.tq : 0) + t] : int2{0, 0};
  float m = kNegInf, l = 0.0f;
  const float* kbase = reinterpret_cast<const float*>(px ? prm.kx : prm.k);
  const float* vbase = reinterpret_cast<const float*>(px ? prm.vx : prm.v);

  for (int ti = item.z; ti < item.w; ++ti) {
    const int code = prm.tiles[ti];
    const int kt = code >> 1;
    const bool masked = (code & 1) != 0;
    {
      __syncthreads();
      // stage and normalise the key tile: 2 threads per key
      for (int e = lane; e < BN * D; e += 64) {
        const int j = e / D, d = e % D;
        const int key = kt * BN + j;
        const bool in = key < tk;
        const size_t off = (size_t(key) * prm.hk + kvh) * D + d;
        ks[j][d] = in ? kbase[off] : 0.0f;
        vs[j][d] = in ? vbase[off] : 0.0f;
      }
      __syncthreads();
      {
        const int j = lane >> 1, half = lane & 1;
        float ss = 0.0f;
        for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) ss += ks[j][d] * ks[j][d];
        ss += __shfl_xor(ss, 1, 64);
        const float r = 1.0f / __builtin_sqrtf(ss / D + prm.eps);
        __syncthreads();
        for (int d = half * (D / 2); d < (half + 1) * (D / 2); ++d) ks[j][d] = ks[j][d] * r * gk[d];
      }
      __syncthreads();
      float s[BN];
      float mx = kNegInf;
      for (int j = 0; j < BN; ++j) {
        float acc = 0.0f;
        for (int d = 0; d < D; ++d) acc += q[d] * ks[j][d];
        const int key = kt * BN + j;
        if (masked && !(key >= rb.x && key < rb.y)) acc = kNegInf;
        s[j] = acc;
        mx = fmaxf(mx, acc);
      }
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = __builtin_exp2f(m - m_use);
      l *= alpha;
      for (int d = 0; d < D; ++d) o[d] *= alpha;
      for (int j = 0; j < BN; ++j) {
        const float p = __builtin_exp2f(s[j] - m_use);
        l += p;
        for (int d = 0; d < D; ++d) o[d] += p * vs[j][d];
      }
      m = m_new;
    }
  }
  if (valid) {
    float* orow = reinterpret_cast<float*>(px ? prm.outx : prm.out) + (size_t(t) * prm.hq + head) * D;
    const bool any = l > 0.0f;                    // false only for a row that sees no key
    const float inv = any ? 1.0f / l : 0.0f;
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    (px ? prm.lsex : prm.lse)[size_t(head) * prm.tq + t] = any ? (m + __builtin_log2f(l)) * kLn2 : kNegInf;
  }
}

// Rows that see no key at all (merge entries without pieces: query tiles of
// chunks without text): out = 0, lse = -inf. One wave per entry, one thread
// per row of the entry's tile_q tokens x heads_per_item heads.
template <int D>
__global__ void __launch_bounds__(64) fp32_clear_kernel(FwdParams prm) {
  const int4 mi = prm.merges[2 * blockIdx.x];
  const bool px = prm.merges[2 * blockIdx.x + 1].x != 0;
  float* const obase = reinterpret_cast<float*>(px ? prm.outx : prm.out);
  float* const lbase = px ? prm.lsex : prm.lse;
  const int h0 = mi.y & 0xffff;
  for (int r = threadIdx.x; r < prm.tile_q * prm.heads_per_item; r += 64) {
    const int head = h0 + r / prm.tile_q, t = mi.x + r % prm.tile_q;
    if (t >= prm.tq) continue;
    float* orow = obase + (size_t(t) * prm.hq + head) * D;
    for (int d = 0; d < D; ++d) orow[d] = 0.0f;
    lbase[size_t(head) * prm.tq + t] = kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdParams& p, int head_dim, int n_items, int n_merges, hipStream_t stream) {
  if (n_items > 0) {
    if (head_dim == 64)
      hipLaunchKernelGGL(fwd_fp32_kernel<64>, dim3(n_items), dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(fwd_fp32_kernel<128>, dim3(n_items), dim3(64), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_merges == 0) return hipSuccess;
  if (head_dim == 64)
    hipLaunchKernelGGL(fp32_clear_kernel<64>, dim3(n_merges), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(fp32_clear_kernel<128>, dim3(n_merges), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace magi
