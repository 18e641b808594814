// Block-causal QK-RMSNorm GQA attention forward, fp32 (head_dim 64 or 128).
//
// Same operation as the bf16 kernel (MAGI-1 pages: paperlayer §2 / Figure 1,
// §2.2.2; paper-notes §3.2.2 and Figure 15), computed entirely in fp32 on the
// vector ALUs for callers that need fp32 accuracy. One wave per work item:
// 64 query tokens of one query head, one thread per query row. Key tiles of
// 32 keys are staged in LDS (shared by the 64 rows), normalised there once,
// and read back as broadcasts. Online softmax in exp2 units with a per-tile
// rescale.
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
  const int lane = threadIdx.x;
  const int kvh = item.y >> 16, head = item.y & 0xffff;
  const int t = item.x + lane;
  const bool valid = t < prm.tq;
  const float* qg = prm.q_gain;
  for (int d = lane; d < D; d += 64) gk[d] = prm.k_gain[d];

  float q[D];
  float o[D];
  {
    const float* qrow = reinterpret_cast<const float*>(prm.q) + (size_t(t) * prm.hq + head) * D;
    float ss = 0.0f;
    for (int d = 0; d < D; ++d) {
      q[d] = valid ? qrow[d] : 0.0f;
      ss += q[d] * q[d];
    }
    const float rq = 1.0f / __builtin_sqrtf(ss / D + prm.eps);
    const float c = prm.scale * kLog2e;
    for (int d = 0; d < D; ++d) {
      q[d] = valid ? q[d] * rq * qg[d] * c : 0.0f;
      o[d] = 0.0f;
    }
  }
  const int2 rb = valid ? prm.rows[t] : int2{0, 0};
  float m = kNegInf, l = 0.0f;
  const float* kbase = reinterpret_cast<const float*>(prm.k);
  const float* vbase = reinterpret_cast<const float*>(prm.v);

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
        const bool in = key < prm.tk;
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
    float* orow = reinterpret_cast<float*>(prm.out) + (size_t(t) * prm.hq + head) * D;
    const float inv = 1.0f / l;
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    prm.lse[size_t(head) * prm.tq + t] = (m + __builtin_log2f(l)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd_fp32(const FwdParams& p, int head_dim, int n_items, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL(fwd_fp32_kernel<64>, dim3(n_items), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_fp32_kernel<128>, dim3(n_items), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace magi
