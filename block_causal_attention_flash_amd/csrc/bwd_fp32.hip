// Backward of the block-causal QK-RMSNorm GQA attention, fp32 (head_dim 64 or
// 128), on the vector ALUs: the same gradients as the bf16 kernels (see
// bwd_bf16.hip; MAGI-1 pages: paperlayer §2 / Figure 1, §2.2.2; paper-notes
// §3.2.2), computed in fp32 throughout for callers that need fp32 accuracy.
//   prep   per (token, query head): q' = rms(q) g_q g_k scale, q_hat =
//          rms(q) g_q, and D = <dO, O>;
//   dq     one thread per query row over the key tiles of its dq item (keys
//          RMS-normalised in LDS), then the RMSNorm backward;
//   dkdv   one thread per key of a 64-key block over the (32-token tile,
//          query head) steps that see it (rows staged in LDS);
//   reduce the gain gradients from per-workgroup partials.
#include "kernels.hpp"

namespace magi {
namespace {

constexpr int BN = 32;
constexpr int KB = 64;                  // keys per dk/dv item
constexpr float kNegInf = -__builtin_inff();

struct F32Layout {
  size_t qp, qh, dd, pgq, pgk, total;
};

F32Layout f32_layout(long long tq, int hq, int d, int n_dq_items, int n_kv_items) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = size_t(tq) * size_t(hq);
  F32Layout L{};
  L.qp = 0;
  L.qh = up(rows * d * 4);
  L.dd = L.qh + up(rows * d * 4);
  L.pgq = L.dd + up(rows * 4);
  L.pgk = L.pgq + up(size_t(n_dq_items) * d * 4);
  L.total = L.pgk + up(size_t(n_kv_items) * d * 4);
  return L;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// One thread per (token, query head) row.
template <int D>
__global__ void __launch_bounds__(64) bwd_prep_f32_kernel(BwdParams p, F32Layout L) {
  const size_t r = size_t(blockIdx.x) * 64 + threadIdx.x;   // row = token * hq + head
  if (r >= size_t(p.tq) * p.hq) return;
  const size_t tok = r / p.hq, h = r % p.hq;
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const float* q = static_cast<const float*>(p.q) + r * D;
  const float* o = static_cast<const float*>(p.out) + r * D;
  const float* dO = static_cast<const float*>(p.dout) + r * D;
  float ss = 0.0f, dd = 0.0f;
  for (int d = 0; d < D; ++d) {
    ss += q[d] * q[d];
    dd += dO[d] * o[d];
  }
  const float rq = 1.0f / __builtin_sqrtf(ss / D + p.eps);
  float* qp = reinterpret_cast<float*>(ws + L.qp) + r * D;
  float* qh = reinterpret_cast<float*>(ws + L.qh) + r * D;
  for (int d = 0; d < D; ++d) {
    qh[d] = q[d] * rq * p.q_gain[d];
    qp[d] = qh[d] * p.k_gain[d] * p.scale;
  }
  reinterpret_cast<float*>(ws + L.dd)[h * p.tq + tok] = dd;
}

template <int D>
__device__ __forceinline__ void write_partial(float (&gp)[D], float* part, int lane) {
  for (int d = 0; d < D; ++d) {
    const float x = wave_sum(gp[d]);
    if (lane == 0) part[d] = x;
  }
}

// dq: one wave per dq item (64 tokens of one query head).
template <int D>
__global__ void __launch_bounds__(64) bwd_dq_f32_kernel(BwdParams p, F32Layout L) {
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int lane = threadIdx.x;
  float* part = reinterpret_cast<float*>(ws + L.pgq) + size_t(blockIdx.x) * D;
  const int4 item = p.dq_items[2 * blockIdx.x];
  if (item.z == item.w) {
    for (int d = lane; d < D; d += 64) part[d] = 0.0f;
    return;
  }
  const int kvh = item.y >> 16, head = item.y & 0xffff;
  const int t = item.x + lane;
  const bool valid = t < p.tq;
  const size_t r = size_t(valid ? t : 0) * p.hq + head;
  const float* qp = reinterpret_cast<const float*>(ws + L.qp) + r * D;
  const float* dO = static_cast<const float*>(p.dout) + r * D;
  float qv[D], dov[D], acc[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = valid ? qp[d] : 0.0f;
    dov[d] = valid ? dO[d] : 0.0f;
    acc[d] = 0.0f;
  }
  const float lse = valid ? p.lse[size_t(head) * p.tq + t] : 0.0f;
  const float dd = valid ? reinterpret_cast<const float*>(ws + L.dd)[size_t(head) * p.tq + t] : 0.0f;
  const int2 rb = valid ? p.rows[t] : int2{0, 0};
  const float* kbase = static_cast<const float*>(p.k);
  const float* vbase = static_cast<const float*>(p.v);
  for (int ti = item.z; ti < item.w; ++ti) {
    const int kt = p.dq_tiles[ti] >> 1;
    __syncthreads();
    for (int e = lane; e < BN * D; e += 64) {
      const int j = e / D, d = e % D, key = kt * BN + j;
      const bool in = key < p.tk;
      const size_t off = (size_t(in ? key : 0) * p.hk + kvh) * D + d;
      ks[j][d] = in ? kbase[off] : 0.0f;
      vs[j][d] = in ? vbase[off] : 0.0f;
    }
    __syncthreads();
    if (lane < BN) {
      float ss = 0.0f;
      for (int d = 0; d < D; ++d) ss += ks[lane][d] * ks[lane][d];
      const float rk = 1.0f / __builtin_sqrtf(ss / D + p.eps);
      for (int d = 0; d < D; ++d) ks[lane][d] *= rk;
    }
    __syncthreads();
    for (int j = 0; j < BN; ++j) {
      const int key = kt * BN + j;
      if (!(key >= rb.x && key < rb.y)) continue;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s += qv[d] * ks[j][d];
        dp += dov[d] * vs[j][d];
      }
      const float ds = __expf(s - lse) * (dp - dd);
      for (int d = 0; d < D; ++d) acc[d] += ds * ks[j][d];
    }
  }
  // dq_hat = scale g_k acc; RMSNorm backward.
  float gp[D];
  const float* q = static_cast<const float*>(p.q) + r * D;
  float ss = 0.0f;
  for (int d = 0; d < D; ++d) ss += valid ? q[d] * q[d] : 0.0f;
  const float rq = 1.0f / __builtin_sqrtf(ss / D + p.eps);
  float m = 0.0f;
  for (int d = 0; d < D; ++d) {
    acc[d] *= p.scale * p.k_gain[d];                       // dq_hat
    const float u = valid ? q[d] * rq : 0.0f;
    m += u * p.q_gain[d] * acc[d];
    gp[d] = u * acc[d];
  }
  m /= D;
  if (valid) {
    float* dq = static_cast<float*>(p.dq) + r * D;
    for (int d = 0; d < D; ++d) dq[d] = (p.q_gain[d] * acc[d] - q[d] * rq * m) * rq;
  }
  write_partial<D>(gp, part, lane);
}

// dk/dv: one wave per (64-key block, KV head).
template <int D>
__global__ void __launch_bounds__(64) bwd_dkdv_f32_kernel(BwdParams p, F32Layout L) {
  __shared__ float sq[BN][D];      // q' rows of the step
  __shared__ float sh[BN][D];      // q_hat rows
  __shared__ float sd[BN][D];      // dO rows
  __shared__ float sl[BN], sdd[BN];
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  const int lane = threadIdx.x;
  float* part = reinterpret_cast<float*>(ws + L.pgk) + size_t(blockIdx.x) * D;
  const int4 item = p.kv_items[2 * blockIdx.x];
  if (item.z == item.w) {
    for (int d = lane; d < D; d += 64) part[d] = 0.0f;
    return;
  }
  const int n_full = p.kv_items[2 * blockIdx.x + 1].x;
  const int kb = item.x, kvh = item.y;
  const int G = p.hq / p.hk;
  const int key = kb * KB + lane;
  const bool valid = key < p.tk;
  const size_t kr = (size_t(valid ? key : 0) * p.hk + kvh) * D;
  const float* k = static_cast<const float*>(p.k) + kr;
  const float* v = static_cast<const float*>(p.v) + kr;
  float ku[D], vv[D], ak[D], av[D];
  float ss = 0.0f;
  for (int d = 0; d < D; ++d) ss += valid ? k[d] * k[d] : 0.0f;
  const float rk = 1.0f / __builtin_sqrtf(ss / D + p.eps);
  for (int d = 0; d < D; ++d) {
    ku[d] = valid ? k[d] * rk : 0.0f;
    vv[d] = valid ? v[d] : 0.0f;
    ak[d] = av[d] = 0.0f;
  }
  const int4 kbnd = valid ? p.key_rows[key] : int4{0, 0, 0, 0};
  const float* qp = reinterpret_cast<const float*>(ws + L.qp);
  const float* qh = reinterpret_cast<const float*>(ws + L.qh);
  const float* dd = reinterpret_cast<const float*>(ws + L.dd);
  for (int e = item.z; e < item.w; ++e) {
    const int tt = p.kv_tiles[e] >> 1;
    const bool masked = e - item.z >= n_full;
    for (int hh = 0; hh < G; ++hh) {
      const int head = kvh * G + hh;
      __syncthreads();
      for (int x = lane; x < BN * D; x += 64) {
        const int j = x / D, d = x % D, tok = tt * BN + j;
        const bool in = tok < p.tq;
        const size_t off = (size_t(in ? tok : 0) * p.hq + head) * D + d;
        sq[j][d] = in ? qp[off] : 0.0f;
        sh[j][d] = in ? qh[off] : 0.0f;
        sd[j][d] = in ? static_cast<const float*>(p.dout)[off] : 0.0f;
      }
      if (lane < BN) {
        const int tok = tt * BN + lane;
        const bool in = tok < p.tq;
        sl[lane] = in ? p.lse[size_t(head) * p.tq + tok] : 0.0f;
        sdd[lane] = in ? dd[size_t(head) * p.tq + tok] : 0.0f;
      }
      __syncthreads();
      for (int j = 0; j < BN; ++j) {
        const int tok = tt * BN + j;
        if (tok >= p.tq ||
            (masked && !(tok >= kbnd.x && tok < kbnd.y) && !(tok >= kbnd.z && tok < kbnd.w)))
          continue;
        float s = 0.0f, dp = 0.0f;
        for (int d = 0; d < D; ++d) {
          s += sq[j][d] * ku[d];
          dp += sd[j][d] * vv[d];
        }
        const float pv = __expf(s - sl[j]);
        const float ds = pv * (dp - sdd[j]);
        for (int d = 0; d < D; ++d) {
          av[d] += pv * sd[j][d];
          ak[d] += ds * sh[j][d];
        }
      }
    }
  }
  float gp[D];
  float m = 0.0f;
  for (int d = 0; d < D; ++d) {
    ak[d] *= p.scale;                                       // dk_hat
    m += ku[d] * p.k_gain[d] * ak[d];
    gp[d] = ku[d] * ak[d];
  }
  m /= D;
  if (valid) {
    float* dk = static_cast<float*>(p.dk) + kr;
    float* dv = static_cast<float*>(p.dv) + kr;
    for (int d = 0; d < D; ++d) {
      dk[d] = (p.k_gain[d] * ak[d] - ku[d] * m) * rk;
      dv[d] = av[d];
    }
  }
  write_partial<D>(gp, part, lane);
}

template <int D>
__global__ void __launch_bounds__(256) bwd_gain_reduce_f32_kernel(const float* pgq, int nq, const float* pgk, int nk,
                                                                 float* dq_gain, float* dk_gain) {
  const int t = threadIdx.x;
  if (t >= 2 * D) return;
  const int d = t % D;
  const float* src = t < D ? pgq : pgk;
  const int n = t < D ? nq : nk;
  float x = 0.0f;
  for (int i = 0; i < n; ++i) x += src[size_t(i) * D + d];
  (t < D ? dq_gain : dk_gain)[d] = x;
}

template <int D>
hipError_t launch(const BwdParams& p, hipStream_t stream) {
  const F32Layout L = f32_layout(p.tq, p.hq, D, p.n_dq_items, p.n_kv_items);
  const size_t rows = size_t(p.tq) * p.hq;
  hipLaunchKernelGGL(bwd_prep_f32_kernel<D>, dim3(unsigned((rows + 63) / 64)), dim3(64), 0, stream, p, L);
  if (p.n_dq_items > 0) hipLaunchKernelGGL(bwd_dq_f32_kernel<D>, dim3(p.n_dq_items), dim3(64), 0, stream, p, L);
  if (p.n_kv_items > 0) hipLaunchKernelGGL(bwd_dkdv_f32_kernel<D>, dim3(p.n_kv_items), dim3(64), 0, stream, p, L);
  const hipError_t ez = launch_bwd_zero_rows(p, D * 4, stream);
  if (ez != hipSuccess) return ez;
  unsigned char* ws = static_cast<unsigned char*>(p.ws);
  hipLaunchKernelGGL(bwd_gain_reduce_f32_kernel<D>, dim3(1), dim3(256), 0, stream,
                     reinterpret_cast<const float*>(ws + L.pgq), p.n_dq_items,
                     reinterpret_cast<const float*>(ws + L.pgk), p.n_kv_items, p.dq_gain, p.dk_gain);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes_fp32(long long tq, long long tk, int hq, int hk, int head_dim, int n_dq_items,
                                int n_kv_items) {
  (void)tk;
  (void)hk;
  return f32_layout(tq, hq, head_dim, n_dq_items, n_kv_items).total;
}

hipError_t launch_bwd_fp32(const BwdParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch<64>(p, stream) : launch<128>(p, stream);
}

}  // namespace magi
