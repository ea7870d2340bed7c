// Query preparation shared by attention and the inner-product scan:
//   q' = RoPE(q) (optional), q_rot = H_d (D * q') / sqrt(d), Sq = S q_rot.
// The query is not normalised: the estimate of <q, x> is linear in q
// ("Google presenta TurboQuant ...", "Eliminación del sesgo interno del
// producto").  One workgroup of d threads per query row; the butterflies
// run through LDS, the S q_rot rows are d-long dot products.

#include "device_common.hpp"
#include "internal.hpp"
#include "qprep.hpp"

namespace tqk {

template <int D, typename T, bool ROPE>
__global__ __launch_bounds__(D) void qprep_kernel(QPrepParams p) {
  __shared__ float s_v[D];
  const int i = threadIdx.x;
  const int64_t row = blockIdx.x;
  const T* q = reinterpret_cast<const T*>(p.q) + row * D;
  float v = (float)q[i];
  if constexpr (ROPE) {
    s_v[i] = v;
    __syncthreads();
    const int pair = i >> 1;
    const int64_t pos = (int64_t)p.pos0 + (row % p.n_q);
    float s, c;
    sincos_reduced((double)pos * p.theta[pair], s, c);
    const float a = s_v[2 * pair], b = s_v[2 * pair + 1];
    v = (i & 1) ? (a * s + b * c) : (a * c - b * s);
    __syncthreads();
  }
  const uint32_t bit = (p.flip[i >> 5] >> (i & 31)) & 1u;
  v = bit ? -v : v;
  // natural-order butterflies through LDS
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
    s_v[i] = v;
    __syncthreads();
    const float o = s_v[i ^ h];
    v = (i & h) ? (o - v) : (v + o);
    __syncthreads();
  }
  v *= p.inv_sqrt_d;
  s_v[i] = v;
  p.qrot[row * D + i] = v;
  if (p.S != nullptr) {
    __syncthreads();
    const float4* srow = reinterpret_cast<const float4*>(p.S + (size_t)i * D);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int k = 0; k < D / 4; ++k) {
      const float4 s = srow[k];
      acc[0] = fmaf(s.x, s_v[4 * k], acc[0]);
      acc[1] = fmaf(s.y, s_v[4 * k + 1], acc[1]);
      acc[2] = fmaf(s.z, s_v[4 * k + 2], acc[2]);
      acc[3] = fmaf(s.w, s_v[4 * k + 3], acc[3]);
    }
    p.sq[row * D + i] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
}

template <int D, typename T>
static hipError_t run_qprep(const QPrepParams& p, bool rope, hipStream_t s) {
  if (rope)
    hipLaunchKernelGGL((qprep_kernel<D, T, true>), dim3((unsigned)p.n_rows), dim3(D), 0, s, p);
  else
    hipLaunchKernelGGL((qprep_kernel<D, T, false>), dim3((unsigned)p.n_rows), dim3(D), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_qprep(const tq_codec& c, const void* q, int q_dtype, int64_t n_rows,
                        int64_t n_q, const RopeHost& rope, float* qrot, float* sq,
                        hipStream_t stream) {
  QPrepParams p = {};
  p.q = q;
  p.n_rows = n_rows;
  p.n_q = n_q > 0 ? n_q : 1;
  p.pos0 = rope.on ? rope.pos0 : 0;
  for (int w = 0; w < 48; ++w) p.flip[w] = c.flip[w];
  p.S = c.mode == TQ_PROD ? c.S : nullptr;
  p.qrot = qrot;
  p.sq = sq;
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)c.d));
  if (rope.on)
    for (int i = 0; i < c.d / 2 && i < 64; ++i)
      p.theta[i] = std::pow((double)rope.base, -2.0 * i / (double)c.d);
  if (n_rows == 0) return hipSuccess;
  if (c.d == 128)
    return q_dtype == TQ_F16 ? run_qprep<128, _Float16>(p, rope.on, stream)
                             : run_qprep<128, float>(p, rope.on, stream);
  if (c.d == 64)
    return q_dtype == TQ_F16 ? run_qprep<64, _Float16>(p, rope.on, stream)
                             : run_qprep<64, float>(p, rope.on, stream);
  return hipErrorInvalidValue;
}

}  // namespace tqk
