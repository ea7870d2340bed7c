// Query preparation shared by attention and the inner-product scan:
//   q' = RoPE(q) (optional), q_rot = H_d (D * q') / sqrt(d), Sq = S q_rot.
// The query is not normalised: the
// estimate of <q, x> is linear in q ("Google presenta TurboQuant ...",
// "Eliminación del sesgo interno del producto").
//
// A workgroup prepares QR query rows (8, or 64 when there are many rows, so
// that S is staged and the butterfly barriers are paid once per 64 rows):
// their butterflies run through LDS, and S is staged once into LDS with a
// padded row stride (d + 1 floats, so that the lanes of a wave reading
// S[i][k] for consecutive i hit distinct banks) and read from there for the
// d-long dot products.

#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"
#include "qprep.hpp"

namespace tqk {

constexpr int kQThreads = 256;

template <int D, typename T, bool ROPE, int kQRows>
__global__ __launch_bounds__(kQThreads) void qprep_kernel(QPrepParams p) {
  constexpr int SP = D + 1;                         // padded S row stride
  __shared__ float s_S[D * SP];
  __shared__ float s_v[kQRows][D];
  __shared__ uint32_t s_flip[D / 32];
  __shared__ double s_theta[D / 2];

  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * kQRows;
  const int nrows = (p.n_rows - row0) < kQRows ? (int)(p.n_rows - row0) : kQRows;
  const uint32_t* kflip = reinterpret_cast<const uint32_t*>(
      (const char*)__builtin_amdgcn_kernarg_segment_ptr() +
      offsetof(QPrepParams, flip));
  const double* ktheta = reinterpret_cast<const double*>(
      (const char*)__builtin_amdgcn_kernarg_segment_ptr() +
      offsetof(QPrepParams, theta));
  if (tid < D / 32) s_flip[tid] = kflip[tid];
  if (ROPE && tid < D / 2) s_theta[tid] = ktheta[tid];

  // S into LDS (coalesced 16-byte reads, padded rows)
  if (p.S != nullptr) {
    const float4* S4 = reinterpret_cast<const float4*>(p.S);
    for (int t = tid; t < D * D / 4; t += kQThreads) {
      const float4 v = S4[t];
      const int i = (4 * t) / D, k = (4 * t) % D;
      float* dst = s_S + i * SP + k;
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
  }
  // query rows
  const T* q = reinterpret_cast<const T*>(p.q);
  for (int t = tid; t < kQRows * D; t += kQThreads) {
    const int r = t / D, i = t % D;
    s_v[r][i] = r < nrows ? (float)q[(row0 + r) * D + i] : 0.f;
  }
  __syncthreads();
  constexpr int PER = kQRows * D / kQThreads;
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = tid + u * kQThreads, r = t / D, i = t % D;
    float x = s_v[r][i];
    if constexpr (ROPE) {
      const int pr = i >> 1;
      const int64_t pos = (int64_t)p.pos0 + ((row0 + r) % p.n_q);
      float sn, cs;
      sincos_reduced((double)pos * s_theta[pr], sn, cs);
      const float a = s_v[r][2 * pr], b = s_v[r][2 * pr + 1];
      x = (i & 1) ? (a * sn + b * cs) : (a * cs - b * sn);
    }
    const uint32_t bit = (s_flip[i >> 5] >> (i & 31)) & 1u;
    v[u] = bit ? -x : x;
  }
  // natural-order butterflies through LDS
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = tid + u * kQThreads;
      s_v[t / D][t % D] = v[u];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = tid + u * kQThreads, r = t / D, i = t % D;
      const float o = s_v[r][i ^ h];
      v[u] = (i & h) ? (o - v[u]) : (v[u] + o);
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = tid + u * kQThreads, r = t / D, i = t % D;
    const float x = v[u] * p.inv_sqrt_d;
    s_v[r][i] = x;
    if (r < nrows) p.qrot[(row0 + r) * D + i] = x;
  }
  if (p.S == nullptr) return;
  __syncthreads();
  // Sq[r][i] = sum_k S[i][k] q_rot[r][k]; thread -> (row group, i)
  constexpr int RG = kQThreads / D;                 // row groups (2 for d=128)
  constexpr int RPG = kQRows / RG;                  // rows per group
  const int i = tid % D, rg = tid / D;
  float acc[RPG];
#pragma unroll
  for (int a = 0; a < RPG; ++a) acc[a] = 0.f;
  const float* srow = s_S + i * SP;
#pragma unroll 4
  for (int k = 0; k < D; ++k) {
    const float s = srow[k];
#pragma unroll
    for (int a = 0; a < RPG; ++a) acc[a] = fmaf(s, s_v[rg * RPG + a][k], acc[a]);
  }
#pragma unroll
  for (int a = 0; a < RPG; ++a) {
    const int r = rg * RPG + a;
    if (r < nrows) p.sq[(row0 + r) * D + i] = acc[a];
  }
}

template <int D, typename T, int QR>
static hipError_t run_qprep_rows(const QPrepParams& p, bool rope, hipStream_t s) {
  const unsigned blocks = (unsigned)((p.n_rows + QR - 1) / QR);
  if (rope)
    hipLaunchKernelGGL((qprep_kernel<D, T, true, QR>), dim3(blocks), dim3(kQThreads), 0, s, p);
  else
    hipLaunchKernelGGL((qprep_kernel<D, T, false, QR>), dim3(blocks), dim3(kQThreads), 0, s, p);
  return hipGetLastError();
}

template <int D, typename T>
static hipError_t run_qprep(const QPrepParams& p, bool rope, hipStream_t s) {
  if (p.n_rows >= 8192) return run_qprep_rows<D, T, 64>(p, rope, s);
  return run_qprep_rows<D, T, 8>(p, rope, s);
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
