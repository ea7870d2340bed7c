// Inner-product scan over packed codes (+ top-k), d = 64 or 128.
//
// est(a, j) = nu_j ( <q_rot_a, c[idx_j]> + sqrt(pi/2)/m gamma_j
//                    <Sq_a, 2 sigma_j - 1> )
// ("Google presenta TurboQuant ...", "Eliminación del sesgo interno del
// producto" for the estimator, "Velocidad y eficiencia de indexación" for
// search over codes).  One thread per database row: the row is dequantized
// once into registers (c[idx_i] from the LDS table) and scored against a
// block of queries read from LDS as broadcasts.  The QJL term uses
// <Sq, 2 sigma - 1> = 2 sum_{sigma_i = 1} Sq_i - sum_i Sq_i.
//
// Top-k: one wavefront per query keeps, per lane, a sorted list of its best
// k (rows scanned in increasing order, strict comparison, so equal scores
// keep the lower row first), then merges the 64 lists with k wave-wide
// arg-max rounds (ties to the lower row).

#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"
#include "qprep.hpp"

namespace tqk {

constexpr int kScanRows = 256;
constexpr int kScanQB = 8;

struct ScanParams {
  const uint8_t* idx;
  const uint8_t* qjl;
  const float* norm;
  const float* rnorm;
  int64_t n;
  int64_t n_q;
  const float* qrot;
  const float* sq;
  float* out;          // [n_q][n]
  float centroids[16];
  float qjl_scale;     // sqrt(pi/2) / m
};

template <int D, int CB, bool PROD>
__global__ __launch_bounds__(kScanRows) void scan_kernel(ScanParams p) {
  constexpr int W = D * CB / 32;
  constexpr int ROW_BYTES = D * CB / 8;
  constexpr int ALIGN = ROW_BYTES % 16 == 0 ? 16 : 8;
  __shared__ float s_cent[16];
  __shared__ float s_q[kScanQB][D];
  __shared__ float s_s[kScanQB][D];
  __shared__ float s_tot[kScanQB];
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (tid == k) s_cent[k] = p.centroids[k];
  const int64_t q0 = (int64_t)blockIdx.y * kScanQB;
  const int nqb = (int)((p.n_q - q0) < kScanQB ? (p.n_q - q0) : kScanQB);
  for (int t = tid; t < kScanQB * D; t += kScanRows) {
    const int a = t / D, i = t % D;
    s_q[a][i] = a < nqb ? p.qrot[(q0 + a) * D + i] : 0.f;
    if constexpr (PROD) s_s[a][i] = a < nqb ? p.sq[(q0 + a) * D + i] : 0.f;
  }
  __syncthreads();
  if constexpr (PROD) {
    if (tid < kScanQB) {
      float t = 0.f;
      for (int i = 0; i < D; ++i) t += s_s[tid][i];
      s_tot[tid] = t;
    }
    __syncthreads();
  }
  const int64_t row = (int64_t)blockIdx.x * kScanRows + tid;
  if (row >= p.n) return;
  uint32_t w[W];
  load_words<W, ALIGN>(p.idx + row * ROW_BYTES, w);
  float c[D];
#pragma unroll
  for (int i = 0; i < D; ++i) c[i] = s_cent[get_code<CB, W>(w, i)];
  const float nu = p.norm[row];
  uint32_t sb[D / 32] = {};
  float gk = 0.f;
  if constexpr (PROD) {
    load_words<D / 32, (D / 8) % 16 == 0 ? 16 : 8>(p.qjl + row * (D / 8), sb);
    gk = p.rnorm[row] * p.qjl_scale;
  }
  for (int a = 0; a < nqb; ++a) {
    float m0 = 0.f, m1 = 0.f;
#pragma unroll
    for (int i = 0; i < D; i += 2) {
      m0 = fmaf(c[i], s_q[a][i], m0);
      m1 = fmaf(c[i + 1], s_q[a][i + 1], m1);
    }
    float est = m0 + m1;
    if constexpr (PROD) {
      float pos0 = 0.f, pos1 = 0.f;
#pragma unroll
      for (int i = 0; i < D; i += 2) {
        pos0 += ((sb[i >> 5] >> (i & 31)) & 1u) ? s_s[a][i] : 0.f;
        pos1 += ((sb[(i + 1) >> 5] >> ((i + 1) & 31)) & 1u) ? s_s[a][i + 1] : 0.f;
      }
      est = fmaf(gk, 2.f * (pos0 + pos1) - s_tot[a], est);
    }
    p.out[(q0 + a) * p.n + row] = nu * est;
  }
}

// ---- top-k ---------------------------------------------------------------
constexpr int kTopMax = 64;

struct TopKParams {
  const float* scores;   // [n_q][n]
  int64_t n;
  int k;
  int64_t* ids;
  float* vals;
};

__global__ __launch_bounds__(kWave) void topk_kernel(TopKParams p) {
  __shared__ float s_val[kWave][kTopMax + 1];
  __shared__ int64_t s_id[kWave][kTopMax + 1];
  const int lane = threadIdx.x;
  const int64_t qa = blockIdx.x;
  const float* sc = p.scores + qa * p.n;
  const int k = p.k;
  int cnt = 0;
  for (int64_t j = lane; j < p.n; j += kWave) {
    const float s = sc[j];
    if (cnt == k && !(s > s_val[lane][k - 1])) continue;
    int pos = cnt < k ? cnt : k - 1;
    while (pos > 0 && s_val[lane][pos - 1] < s) {
      s_val[lane][pos] = s_val[lane][pos - 1];
      s_id[lane][pos] = s_id[lane][pos - 1];
      --pos;
    }
    s_val[lane][pos] = s;
    s_id[lane][pos] = j;
    if (cnt < k) ++cnt;
  }
  int head = 0;
  for (int r = 0; r < k; ++r) {
    float bv = head < cnt ? s_val[lane][head] : -INFINITY;
    int64_t bi = head < cnt ? s_id[lane][head] : INT64_MAX;
    int bl = lane;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int64_t oi = __shfl_xor(bi, off);
      const int ol = __shfl_xor(bl, off);
      const bool take = ov > bv || (ov == bv && oi < bi);
      bv = take ? ov : bv;
      bi = take ? oi : bi;
      bl = take ? ol : bl;
    }
    if (lane == bl) ++head;
    if (lane == 0) {
      p.ids[qa * k + r] = bi;
      p.vals[qa * k + r] = bv;
    }
  }
}

size_t scan_workspace_bytes(int64_t n_q, int64_t n, int d, int top_k) {
  size_t b = (size_t)n_q * d * 2 * sizeof(float);
  b = (b + 255) & ~(size_t)255;
  if (top_k > 0) b += (size_t)n_q * n * sizeof(float);
  return b;
}

template <int D, int CB, bool PROD>
static hipError_t run_scan(const ScanParams& p, hipStream_t s) {
  const dim3 grid((unsigned)((p.n + kScanRows - 1) / kScanRows),
                  (unsigned)((p.n_q + kScanQB - 1) / kScanQB));
  hipLaunchKernelGGL((scan_kernel<D, CB, PROD>), grid, dim3(kScanRows), 0, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t pick_scan(int cb, bool prod, const ScanParams& p, hipStream_t s) {
  switch (cb) {
    case 1: return prod ? run_scan<D, 1, true>(p, s) : run_scan<D, 1, false>(p, s);
    case 2: return prod ? run_scan<D, 2, true>(p, s) : run_scan<D, 2, false>(p, s);
    case 3: return prod ? run_scan<D, 3, true>(p, s) : run_scan<D, 3, false>(p, s);
    case 4: return prod ? run_scan<D, 4, true>(p, s) : run_scan<D, 4, false>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan(const tq_codec& c, const void* q, int q_dtype, int64_t n_q,
                       const tq_packed& x, int64_t n, float* out, int top_k,
                       int64_t* top_ids, float* top_scores, void* workspace,
                       hipStream_t stream) {
  const int d = c.d;
  float* qrot = reinterpret_cast<float*>(workspace);
  float* sq = qrot + (size_t)n_q * d;
  size_t off = ((size_t)n_q * d * 2 * sizeof(float) + 255) & ~(size_t)255;
  float* scores = out;
  if (top_k > 0 && scores == nullptr)
    scores = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + off);
  hipError_t e = launch_qprep(c, q, q_dtype, n_q, n_q, RopeHost{}, qrot, sq, stream);
  if (e != hipSuccess) return e;
  ScanParams p = {};
  p.idx = x.idx;
  p.qjl = x.qjl;
  p.norm = x.norm;
  p.rnorm = x.rnorm;
  p.n = n;
  p.n_q = n_q;
  p.qrot = qrot;
  p.sq = sq;
  p.out = scores;
  for (int k = 0; k < 16; ++k) p.centroids[k] = c.centroids[k];
  p.qjl_scale = c.mode == TQ_PROD ? (float)(std::sqrt(M_PI / 2.0) / c.m) : 0.f;
  const bool prod = c.mode == TQ_PROD;
  if (d == 128) e = pick_scan<128>(c.code_bits, prod, p, stream);
  else if (d == 64) e = pick_scan<64>(c.code_bits, prod, p, stream);
  else return hipErrorInvalidValue;
  if (e != hipSuccess || top_k == 0) return e;
  TopKParams t = {scores, n, top_k, top_ids, top_scores};
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)n_q), dim3(kWave), 0, stream, t);
  return hipGetLastError();
}

}  // namespace tqk
