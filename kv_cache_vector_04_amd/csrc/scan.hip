// Inner-product scan over packed codes (+ top-k); d = 64 and 128 here,
// d = 1536 in wide.hip.
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
// Top-k runs over the score matrix in two passes (below).

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
// Two passes.  Pass 1: one wavefront per (query, chunk of rows) keeps, per
// lane, a sorted list of its best k (descending score, ties to the lower row
// index), then merges the 64 lists with k wave-wide arg-max rounds into the
// chunk's k candidates.  Pass 2 runs the same wavefront routine over the
// candidates of all chunks of a query.  Lists shorter than k are padded with
// (-inf, INT64_MAX), which every real entry beats.
constexpr int kTopMax = 64;

struct TopKParams {
  const float* val;      // pass 1: scores [n_q][len]; pass 2: candidates [n_q][len]
  const int64_t* id;     // pass 2: candidate ids; pass 1: nullptr (id = position)
  int64_t len;           // items per query
  int64_t chunk;         // items per wavefront
  int nchunks;           // wavefronts per query
  int k;
  float* oval;           // [n_q][nchunks][k]
  int64_t* oid;
};

__device__ __forceinline__ bool better(float v1, int64_t i1, float v2, int64_t i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <int KM>
__global__ __launch_bounds__(kWave) void topk_kernel(TopKParams p) {
  __shared__ float s_val[kWave][KM];
  __shared__ int64_t s_id[kWave][KM];
  const int lane = threadIdx.x;
  const int64_t qa = blockIdx.x / p.nchunks;
  const int c = (int)(blockIdx.x % p.nchunks);
  const int64_t beg = (int64_t)c * p.chunk;
  const int64_t end = (beg + p.chunk) < p.len ? (beg + p.chunk) : p.len;
  const float* val = p.val + qa * p.len;
  const int64_t* ids = p.id != nullptr ? p.id + qa * p.len : nullptr;
  const int k = p.k;
  int cnt = 0;
  float kv = -INFINITY;          // the lane's k-th entry once its list is full
  int64_t ki = INT64_MAX;
  for (int64_t j0 = beg + lane; j0 < end; j0 += 4 * kWave) {
    float v[4];
    int64_t id[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = j0 + u * kWave;
      const bool in = j < end;
      v[u] = in ? val[j] : -INFINITY;
      id[u] = in ? (ids != nullptr ? ids[j] : j) : INT64_MAX;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (id[u] == INT64_MAX) continue;                    // padding
      if (cnt == k && !better(v[u], id[u], kv, ki)) continue;
      int pos = cnt < k ? cnt : k - 1;
      while (pos > 0 && better(v[u], id[u], s_val[lane][pos - 1], s_id[lane][pos - 1])) {
        s_val[lane][pos] = s_val[lane][pos - 1];
        s_id[lane][pos] = s_id[lane][pos - 1];
        --pos;
      }
      s_val[lane][pos] = v[u];
      s_id[lane][pos] = id[u];
      if (cnt < k) ++cnt;
      if (cnt == k) {
        kv = s_val[lane][k - 1];
        ki = s_id[lane][k - 1];
      }
    }
  }
  int head = 0;
  float* ov = p.oval + ((int64_t)qa * p.nchunks + c) * k;
  int64_t* oi = p.oid + ((int64_t)qa * p.nchunks + c) * k;
  for (int r = 0; r < k; ++r) {
    float bv = head < cnt ? s_val[lane][head] : -INFINITY;
    int64_t bi = head < cnt ? s_id[lane][head] : INT64_MAX;
    int bl = lane;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float xv = __shfl_xor(bv, off);
      const int64_t xi = __shfl_xor(bi, off);
      const int xl = __shfl_xor(bl, off);
      const bool take = better(xv, xi, bv, bi) || (xv == bv && xi == bi && xl < bl);
      bv = take ? xv : bv;
      bi = take ? xi : bi;
      bl = take ? xl : bl;
    }
    if (lane == bl) ++head;
    if (lane == 0) {
      ov[r] = bv;
      oi[r] = bi;
    }
  }
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// wavefronts per query in pass 1: enough to fill the device, at least about
// a thousand rows each
static int topk_chunks(int64_t n_q, int64_t n) {
  int64_t want = (16384 + n_q - 1) / n_q;
  const int64_t cap = (n + 1023) / 1024;
  if (want > cap) want = cap;
  if (want > 4096) want = 4096;
  if (want < 1) want = 1;
  return (int)want;
}

static size_t prep_bytes(int64_t n_q, int d) {
  return d == 1536 ? wide_scan_workspace_bytes(n_q)
                   : align256((size_t)n_q * d * 2 * sizeof(float));
}

size_t scan_workspace_bytes(int64_t n_q, int64_t n, int d, int top_k) {
  size_t b = prep_bytes(n_q, d);
  if (top_k > 0) {
    const size_t cand = (size_t)n_q * topk_chunks(n_q, n) * top_k;
    b += align256((size_t)n_q * n * sizeof(float));     // scores when `out` is NULL
    b += align256(cand * sizeof(float)) + align256(cand * sizeof(int64_t));
  }
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

static hipError_t run_topk(const TopKParams& t, int64_t n_q, hipStream_t s) {
  const unsigned blocks = (unsigned)(n_q * t.nchunks);
  if (t.k <= 16)
    hipLaunchKernelGGL(topk_kernel<16>, dim3(blocks), dim3(kWave), 0, s, t);
  else
    hipLaunchKernelGGL(topk_kernel<kTopMax>, dim3(blocks), dim3(kWave), 0, s, t);
  return hipGetLastError();
}

hipError_t launch_scan(const tq_codec& c, const void* q, int q_dtype, int64_t n_q,
                       const tq_packed& x, int64_t n, float* out, int top_k,
                       int64_t* top_ids, float* top_scores, void* workspace,
                       hipStream_t stream) {
  const int d = c.d;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  size_t off = prep_bytes(n_q, d);
  float* scores = out;
  if (top_k > 0) {
    if (scores == nullptr) scores = reinterpret_cast<float*>(ws + off);
    off += align256((size_t)n_q * n * sizeof(float));
  }
  hipError_t e;
  if (d == 1536) {
    e = launch_wide_scan(c, q, q_dtype, n_q, x, n, scores, workspace, stream);
  } else {
    float* qrot = reinterpret_cast<float*>(ws);
    float* sq = qrot + (size_t)n_q * d;
    e = launch_qprep(c, q, q_dtype, n_q, n_q, RopeHost{}, qrot, sq, stream);
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
  }
  if (e != hipSuccess || top_k == 0) return e;
  const int nch = topk_chunks(n_q, n);
  const size_t cand = (size_t)n_q * nch * top_k;
  float* cval = reinterpret_cast<float*>(ws + off);
  int64_t* cid = reinterpret_cast<int64_t*>(ws + off + align256(cand * sizeof(float)));
  TopKParams t1 = {scores, nullptr, n, (n + nch - 1) / nch, nch, top_k, cval, cid};
  if ((e = run_topk(t1, n_q, stream)) != hipSuccess) return e;
  const int64_t len2 = (int64_t)nch * top_k;
  TopKParams t2 = {cval, cid, len2, len2, 1, top_k, top_scores, top_ids};
  return run_topk(t2, n_q, stream);
}

}  // namespace tqk
