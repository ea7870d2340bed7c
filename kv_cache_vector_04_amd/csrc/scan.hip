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
// Two passes.  Pass 1: one wavefront per (query, chunk of rows) keeps the
// chunk's best k as a sorted list spread over lanes 0..k-1 (descending
// score, ties to the lower row index).  Items stream through in batches; a
// ballot against the list's k-th entry picks the few that can enter, and each
// enters with one wave-wide shift.  Pass 2 runs the same routine over the
// candidates of all chunks of a query.  Lists shorter than k are padded with
// (-inf, INT64_MAX), which every real entry beats.

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

__device__ __forceinline__ int64_t readlane64(int64_t x, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)(uint64_t)x, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)x >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

struct WaveTopK {
  float lv = -INFINITY;          // lane i < k: the i-th best so far
  int64_t li = INT64_MAX;
  float tv = -INFINITY;          // the k-th best (wave-uniform)
  int64_t ti = INT64_MAX;

  // offer one item per lane; the lanes whose item beats the k-th best enter
  // one at a time
  __device__ __forceinline__ void offer(float v, int64_t id, int k, int lane) {
    uint64_t m = __ballot(better(v, id, tv, ti));
    while (m) {
      const int src = __builtin_ctzll(m);
      m &= m - 1;
      const float x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
      const int64_t xi = readlane64(id, src);
      if (!better(x, xi, tv, ti)) continue;            // the bound rose meanwhile
      // entries that beat x form a prefix of the sorted list
      const uint64_t ahead = __ballot(lane < k && better(lv, li, x, xi));
      const int pos = __popcll(ahead);
      const float uv = __shfl_up(lv, 1);
      const int64_t ui = __shfl_up(li, 1);
      if (lane > pos) {
        lv = uv;
        li = ui;
      } else if (lane == pos) {
        lv = x;
        li = xi;
      }
      tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), k - 1));
      ti = readlane64(li, k - 1);
    }
  }
};

template <bool VEC>
__global__ __launch_bounds__(kWave) void topk_kernel(TopKParams p) {
  const int lane = threadIdx.x;
  const int64_t qa = blockIdx.x / p.nchunks;
  const int c = (int)(blockIdx.x % p.nchunks);
  const int64_t beg = (int64_t)c * p.chunk;
  const int64_t end = (beg + p.chunk) < p.len ? (beg + p.chunk) : p.len;
  const float* val = p.val + qa * p.len;
  const int64_t* ids = p.id != nullptr ? p.id + qa * p.len : nullptr;
  const int k = p.k;
  WaveTopK t;
  constexpr int U = 16;
  if constexpr (VEC) {
    // 16-byte aligned rows and chunks: 16 float4 loads (64 items) in flight per lane
    for (int64_t j0 = beg + 4 * lane; j0 < end; j0 += 4 * U * kWave) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + 4 * u * kWave;
        v[u] = j < end ? *reinterpret_cast<const float4*>(val + j)
                       : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + 4 * u * kWave;
        const bool in = j < end;
        t.offer(v[u].x, in ? j : INT64_MAX, k, lane);
        t.offer(v[u].y, in ? j + 1 : INT64_MAX, k, lane);
        t.offer(v[u].z, in ? j + 2 : INT64_MAX, k, lane);
        t.offer(v[u].w, in ? j + 3 : INT64_MAX, k, lane);
      }
    }
  } else {
    for (int64_t j0 = beg + lane; j0 < end; j0 += U * kWave) {
      float v[U];
      int64_t id[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + u * kWave;
        const bool in = j < end;
        v[u] = in ? val[j] : -INFINITY;
        id[u] = in ? (ids != nullptr ? ids[j] : j) : INT64_MAX;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) t.offer(v[u], id[u], k, lane);
    }
  }
  if (lane < k) {
    const int64_t o = ((int64_t)qa * p.nchunks + c) * k + lane;
    p.oval[o] = t.lv;
    p.oid[o] = t.li;
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
  // float4 loads need 16-byte aligned query rows and chunk starts
  const bool vec = t.id == nullptr && t.len % 4 == 0 && t.chunk % 4 == 0 &&
                   ((uintptr_t)t.val % 16) == 0;
  if (vec) hipLaunchKernelGGL((topk_kernel<true>), dim3(blocks), dim3(kWave), 0, s, t);
  else hipLaunchKernelGGL((topk_kernel<false>), dim3(blocks), dim3(kWave), 0, s, t);
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
  const int64_t chunk = ((n + nch - 1) / nch + 3) / 4 * 4;
  TopKParams t1 = {scores, nullptr, n, chunk, nch, top_k, cval, cid};
  if ((e = run_topk(t1, n_q, stream)) != hipSuccess) return e;
  const int64_t len2 = (int64_t)nch * top_k;
  TopKParams t2 = {cval, cid, len2, len2, 1, top_k, top_scores, top_ids};
  return run_topk(t2, n_q, stream);
}

}  // namespace tqk
