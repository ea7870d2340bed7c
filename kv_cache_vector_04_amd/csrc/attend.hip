// Attention straight from packed codes, d = 64 or 128 ("TurboESM", "2.
// Metodologia" part E: unpack, correct, attend with an online softmax in one
// pass with no dequantized copy in memory; "FibQuant", "5. Significato e
// Affermazioni": fixed addresses make that fusion possible).
//
// For query row r (batch b, query head h, query a; KV head g = h / G):
//   s_j = scale * nu_j * ( <q_rot, c_K[idx_j]> + sqrt(pi/2)/m gamma_j <Sq, 2 sigma_j - 1> )
//   acc = sum_j softmax(s)_j nu^V_j c_V[idx^V_j]      (rotated domain)
//   o   = Pi_V^T acc = D_V * H_d acc / sqrt(d)           (once per row)
// The inverse rotation is applied once to the weighted sum instead of to
// every token (linearity), and the query is rotated instead of the keys.
//
// Work split: a workgroup owns one (batch, KV head), a chunk of up to 16
// query rows of that KV head, and one token range; it scans the range in
// tiles of 256 tokens (one token per thread for the scores, a (row,
// 8-coordinate group) per thread for the value sum) with a running max and
// sum per row, and writes (acc, max, sum).  A second kernel merges the
// ranges by log-sum-exp and applies Pi_V^T.

#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"
#include "qprep.hpp"

namespace tqk {

constexpr int kAttTile = 256;
constexpr int kAttRows = 16;

struct AttendParams {
  const uint8_t* kidx;
  const uint8_t* kqjl;
  const float* knorm;
  const float* krnorm;
  const uint8_t* vidx;
  const float* vnorm;
  const float* qrot;      // [rows][D]
  const float* sq;        // [rows][D]
  float* part;            // partial records
  float* scores_out;      // optional [rows][ctx]
  int64_t ctx;
  int batch, hq, hkv, n_q, G;
  int nchunks, splits;
  int64_t split_len;
  float scale;
  float qjl_scale;
  float kcent[16];
  float vcent[16];
};

template <int D>
struct PartRec {
  static constexpr int FLOATS = D + 2;   // acc[D], max, sum
};

template <int D, int CBK, int CBV>
__global__ __launch_bounds__(kAttTile) void attend_kernel(AttendParams p) {
  constexpr int WK = D * CBK / 32;
  constexpr int WV = D * CBV / 32;
  constexpr int KROW = D * CBK / 8;
  constexpr int VROW = D * CBV / 8;
  constexpr int KALIGN = KROW % 16 == 0 ? 16 : 8;
  constexpr int VALIGN = VROW % 16 == 0 ? 16 : 8;
  constexpr int CG = D / 8;               // 8-coordinate groups per row
  constexpr int RPT = kAttTile / CG;      // rows covered per pass of the value sum

  __shared__ float s_kc[16], s_vc[16];
  __shared__ float s_q[kAttRows][D];
  __shared__ float s_s[kAttRows][D];
  __shared__ float s_tot[kAttRows];
  __shared__ float s_w[kAttRows][kAttTile];
  __shared__ uint32_t s_vcode[kAttTile][WV + 1];
  __shared__ float s_m[kAttRows], s_l[kAttRows], s_alpha[kAttRows];

  const int tid = threadIdx.x;
  const int bg = blockIdx.x / p.nchunks;
  const int chunk = blockIdx.x % p.nchunks;
  const int split = blockIdx.y;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int qr_total = p.G * p.n_q;
  const int lr0 = chunk * kAttRows;
  const int nrows = (qr_total - lr0) < kAttRows ? (qr_total - lr0) : kAttRows;
  const int64_t row_base = ((int64_t)b * p.hq + (int64_t)g * p.G) * p.n_q + lr0;

#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (tid == k) { s_kc[k] = p.kcent[k]; s_vc[k] = p.vcent[k]; }
  for (int t = tid; t < kAttRows * D; t += kAttTile) {
    const int r = t / D, i = t % D;
    s_q[r][i] = r < nrows ? p.qrot[(row_base + r) * D + i] : 0.f;
    s_s[r][i] = r < nrows ? p.sq[(row_base + r) * D + i] : 0.f;
  }
  if (tid < kAttRows) { s_m[tid] = -INFINITY; s_l[tid] = 0.f; }
  __syncthreads();
  if (tid < kAttRows) {
    float t = 0.f;
    for (int i = 0; i < D; ++i) t += s_s[tid][i];
    s_tot[tid] = t;
  }

  const int64_t t0 = (int64_t)split * p.split_len;
  int64_t t1 = t0 + p.split_len;
  if (t1 > p.ctx) t1 = p.ctx;
  const int64_t kv_base = (int64_t)bg * p.ctx;

  // value-sum ownership: row vr, coordinates 8 cg .. 8 cg + 7
  const int vr_base = tid / CG;
  const int cg = tid % CG;
  float acc[(kAttRows + RPT - 1) / RPT][8];
#pragma unroll
  for (int u = 0; u < (kAttRows + RPT - 1) / RPT; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;

  for (int64_t tile0 = t0; tile0 < t1; tile0 += kAttTile) {
    const int64_t tok = tile0 + tid;
    const bool valid = tok < t1;
    __syncthreads();   // previous tile's weights and codes are consumed
    // ---- scores, one token per thread ----
    if (valid) {
      const int64_t kr = kv_base + tok;
      uint32_t kw[WK];
      load_words<WK, KALIGN>(p.kidx + kr * KROW, kw);
      float c[D];
#pragma unroll
      for (int i = 0; i < D; ++i) c[i] = s_kc[get_code<CBK, WK>(kw, i)];
      uint32_t sb[D / 32];
      load_words<D / 32, (D / 8) % 16 == 0 ? 16 : 8>(p.kqjl + kr * (D / 8), sb);
      const float nu = p.knorm[kr] * p.scale;
      const float gk = p.krnorm[kr] * p.qjl_scale;
      uint32_t vw[WV];
      load_words<WV, VALIGN>(p.vidx + kr * VROW, vw);
#pragma unroll
      for (int j = 0; j < WV; ++j) s_vcode[tid][j] = vw[j];
      s_vcode[tid][WV] = __float_as_uint(p.vnorm[kr]);
      for (int r = 0; r < nrows; ++r) {
        float m0 = 0.f, m1 = 0.f, ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int i = 0; i < D; i += 2) {
          m0 = fmaf(c[i], s_q[r][i], m0);
          m1 = fmaf(c[i + 1], s_q[r][i + 1], m1);
          ps0 += ((sb[i >> 5] >> (i & 31)) & 1u) ? s_s[r][i] : 0.f;
          ps1 += ((sb[(i + 1) >> 5] >> ((i + 1) & 31)) & 1u) ? s_s[r][i + 1] : 0.f;
        }
        const float s = nu * fmaf(gk, 2.f * (ps0 + ps1) - s_tot[r], m0 + m1);
        s_w[r][tid] = s;
        if (p.scores_out) p.scores_out[(row_base + r) * p.ctx + tok] = s;
      }
    } else {
      for (int r = 0; r < nrows; ++r) s_w[r][tid] = -INFINITY;
      s_vcode[tid][WV] = 0u;
    }
    __syncthreads();
    // ---- online softmax: one wave per row at a time ----
    const int wave = tid >> 6, lane = tid & 63;
    for (int r = wave; r < nrows; r += kAttTile / kWave) {
      float mx = -INFINITY;
      for (int j = lane; j < kAttTile; j += kWave) mx = fmaxf(mx, s_w[r][j]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_old = s_m[r];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
      for (int j = lane; j < kAttTile; j += kWave) {
        const float e = expf(s_w[r][j] - m_new);
        sum += e;
        s_w[r][j] = e * __uint_as_float(s_vcode[j][WV]);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
      if (lane == 0) {
        const float alpha = expf(m_old - m_new);
        s_alpha[r] = alpha;
        s_l[r] = s_l[r] * alpha + sum;
        s_m[r] = m_new;
      }
    }
    __syncthreads();
    // ---- value sum, (row, 8 coordinates) per thread ----
    const int ntok = (int)((t1 - tile0) < kAttTile ? (t1 - tile0) : kAttTile);
#pragma unroll
    for (int u = 0; u < (kAttRows + RPT - 1) / RPT; ++u) {
      const int vr = vr_base + u * RPT;
      if (vr >= nrows) continue;
      const float alpha = s_alpha[vr];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] *= alpha;
      for (int j = 0; j < ntok; ++j) {
        const float w = s_w[vr][j];
        const int off0 = 8 * cg * CBV;
        const int word = off0 >> 5, sh = off0 & 31;
        uint64_t bits = s_vcode[j][word];
        if (word + 1 < WV) bits |= (uint64_t)s_vcode[j][word + 1] << 32;
        bits >>= sh;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t code = (uint32_t)(bits >> (e * CBV)) & ((1u << CBV) - 1u);
          acc[u][e] = fmaf(w, s_vc[code], acc[u][e]);
        }
      }
    }
  }
  // ---- partial record ----
  const int64_t rec0 = (((int64_t)bg * p.nchunks + chunk) * p.splits + split) * kAttRows;
#pragma unroll
  for (int u = 0; u < (kAttRows + RPT - 1) / RPT; ++u) {
    const int vr = vr_base + u * RPT;
    if (vr >= nrows) continue;
    float* rec = p.part + (rec0 + vr) * PartRec<D>::FLOATS;
#pragma unroll
    for (int e = 0; e < 8; ++e) rec[8 * cg + e] = acc[u][e];
    if (cg == 0) {
      rec[D] = s_m[vr];
      rec[D + 1] = s_l[vr];
    }
  }
}

struct CombineParams {
  const float* part;
  float* out;
  int hq, hkv, n_q, G, nchunks, splits;
  uint32_t flip[48];
  float inv_sqrt_d;
};

// Merge the token ranges of one query row by log-sum-exp, then o = Pi_V^T a.
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(CombineParams p) {
  __shared__ float s_v[D];
  const int i = threadIdx.x;
  const int64_t row = blockIdx.x;                 // (b, h, a)
  const int a = (int)(row % p.n_q);
  const int64_t bh = row / p.n_q;
  const int h = (int)(bh % p.hq);
  const int b = (int)(bh / p.hq);
  const int g = h / p.G;
  const int lr = (h - g * p.G) * p.n_q + a;
  const int chunk = lr / kAttRows, r = lr % kAttRows;
  const int64_t bg = (int64_t)b * p.hkv + g;
  const int64_t rec0 = ((bg * p.nchunks + chunk) * p.splits) * kAttRows + r;
  float M = -INFINITY;
  for (int s = 0; s < p.splits; ++s)
    M = fmaxf(M, p.part[(rec0 + (int64_t)s * kAttRows) * PartRec<D>::FLOATS + D]);
  float L = 0.f, v = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float* rec = p.part + (rec0 + (int64_t)s * kAttRows) * PartRec<D>::FLOATS;
    const float f = expf(rec[D] - M);
    L = fmaf(rec[D + 1], f, L);
    v = fmaf(rec[i], f, v);
  }
  v /= L;
  // inverse rotation: D * (H v) / sqrt(d)
#pragma unroll
  for (int hh = 1; hh < D; hh <<= 1) {
    s_v[i] = v;
    __syncthreads();
    const float o = s_v[i ^ hh];
    v = (i & hh) ? (o - v) : (v + o);
    __syncthreads();
  }
  const uint32_t bit = (p.flip[i >> 5] >> (i & 31)) & 1u;
  v *= p.inv_sqrt_d;
  p.out[row * D + i] = bit ? -v : v;
}

static void plan(int batch, int n_q, int hq, int hkv, int64_t ctx, int& nchunks, int& splits,
                 int64_t& split_len) {
  const int G = hq / hkv;
  nchunks = (G * n_q + kAttRows - 1) / kAttRows;
  const int64_t groups = (int64_t)batch * hkv * nchunks;
  const int64_t max_split = (ctx + kAttTile - 1) / kAttTile;
  int64_t want = (1024 + groups - 1) / groups;
  if (want > max_split) want = max_split;
  if (want < 1) want = 1;
  split_len = ((ctx + want - 1) / want + kAttTile - 1) / kAttTile * kAttTile;
  splits = (int)((ctx + split_len - 1) / split_len);
}

size_t attend_workspace_bytes(int batch, int n_q, int hq, int hkv, int64_t ctx, int d) {
  if (decode_path(n_q, hq, hkv)) return decode_workspace_bytes(batch, n_q, hq, hkv, ctx, d);
  if (mq_path(n_q, hq, hkv, d)) return mq_workspace_bytes(batch, n_q, hq);
  int nchunks, splits;
  int64_t split_len;
  plan(batch, n_q, hq, hkv, ctx, nchunks, splits, split_len);
  const size_t rows = (size_t)batch * hq * n_q;
  size_t b = rows * d * 2 * sizeof(float);
  b = (b + 255) & ~(size_t)255;
  b += (size_t)batch * hkv * nchunks * splits * kAttRows * (d + 2) * sizeof(float);
  return b;
}

template <int D, int CBK, int CBV>
static hipError_t run_attend(const AttendParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((attend_kernel<D, CBK, CBV>), grid, dim3(kAttTile), 0, s, p);
  return hipGetLastError();
}

template <int D, int CBK>
static hipError_t pick_v(int cbv, const AttendParams& p, dim3 grid, hipStream_t s) {
  switch (cbv) {
    case 1: return run_attend<D, CBK, 1>(p, grid, s);
    case 2: return run_attend<D, CBK, 2>(p, grid, s);
    case 3: return run_attend<D, CBK, 3>(p, grid, s);
    case 4: return run_attend<D, CBK, 4>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t pick_k(int cbk, int cbv, const AttendParams& p, dim3 grid, hipStream_t s) {
  switch (cbk) {
    case 1: return pick_v<D, 1>(cbv, p, grid, s);
    case 2: return pick_v<D, 2>(cbv, p, grid, s);
    case 3: return pick_v<D, 3>(cbv, p, grid, s);
    case 4: return pick_v<D, 4>(cbv, p, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attend(const tq_codec& kc, const tq_codec& vc, const void* q, int q_dtype,
                         int batch, int n_q, int hq, int hkv, const RopeHost& rope,
                         const tq_packed& k, const tq_packed& v, int64_t ctx, float scale,
                         float* out, float* scores_out, void* workspace, hipStream_t stream) {
  if (decode_path(n_q, hq, hkv))
    return launch_decode(kc, vc, q, q_dtype, batch, n_q, hq, hkv, rope, k, v, ctx, scale, out,
                         scores_out, workspace, stream);
  if (mq_path(n_q, hq, hkv, kc.d))
    return launch_attend_mq(kc, vc, q, q_dtype, batch, n_q, hq, hkv, rope, k, v, ctx, scale, out,
                            scores_out, workspace, stream);
  const int d = kc.d;
  int nchunks, splits;
  int64_t split_len;
  plan(batch, n_q, hq, hkv, ctx, nchunks, splits, split_len);
  const int64_t rows = (int64_t)batch * hq * n_q;
  float* qrot = reinterpret_cast<float*>(workspace);
  float* sq = qrot + (size_t)rows * d;
  const size_t off = ((size_t)rows * d * 2 * sizeof(float) + 255) & ~(size_t)255;
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(workspace) + off);
  hipError_t e = launch_qprep(kc, q, q_dtype, rows, n_q, rope, qrot, sq, stream);
  if (e != hipSuccess) return e;
  AttendParams p = {};
  p.kidx = k.idx; p.kqjl = k.qjl; p.knorm = k.norm; p.krnorm = k.rnorm;
  p.vidx = v.idx; p.vnorm = v.norm;
  p.qrot = qrot; p.sq = sq; p.part = part; p.scores_out = scores_out;
  p.ctx = ctx; p.batch = batch; p.hq = hq; p.hkv = hkv; p.n_q = n_q; p.G = hq / hkv;
  p.nchunks = nchunks; p.splits = splits; p.split_len = split_len;
  p.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)d));
  p.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / kc.m);
  for (int i = 0; i < 16; ++i) { p.kcent[i] = kc.centroids[i]; p.vcent[i] = vc.centroids[i]; }
  const dim3 grid((unsigned)((int64_t)batch * hkv * nchunks), (unsigned)splits);
  if (d == 128) e = pick_k<128>(kc.code_bits, vc.code_bits, p, grid, stream);
  else if (d == 64) e = pick_k<64>(kc.code_bits, vc.code_bits, p, grid, stream);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  CombineParams cp = {};
  cp.part = part; cp.out = out; cp.hq = hq; cp.hkv = hkv; cp.n_q = n_q; cp.G = hq / hkv;
  cp.nchunks = nchunks; cp.splits = splits;
  for (int w = 0; w < 48; ++w) cp.flip[w] = vc.flip[w];
  cp.inv_sqrt_d = (float)(1.0 / std::sqrt((double)d));
  if (d == 128)
    hipLaunchKernelGGL((combine_kernel<128>), dim3((unsigned)rows), dim3(128), 0, stream, cp);
  else
    hipLaunchKernelGGL((combine_kernel<64>), dim3((unsigned)rows), dim3(64), 0, stream, cp);
  return hipGetLastError();
}

}  // namespace tqk
