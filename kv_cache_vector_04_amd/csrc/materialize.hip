// Materializing decoder: packed codes back to vectors.
//
// "FibQuant", "2.3 Codifica e Decodifica" (decode looks the centroids up,
// rotates back with the shared rotation and rescales by the stored norm);
// "Google presenta TurboQuant", "Eliminación del sesgo interno del producto"
// (TurboQuant_prod adds the 1-bit QJL term to the centroid vector):
//   mse:  x_hat = nu * Pi^T c[idx]
//   prod: x_hat = nu * Pi^T ( c[idx] + sqrt(pi/2)/m * gamma * S^T (2 sigma - 1) )
// with Pi^T w = D (H_d w) / sqrt(d) (H_d symmetric).
//
// Layout as in the two-lanes-per-vector encoder: lane l of a wave owns row
// 32 tile + l%32 and the coordinate half h = l/32 (coordinates
// h d/2 .. h d/2 + d/2 - 1).
// - c[idx] comes from the 16-entry table in LDS.
// - prod: S^T (2 sigma - 1) for the wave's 32 rows is a (d x m) x (m x 32)
//   product on the matrix cores.  The +-1 operand is exact in fp16 (from a
//   256-entry LDS table of 8-sign patterns), S^T is split into fp16 hi + lo
//   (two passes, fp32 accumulation).  k slot j of lane half h at step ks is
//   QJL row (d/2) h + 8 ks + j, i.e. the lane's own sign byte ks; the rows
//   of S^T in the A fragments are ordered so that register v of output tile
//   mt lands, in lane half h, on coordinate (d/2) h + 16 mt + v: the lane's
//   own half.
// - H_d: in-register butterflies over the lane's d/2 coordinates, then the
//   stage across the halves with one v_permlane32_swap per coordinate.
// - D and nu / sqrt(d) in one multiply per coordinate (the sign bit of the
//   scale is set from the flip bit), then fp16 or fp32 stores.

#include <atomic>
#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"

namespace tqk {

constexpr int kMatWaves = 4;

struct MatParams {
  const uint8_t* idx;
  const uint8_t* qjl;
  const float* norm;
  const float* rnorm;
  void* out;
  int64_t out_stride;       // elements between consecutive output rows
  int64_t n_rows;
  float qjl_scale;          // sqrt(pi/2) / m
  float inv_sqrt_d;
  const float* S;           // m x d row-major fp32 (prod)
  float centroids[16];
  uint32_t flip[4];         // bit i%32 of word i/32 set <=> D_i = -1 (d <= 128)
};

// Waves per SIMD the register budget is sized for: d = 128 holds 64 fp32
// coordinates per lane through the butterflies, d = 64 half that.
template <int D>
struct MatLaunch {
  static constexpr int kMinWavesPerEU = D == 128 ? 2 : 4;
};

template <int D, int CB, bool PROD, bool F16>
__global__ __launch_bounds__(kMatWaves * kWave, MatLaunch<D>::kMinWavesPerEU) void materialize_kernel(MatParams p) {
  constexpr int HALF = D / 2;
  constexpr int ROW_BYTES = D * CB / 8;
  constexpr int HB = ROW_BYTES / 2;                 // code bytes of a half row
  constexpr int HW = HB / 4;
  constexpr int HALIGN = HB % 16 == 0 ? 16 : (HB % 8 == 0 ? 8 : 4);
  constexpr int KS = D / 16, MT = D / 32, FRAGS = MT * KS;
  constexpr int QB = HALF / 8;                      // QJL bytes of a half row
  constexpr int QW = QB / 4;

  __shared__ float s_cent[16];
  __shared__ uint4 s_pm[PROD ? 256 : 1];            // 8 signs -> 8 fp16 (+1 / -1)
  __shared__ uint4 s_st[PROD ? FRAGS * 2 * kWave : 1];
  // mse: each wave's 32 output rows staged in LDS (rows padded by 16 bytes)
  // so that a row's bytes are stored in whole 16-byte chunks by consecutive
  // lanes; prod keeps half-row stores (its S fragments fill the LDS)
  constexpr bool STAGE = !PROD;
  constexpr int RBYTES = D * (F16 ? 2 : 4);
  constexpr int PITCH = RBYTES + 16;
  __shared__ __align__(16) unsigned char s_out[STAGE ? kMatWaves : 1][STAGE ? 32 * PITCH : 16];

  const int tid = threadIdx.x;
  const MatParams* kp = (const MatParams*)__builtin_amdgcn_kernarg_segment_ptr();
  if (tid < 16) s_cent[tid] = kp->centroids[tid];
  if constexpr (PROD) {
    for (int b = tid; b < 256; b += blockDim.x) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = ((b >> (2 * j)) & 1) ? 0x3C00u : 0xBC00u;
        const uint32_t hi = ((b >> (2 * j + 1)) & 1) ? 0x3C00u : 0xBC00u;
        w[j] = lo | (hi << 16);
      }
      s_pm[b] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    // fragment (mt, ks), lane l: row sigma = (d/2) ((l/4)%2) + 16 mt +
    // 4 ((l%32)/8) + l%4 of S^T, columns (QJL rows) (d/2) (l/32) + 8 ks + j
    for (int t = tid; t < FRAGS * kWave; t += blockDim.x) {
      const int lane = t & 63, f = t >> 6;
      const int mt = f / KS, ks = f % KS;
      const int rho = lane & 31;
      const int sig = HALF * ((rho >> 2) & 1) + 16 * mt + 4 * (rho >> 3) + (rho & 3);
      const int pi0 = HALF * (lane >> 5) + 8 * ks;
      _Float16 hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = p.S[(size_t)(pi0 + j) * D + sig];
        hi[j] = (_Float16)v;
        lo[j] = (_Float16)(v - (float)hi[j]);
      }
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wh[j] = (uint32_t)__builtin_bit_cast(uint16_t, hi[2 * j]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, hi[2 * j + 1]) << 16);
        wl[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo[2 * j]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, lo[2 * j + 1]) << 16);
      }
      s_st[(2 * f) * kWave + lane] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
      s_st[(2 * f + 1) * kWave + lane] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int64_t ntiles = (p.n_rows + 31) / 32;
  const int64_t tstride = (int64_t)gridDim.x * kMatWaves;
  // this lane's flip bits: coordinates (d/2) h .. (d/2) h + d/2 - 1
  uint32_t fl[HALF / 32 > 0 ? HALF / 32 : 1];
#pragma unroll
  for (int j = 0; j < (HALF / 32 > 0 ? HALF / 32 : 1); ++j) fl[j] = kp->flip[(HALF * h) / 32 + j];

  for (int64_t tile = (int64_t)blockIdx.x * kMatWaves + wave; tile < ntiles; tile += tstride) {
    int64_t row = tile * 32 + (lane & 31);
    const bool valid = row < p.n_rows;
    if (!valid) row = p.n_rows - 1;     // a lane's row only reaches its own product column

    // w = sqrt(pi/2)/m gamma S^T (2 sigma - 1) (prod) + c[idx]
    float w[HALF];
    if constexpr (PROD) {
      uint32_t qw[QW > 0 ? QW : 1];
      load_words<(QW > 0 ? QW : 1), (QB % 8 == 0 ? 8 : 4)>(p.qjl + row * (D / 8) + h * QB, qw);
      const float g = p.rnorm[row] * p.qjl_scale;
      f32x16 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t byte = (qw[ks >> 2] >> (8 * (ks & 3))) & 255u;
        const half8_t b = __builtin_bit_cast(half8_t, s_pm[byte]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int f = mt * KS + ks;
          const half8_t ah = __builtin_bit_cast(half8_t, s_st[(2 * f) * kWave + lane]);
          const half8_t al = __builtin_bit_cast(half8_t, s_st[(2 * f + 1) * kWave + lane]);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, b, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, b, acc[mt], 0, 0, 0);
        }
        // bounds the fragment registers in flight to one step's
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) w[16 * mt + v] = g * acc[mt][v];
    } else {
#pragma unroll
      for (int i = 0; i < HALF; ++i) w[i] = 0.f;
    }
    uint32_t cw[HW];
    load_words<HW, HALIGN>(p.idx + row * ROW_BYTES + h * HB, cw);
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const int off = i * CB, wd = off >> 5, sh = off & 31;
      uint32_t c = cw[wd] >> sh;
      if (sh + CB > 32) c |= cw[wd + 1] << (32 - sh);
      w[i] += s_cent[c & ((1u << CB) - 1u)];
      // bounds the table reads in flight
      if ((i & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
    // H_d: stages inside the lane, then the stage across the halves
#pragma unroll
    for (int hh = 1; hh < HALF; hh <<= 1) {
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        if ((i & hh) == 0) {
          const float a = w[i], b = w[i + hh];
          w[i] = a + b;
          w[i + hh] = a - b;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // across the halves: one swap of (w[i], w[i]) gives every lane the low
    // lane's value in a and the high lane's in b; y = a + b (low), a - b (high)
    const float sgn = h ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      uint32_t a = __float_as_uint(w[i]), b = a;
      swap_halves(a, b);
      w[i] = fmaf(sgn, __uint_as_float(b), __uint_as_float(a));
      // bounds the exchanged values in flight
      if ((i & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
    // D and nu / sqrt(d): the scale is >= 0, its sign bit becomes the flip bit
    const float sc = p.norm[row] * p.inv_sqrt_d;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const uint32_t fb = fl[i >> 5] << (31 - (i & 31));
      w[i] *= __uint_as_float((fb & 0x80000000u) | __float_as_uint(sc));
    }
    if constexpr (STAGE) {
      unsigned char* stage = s_out[wave];
      uint4* sdst = reinterpret_cast<uint4*>(stage + (lane & 31) * PITCH + h * (RBYTES / 2));
      if constexpr (F16) {
#pragma unroll
        for (int q = 0; q < HALF / 8; ++q) {
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w[8 * q + 2 * j], w[8 * q + 2 * j + 1]));
          sdst[q] = make_uint4(o[0], o[1], o[2], o[3]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < HALF / 4; ++q)
          sdst[q] = make_uint4(__float_as_uint(w[4 * q]), __float_as_uint(w[4 * q + 1]),
                               __float_as_uint(w[4 * q + 2]), __float_as_uint(w[4 * q + 3]));
      }
      // LDS operations of one wave complete in order: no workgroup barrier
      __builtin_amdgcn_wave_barrier();
      constexpr int CPR = RBYTES / 16;                      // 16-byte chunks per row
      const int64_t row0 = tile * 32;
      const int64_t rows = (p.n_rows - row0) < 32 ? (p.n_rows - row0) : 32;
      const int64_t pitch_out = p.out_stride * (F16 ? 2 : 4);
      unsigned char* gout = reinterpret_cast<unsigned char*>(p.out) + row0 * pitch_out;
#pragma unroll
      for (int k = 0; k < 32 * CPR / kWave; ++k) {
        const int c = lane + kWave * k;
        const int r = c / CPR, col = c % CPR;
        if (r < rows)
          *reinterpret_cast<uint4*>(gout + r * pitch_out + col * 16) =
              *reinterpret_cast<const uint4*>(stage + r * PITCH + col * 16);
      }
      __builtin_amdgcn_wave_barrier();
    } else if (valid) {
      if constexpr (F16) {
        _Float16* dst = reinterpret_cast<_Float16*>(p.out) + row * p.out_stride + h * HALF;
#pragma unroll
        for (int q = 0; q < HALF / 8; ++q) {
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w[8 * q + 2 * j], w[8 * q + 2 * j + 1]));
          reinterpret_cast<uint4*>(dst)[q] = make_uint4(o[0], o[1], o[2], o[3]);
        }
      } else {
        float* dst = reinterpret_cast<float*>(p.out) + row * p.out_stride + h * HALF;
#pragma unroll
        for (int q = 0; q < HALF / 4; ++q)
          reinterpret_cast<float4*>(dst)[q] = make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
      }
    }
  }
}

template <int D, int CB, bool PROD, bool F16>
static hipError_t run_mat(const MatParams& p, hipStream_t stream) {
  // occupancy depends only on the kernel's resources (one code object for
  // every device): computed once, read by any host thread
  static std::atomic<int> per_cu{0};
  if (per_cu.load(std::memory_order_relaxed) == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, materialize_kernel<D, CB, PROD, F16>,
                                                     kMatWaves * kWave, 0) != hipSuccess || nb < 1)
      nb = 1;
    per_cu.store(nb, std::memory_order_relaxed);
  }
  const int64_t ntiles = (p.n_rows + 31) / 32;
  int64_t blocks = (ntiles + kMatWaves - 1) / kMatWaves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu.load(std::memory_order_relaxed);
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((materialize_kernel<D, CB, PROD, F16>), dim3((unsigned)blocks),
                     dim3(kMatWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool PROD, bool F16>
static hipError_t pick_mat(int cb, const MatParams& p, hipStream_t s) {
  switch (cb) {
    case 1: return run_mat<D, 1, PROD, F16>(p, s);
    case 2: return run_mat<D, 2, PROD, F16>(p, s);
    case 3: return run_mat<D, 3, PROD, F16>(p, s);
    case 4: return run_mat<D, 4, PROD, F16>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t pick_mat_d(const tq_codec& c, bool f16, const MatParams& p, hipStream_t s) {
  const bool prod = c.mode == TQ_PROD;
  if (prod) return f16 ? pick_mat<D, true, true>(c.code_bits, p, s) : pick_mat<D, true, false>(c.code_bits, p, s);
  return f16 ? pick_mat<D, false, true>(c.code_bits, p, s) : pick_mat<D, false, false>(c.code_bits, p, s);
}

hipError_t launch_materialize(const tq_codec& c, const tq_packed& in, int64_t n_rows, void* out,
                              int out_dtype, hipStream_t stream, int64_t out_stride) {
  if (n_rows == 0) return hipSuccess;
  MatParams p = {};
  p.idx = in.idx;
  p.qjl = in.qjl;
  p.norm = in.norm;
  p.rnorm = in.rnorm;
  p.out = out;
  p.out_stride = out_stride > 0 ? out_stride : c.d;
  p.n_rows = n_rows;
  p.qjl_scale = c.m > 0 ? (float)(std::sqrt(M_PI / 2.0) / c.m) : 0.f;
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)c.d));
  p.S = c.S;
  for (int k = 0; k < 16; ++k) p.centroids[k] = c.centroids[k];
  for (int w = 0; w < 4; ++w) p.flip[w] = c.flip[w];
  const bool f16 = out_dtype == TQ_F16;
  if (c.d == 128) return pick_mat_d<128>(c, f16, p, stream);
  if (c.d == 64) return pick_mat_d<64>(c, f16, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace tqk
