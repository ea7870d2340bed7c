// FibQuant k = 2 on the GPU: encode rows to 2-coordinate block codes and
// decode them back ("FibQuant", "2.3 Codifica e Decodifica").
//
// Both kernels use the two-lanes-per-vector layout: lane l of a wave owns
// row 32 tile + l%32 and the coordinate half h = l/32 (coordinates
// h d/2 .. h d/2 + d/2 - 1, blocks h d/4 .. h d/4 + d/4 - 1).
//
// Encode: nu^2 from the lane's half plus one exchange; D, then H_d as
// butterflies over the lane's coordinates and one v_permlane32_swap per
// coordinate for the stage across the halves; z = y / (sqrt(d) nu).  The
// nearest codeword of block (z_2j, z_2j+1) maximizes <y, c_n> - |c_n|^2 / 2
// (ties keep the lower n).  The codewords are lane-uniform: they stream from
// the kernel arguments through scalar loads, with no LDS.
// Decode: codewords from an LDS copy of the table, then the same
// butterflies, D and nu / sqrt(d).
//
// A lane's half row holds (d/4) log2(N) bits: whole 32-bit words at d = 128,
// whole 16-bit units at d = 64 (its start is only 2-byte aligned for odd
// log2 N), so the store and load unit is chosen per shape.

#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"

namespace tqk {

constexpr int kVqWaves = 4;

struct VqParams {
  const void* x;
  uint8_t* idx;
  float* norm;
  void* out;
  const uint8_t* idx_in;
  const float* norm_in;
  const uint8_t* search;            // TQ_VQ_SEARCH_BYTES table or null
  int64_t n_rows;
  float inv_sqrt_d;
  uint32_t flip[4];
  float codewords[2 * TQ_VQ_MAX_CODES];
  float half_sq[TQ_VQ_MAX_CODES];   // -|c_n|^2 / 2
};
static_assert(sizeof(VqParams) <= 4096, "kernel argument segment");

// the lane's half row of block codes: HB bytes in 32-bit words (HB % 4 == 0)
// or 16-bit units
template <int HB>
struct HalfRowIO {
  static constexpr bool kWords = HB % 4 == 0;
  static constexpr int kUnits = kWords ? HB / 4 : HB / 2;
  static constexpr int kUnitBits = kWords ? 32 : 16;
};

template <int HB>
__device__ __forceinline__ void store_half_row(uint8_t* dst, const uint32_t (&bits)[(HB + 3) / 4]) {
  using IO = HalfRowIO<HB>;
  if constexpr (IO::kWords) {
#pragma unroll
    for (int j = 0; j < IO::kUnits; ++j) reinterpret_cast<uint32_t*>(dst)[j] = bits[j];
  } else {
#pragma unroll
    for (int j = 0; j < IO::kUnits; ++j)
      reinterpret_cast<uint16_t*>(dst)[j] = (uint16_t)(bits[j >> 1] >> (16 * (j & 1)));
  }
}

template <int HB>
__device__ __forceinline__ void load_half_row(const uint8_t* src, uint32_t (&bits)[(HB + 3) / 4]) {
  using IO = HalfRowIO<HB>;
#pragma unroll
  for (int j = 0; j < (HB + 3) / 4; ++j) bits[j] = 0u;
  if constexpr (IO::kWords) {
#pragma unroll
    for (int j = 0; j < IO::kUnits; ++j) bits[j] = reinterpret_cast<const uint32_t*>(src)[j];
  } else {
#pragma unroll
    for (int j = 0; j < IO::kUnits; ++j)
      bits[j >> 1] |= (uint32_t)reinterpret_cast<const uint16_t*>(src)[j] << (16 * (j & 1));
  }
}

// H_d over the two lanes of a row: in-lane stages, then across the halves
template <int HALF>
__device__ __forceinline__ void wht_two_lanes(float (&w)[HALF], int h) {
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
  const float sgn = h ? -1.f : 1.f;
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    // one swap of (w[i], w[i]) gives every lane the low lane's value in a
    // and the high lane's in b
    uint32_t a = __float_as_uint(w[i]), b = a;
    swap_halves(a, b);
    w[i] = fmaf(sgn, __uint_as_float(b), __uint_as_float(a));
    if ((i & 15) == 15) __builtin_amdgcn_sched_barrier(0);
  }
}

constexpr int kGrid = TQ_VQ_GRID;
constexpr int kOffsets = kGrid * kGrid + 8;                     // uint16 cell offsets
constexpr int kTableBytes = 2 * kOffsets + TQ_VQ_ENTRIES;      // after the 16-byte header
static_assert(kTableBytes % 16 == 0 && TQ_VQ_SEARCH_BYTES == 16 + kTableBytes, "search table layout");

template <int D, int B, typename T>
__global__ __launch_bounds__(kVqWaves * kWave, 2) void encode_vq_kernel(VqParams p) {
  constexpr int HALF = D / 2, NBK = HALF / 2, N = 1 << B;
  constexpr int HB = NBK * B / 8;
  constexpr int RB = 2 * HB;                         // bytes per row
  constexpr int HWD = (HB + 3) / 4;
  const VqParams* kp = (const VqParams*)__builtin_amdgcn_kernarg_segment_ptr();
  // grid search: the table and the codewords in LDS
  __shared__ uint4 s_tab[kTableBytes / 16];
  __shared__ float4 s_cw[N];             // (x, y, -|c|^2 / 2, 0)
  const bool grid = p.search != nullptr;
  float grid_a = 1.f, grid_half = 0.f;
  if (grid) {
    const uint4* src = reinterpret_cast<const uint4*>(p.search + 16);
    for (int i = threadIdx.x; i < kTableBytes / 16; i += blockDim.x) s_tab[i] = src[i];
    for (int n = threadIdx.x; n < N; n += blockDim.x)
      s_cw[n] = make_float4(kp->codewords[2 * n], kp->codewords[2 * n + 1], kp->half_sq[n], 0.f);
    grid_a = reinterpret_cast<const float*>(p.search)[0];
    grid_half = reinterpret_cast<const float*>(p.search)[1];
    __syncthreads();
  }
  const uint16_t* s_off = reinterpret_cast<const uint16_t*>(s_tab);
  const uint8_t* s_pool = reinterpret_cast<const uint8_t*>(s_off + kOffsets);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int64_t ntiles = (p.n_rows + 31) / 32;
  uint32_t fl[HALF / 32 > 0 ? HALF / 32 : 1];
#pragma unroll
  for (int j = 0; j < (HALF / 32 > 0 ? HALF / 32 : 1); ++j) fl[j] = kp->flip[(HALF * h) / 32 + j];

  for (int64_t tile = (int64_t)blockIdx.x * kVqWaves + wave; tile < ntiles;
       tile += (int64_t)gridDim.x * kVqWaves) {
    int64_t row = tile * 32 + (lane & 31);
    const bool valid = row < p.n_rows;
    if (!valid) row = p.n_rows - 1;     // a lane's row reaches only its own outputs
    float w[HALF];
    const T* src = reinterpret_cast<const T*>(p.x) + row * D + h * HALF;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int q = 0; q < HALF / 8; ++q) {
        const uint4 u = reinterpret_cast<const uint4*>(src)[q];
        const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[8 * q + 2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(uw[e] & 0xFFFFu));
          w[8 * q + 2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(uw[e] >> 16));
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < HALF / 4; ++q) {
        const float4 u = reinterpret_cast<const float4*>(src)[q];
        w[4 * q] = u.x; w[4 * q + 1] = u.y; w[4 * q + 2] = u.z; w[4 * q + 3] = u.w;
      }
    }
    float s2 = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) s2 = fmaf(w[i], w[i], s2);
    uint32_t sa = __float_as_uint(s2), sb = sa;
    swap_halves(sa, sb);
    const float nu2 = __uint_as_float(sa) + __uint_as_float(sb);
    const bool finite = nu2 <= 3.0e38f;
    const float nu = sqrtf(nu2);
    const float inv = (finite && nu > 0.f) ? p.inv_sqrt_d / nu : 0.f;
    // D (sign bit from the flip bit), then H_d
#pragma unroll
    for (int i = 0; i < HALF; ++i)
      w[i] = __uint_as_float(__float_as_uint(w[i]) ^ ((fl[i >> 5] << (31 - (i & 31))) & 0x80000000u));
    wht_two_lanes<HALF>(w, h);
    // a non-finite row becomes z = 0 (inf * 0 would be NaN)
#pragma unroll
    for (int i = 0; i < HALF; ++i) w[i] = finite ? w[i] * inv : 0.f;
    // nearest codeword per block: argmax <y, c_n> - |c_n|^2 / 2, ties to
    // the lower n (strict improvement in ascending order); codes packed
    // LSB-first at B bits
    uint32_t bits[HWD];
#pragma unroll
    for (int j = 0; j < HWD; ++j) bits[j] = 0u;
    auto put = [&](int j, int code) {
      const int off = j * B, wd = off >> 5, sh = off & 31;
      bits[wd] |= (uint32_t)code << sh;
      if (sh + B > 32) bits[wd + 1] |= (uint32_t)code >> (32 - sh);
    };
    if (grid) {
      // the block's cell (companded coordinates u = x / (|x| + a), uniform
      // grid over u) lists every codeword that can win there; an empty list:
      // test all
      auto axis = [&](float x) {
        const float t = (x * __builtin_amdgcn_rcpf(fabsf(x) + grid_a) + 1.f) * grid_half;
        return (int)fminf(fmaxf(t, 0.f), (float)(kGrid - 1));
      };
      // IL blocks at a time: IL independent chains of LDS reads in flight.
      // With long lists (N >= 128) one at a time: the loop runs to the
      // longest of the IL lists.
      constexpr int IL = B >= 7 ? 1 : 4;
      static_assert(NBK % IL == 0, "blocks per lane");
#pragma unroll
      for (int j0 = 0; j0 < NBK; j0 += IL) {
        int beg[IL], cnt[IL], best[IL];
        float bs[IL];
        int iters = 0;
#pragma unroll
        for (int q = 0; q < IL; ++q) {
          const int cell = axis(w[2 * (j0 + q) + 1]) * kGrid + axis(w[2 * (j0 + q)]);
          beg[q] = s_off[cell];
          const int c = (int)s_off[cell + 1] - beg[q];
          cnt[q] = c == 0 ? N : c;               // an empty list: all codewords
          beg[q] = c == 0 ? -1 : beg[q];
          iters = max(iters, cnt[q]);
          bs[q] = -INFINITY;
          best[q] = 0;
        }
        for (int i = 0; i < iters; ++i) {
#pragma unroll
          for (int q = 0; q < IL; ++q) {
            const bool on = i < cnt[q];
            const int n = beg[q] < 0 ? i : (int)s_pool[beg[q] + (on ? i : 0)];
            const float4 c = s_cw[n & (N - 1)];
            const float sc = fmaf(w[2 * (j0 + q) + 1], c.y, fmaf(w[2 * (j0 + q)], c.x, c.z));
            const bool up = on && sc > bs[q];
            bs[q] = up ? sc : bs[q];
            best[q] = up ? n : best[q];
          }
        }
#pragma unroll
        for (int q = 0; q < IL; ++q) put(j0 + q, best[q]);
      }
    } else {
      int best[NBK];
      float bs[NBK];
#pragma unroll
      for (int j = 0; j < NBK; ++j) {
        best[j] = 0;
        bs[j] = -INFINITY;
      }
#pragma unroll 1
      for (int n = 0; n < N; ++n) {
        const float cx = kp->codewords[2 * n], cy = kp->codewords[2 * n + 1], hq = kp->half_sq[n];
#pragma unroll
        for (int j = 0; j < NBK; ++j) {
          const float sc = fmaf(w[2 * j + 1], cy, fmaf(w[2 * j], cx, hq));
          const bool up = sc > bs[j];
          bs[j] = up ? sc : bs[j];
          best[j] = up ? n : best[j];
        }
      }
#pragma unroll
      for (int j = 0; j < NBK; ++j) put(j, best[j]);
    }
    if (valid) {
      store_half_row<HB>(p.idx + row * RB + h * HB, bits);
      if (h == 0) p.norm[row] = finite ? nu : nu2;
    }
  }
}

template <int D, int B, bool F16>
__global__ __launch_bounds__(kVqWaves * kWave, 2) void decode_vq_kernel(VqParams p) {
  constexpr int HALF = D / 2, NBK = HALF / 2, N = 1 << B;
  constexpr int HB = NBK * B / 8;
  constexpr int RB = 2 * HB;
  constexpr int HWD = (HB + 3) / 4;
  __shared__ float2 s_cw[N];
  // each wave's 32 output rows, staged so that the stores of the tile (one
  // contiguous block of 32 rows) are whole 1 KB chunks; rows padded by 16
  // bytes against bank conflicts
  constexpr int RBYTES = D * (F16 ? 2 : 4);
  constexpr int PITCH = RBYTES + 16;
  __shared__ __align__(16) unsigned char s_out[kVqWaves][32 * PITCH];
  const VqParams* kp = (const VqParams*)__builtin_amdgcn_kernarg_segment_ptr();
  for (int n = threadIdx.x; n < N; n += blockDim.x)
    s_cw[n] = make_float2(kp->codewords[2 * n], kp->codewords[2 * n + 1]);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int64_t ntiles = (p.n_rows + 31) / 32;
  uint32_t fl[HALF / 32 > 0 ? HALF / 32 : 1];
#pragma unroll
  for (int j = 0; j < (HALF / 32 > 0 ? HALF / 32 : 1); ++j) fl[j] = kp->flip[(HALF * h) / 32 + j];

  // the next tile's codes and norm load while the current one is decoded
  const int64_t tstride = (int64_t)gridDim.x * kVqWaves;
  auto row_of = [&](int64_t t) {
    const int64_t r = t * 32 + (lane & 31);
    return r < p.n_rows ? r : p.n_rows - 1;
  };
  int64_t tile = (int64_t)blockIdx.x * kVqWaves + wave;
  uint32_t nbits[HWD];
  float nnorm = 0.f;
  if (tile < ntiles) {
    const int64_t r = row_of(tile);
    load_half_row<HB>(p.idx_in + r * RB + h * HB, nbits);
    nnorm = p.norm_in[r];
  }
  for (; tile < ntiles; tile += tstride) {
    uint32_t bits[HWD];
#pragma unroll
    for (int j = 0; j < HWD; ++j) bits[j] = nbits[j];
    const float norm = nnorm;
    if (tile + tstride < ntiles) {
      const int64_t r = row_of(tile + tstride);
      load_half_row<HB>(p.idx_in + r * RB + h * HB, nbits);
      nnorm = p.norm_in[r];
    }
    float w[HALF];
#pragma unroll
    for (int j = 0; j < NBK; ++j) {
      const int off = j * B, wd = off >> 5, sh = off & 31;
      uint32_t c = bits[wd] >> sh;
      if (sh + B > 32) c |= bits[wd + 1] << (32 - sh);
      const float2 cw = s_cw[c & (N - 1)];
      w[2 * j] = cw.x;
      w[2 * j + 1] = cw.y;
      if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    wht_two_lanes<HALF>(w, h);
    // D and nu / sqrt(d): the scale is >= 0, its sign bit becomes the flip bit
    const float sc = norm * p.inv_sqrt_d;
#pragma unroll
    for (int i = 0; i < HALF; ++i)
      w[i] *= __uint_as_float(((fl[i >> 5] << (31 - (i & 31))) & 0x80000000u) | __float_as_uint(sc));
    unsigned char* stage = s_out[wave];
    {
      uint4* dst = reinterpret_cast<uint4*>(stage + (lane & 31) * PITCH + h * (RBYTES / 2));
      if constexpr (F16) {
#pragma unroll
        for (int q = 0; q < HALF / 8; ++q) {
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(w[8 * q + 2 * j], w[8 * q + 2 * j + 1]));
          dst[q] = make_uint4(o[0], o[1], o[2], o[3]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < HALF / 4; ++q)
          dst[q] = make_uint4(__float_as_uint(w[4 * q]), __float_as_uint(w[4 * q + 1]),
                              __float_as_uint(w[4 * q + 2]), __float_as_uint(w[4 * q + 3]));
      }
    }
    // LDS operations of one wave complete in order: no workgroup barrier
    __builtin_amdgcn_wave_barrier();
    {
      constexpr int CPR = RBYTES / 16;                      // 16-byte chunks per row
      const int64_t row0 = tile * 32;
      const int64_t rows = (p.n_rows - row0) < 32 ? (p.n_rows - row0) : 32;
      uint4* gdst = reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(p.out) + row0 * RBYTES);
#pragma unroll
      for (int k = 0; k < 32 * CPR / kWave; ++k) {
        const int c = lane + kWave * k;
        const int r = c / CPR, col = c % CPR;
        if (r < rows) gdst[c] = *reinterpret_cast<const uint4*>(stage + r * PITCH + col * 16);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <typename K>
static int64_t vq_blocks(K kernel, int64_t n_rows) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kVqWaves * kWave, 0) != hipSuccess || nb < 1)
    nb = 1;
  const int64_t ntiles = (n_rows + 31) / 32;
  int64_t blocks = (ntiles + kVqWaves - 1) / kVqWaves;
  const int64_t cap = (int64_t)device_cu_count() * nb;
  if (blocks > cap) blocks = cap;
  return blocks < 1 ? 1 : blocks;
}

template <int D, int B>
static hipError_t run_vq(bool encode, int dtype, const VqParams& p, hipStream_t s) {
  if (encode) {
    if (dtype == TQ_F16) {
      hipLaunchKernelGGL((encode_vq_kernel<D, B, _Float16>), dim3((unsigned)vq_blocks(encode_vq_kernel<D, B, _Float16>, p.n_rows)),
                         dim3(kVqWaves * kWave), 0, s, p);
    } else {
      hipLaunchKernelGGL((encode_vq_kernel<D, B, float>), dim3((unsigned)vq_blocks(encode_vq_kernel<D, B, float>, p.n_rows)),
                         dim3(kVqWaves * kWave), 0, s, p);
    }
  } else {
    if (dtype == TQ_F16) {
      hipLaunchKernelGGL((decode_vq_kernel<D, B, true>), dim3((unsigned)vq_blocks(decode_vq_kernel<D, B, true>, p.n_rows)),
                         dim3(kVqWaves * kWave), 0, s, p);
    } else {
      hipLaunchKernelGGL((decode_vq_kernel<D, B, false>), dim3((unsigned)vq_blocks(decode_vq_kernel<D, B, false>, p.n_rows)),
                         dim3(kVqWaves * kWave), 0, s, p);
    }
  }
  return hipGetLastError();
}

template <int D>
static hipError_t pick_vq(int b, bool encode, int dtype, const VqParams& p, hipStream_t s) {
  switch (b) {
    case 1: return run_vq<D, 1>(encode, dtype, p, s);
    case 2: return run_vq<D, 2>(encode, dtype, p, s);
    case 3: return run_vq<D, 3>(encode, dtype, p, s);
    case 4: return run_vq<D, 4>(encode, dtype, p, s);
    case 5: return run_vq<D, 5>(encode, dtype, p, s);
    case 6: return run_vq<D, 6>(encode, dtype, p, s);
    case 7: return run_vq<D, 7>(encode, dtype, p, s);
    case 8: return run_vq<D, 8>(encode, dtype, p, s);
  }
  return hipErrorInvalidValue;
}

static void vq_params(const tq_vq_codec& c, int64_t n_rows, VqParams& p) {
  p = {};
  p.n_rows = n_rows;
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)c.d));
  for (int w = 0; w < 4; ++w) p.flip[w] = c.flip[w];
  for (int n = 0; n < 2 * c.n_codes; ++n) p.codewords[n] = c.codewords[n];
  for (int n = 0; n < c.n_codes; ++n) {
    const float x = c.codewords[2 * n], y = c.codewords[2 * n + 1];
    p.half_sq[n] = -0.5f * (x * x + y * y);
  }
}

hipError_t launch_encode_vq(const tq_vq_codec& c, const void* x, int dtype, int64_t n_rows, uint8_t* idx,
                            float* norm, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  VqParams p;
  vq_params(c, n_rows, p);
  p.search = static_cast<const uint8_t*>(c.search);
  p.x = x;
  p.idx = idx;
  p.norm = norm;
  if (c.d == 128) return pick_vq<128>(c.block_bits, true, dtype, p, stream);
  if (c.d == 64) return pick_vq<64>(c.block_bits, true, dtype, p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_vq(const tq_vq_codec& c, const uint8_t* idx, const float* norm, int64_t n_rows,
                            void* out, int out_dtype, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  VqParams p;
  vq_params(c, n_rows, p);
  p.idx_in = idx;
  p.norm_in = norm;
  p.out = out;
  if (c.d == 128) return pick_vq<128>(c.block_bits, false, out_dtype, p, stream);
  if (c.d == 64) return pick_vq<64>(c.block_bits, false, out_dtype, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace tqk
