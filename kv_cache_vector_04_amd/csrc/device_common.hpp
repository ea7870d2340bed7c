// Device-side building blocks shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tqk {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// The parts of a codec a kernel needs, passed by value (lands in SGPRs).
struct CodecArgs {
  float centroids[16];
  float thresholds[16];
  uint32_t flip[48];   // bit i%32 of word i/32 set <=> D_i = -1
  const float* S;      // m x d row-major fp32 (prod only)
  int d, code_bits, mode, m;
};

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// ---------------------------------------------------------------------------
// Randomized Walsh-Hadamard transform of one vector held in registers
// (one vector per lane): D sign flip, then the natural-order butterflies
// (x_i, x_{i+h}) -> (x_i + x_{i+h}, x_i - x_{i+h}) for h = 1, 2, ..., D/2.
// No scaling; the caller folds 1/sqrt(D) into its own scale.
// ("Ablazione, ...", "Configurazione Sperimentale": randomized WHT.)
template <int D>
__device__ __forceinline__ void flip_signs(float (&x)[D], const uint32_t* flip) {
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const uint32_t bit = (flip[i >> 5] >> (i & 31)) & 1u;
    x[i] = __uint_as_float(__float_as_uint(x[i]) ^ (bit << 31));
  }
}

template <int D>
__device__ __forceinline__ void wht_inreg(float (&x)[D]) {
#pragma unroll
  for (int h = 1; h < D; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

// Sum of squares with 16 interleaved accumulators combined pairwise (keeps
// the fp32 rounding error of a 128-term sum near log2 depth).
template <int D>
__device__ __forceinline__ float sum_squares(const float (&x)[D]) {
  constexpr int A = D < 16 ? D : 16;
  float acc[A];
#pragma unroll
  for (int j = 0; j < A; ++j) acc[j] = x[j] * x[j];
#pragma unroll
  for (int i = A; i < D; ++i) acc[i % A] = fmaf(x[i], x[i], acc[i % A]);
#pragma unroll
  for (int w = A / 2; w >= 1; w >>= 1) {
#pragma unroll
    for (int j = 0; j < w; ++j) acc[j] += acc[j + w];
  }
  return acc[0];
}

// Exchange between the two 32-lane halves of a wave: returns
// {a with its upper half replaced by b's lower half,
//  b with its lower half replaced by a's upper half}.
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// Pack per-coordinate codes (CB bits each) into an LSB-first bit stream of
// 32-bit words: code i occupies stream bits [i*CB, (i+1)*CB).
template <int D, int CB>
__device__ __forceinline__ void pack_codes(const int (&q)[D],
                                           uint32_t (&w)[D * CB / 32]) {
#pragma unroll
  for (int j = 0; j < D * CB / 32; ++j) w[j] = 0u;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int off = i * CB;
    const int word = off >> 5, sh = off & 31;
    w[word] |= (uint32_t)q[i] << sh;
    if (sh + CB > 32) w[word + 1] |= (uint32_t)q[i] >> (32 - sh);
  }
}

// Store W words to a row at `dst` (byte alignment of the row: `ALIGN`).
template <int W, int ALIGN>
__device__ __forceinline__ void store_words(uint8_t* dst, const uint32_t (&w)[W]) {
  if constexpr (ALIGN % 16 == 0 && W % 4 == 0) {
#pragma unroll
    for (int j = 0; j < W / 4; ++j)
      reinterpret_cast<uint4*>(dst)[j] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
  } else if constexpr (ALIGN % 8 == 0 && W % 2 == 0) {
#pragma unroll
    for (int j = 0; j < W / 2; ++j)
      reinterpret_cast<uint2*>(dst)[j] = make_uint2(w[2 * j], w[2 * j + 1]);
  } else {
#pragma unroll
    for (int j = 0; j < W; ++j) reinterpret_cast<uint32_t*>(dst)[j] = w[j];
  }
}

template <int W, int ALIGN>
__device__ __forceinline__ void load_words(const uint8_t* src, uint32_t (&w)[W]) {
  if constexpr (ALIGN % 16 == 0 && W % 4 == 0) {
#pragma unroll
    for (int j = 0; j < W / 4; ++j) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[j];
      w[4 * j] = v.x; w[4 * j + 1] = v.y; w[4 * j + 2] = v.z; w[4 * j + 3] = v.w;
    }
  } else if constexpr (ALIGN % 8 == 0 && W % 2 == 0) {
#pragma unroll
    for (int j = 0; j < W / 2; ++j) {
      const uint2 v = reinterpret_cast<const uint2*>(src)[j];
      w[2 * j] = v.x; w[2 * j + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < W; ++j) w[j] = reinterpret_cast<const uint32_t*>(src)[j];
  }
}

// Extract code i (CB bits) from a packed row held as words.
template <int CB, int W>
__device__ __forceinline__ uint32_t get_code(const uint32_t (&w)[W], int i) {
  const int off = i * CB;
  const int word = off >> 5, sh = off & 31;
  uint32_t v = w[word] >> sh;
  if (sh + CB > 32) v |= w[word + 1] << (32 - sh);
  return v & ((1u << CB) - 1u);
}

// Load one row of D elements of type T (fp16 or fp32) into fp32 registers.
template <int D, typename T>
__device__ __forceinline__ void load_row(const T* __restrict__ src, float (&x)[D]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < D / 8; ++j) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[j];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(u[e] & 0xffffu));
        const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(u[e] >> 16));
        x[8 * j + 2 * e] = (float)lo;
        x[8 * j + 2 * e + 1] = (float)hi;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < D / 4; ++j) {
      const float4 v = reinterpret_cast<const float4*>(src)[j];
      x[4 * j] = v.x; x[4 * j + 1] = v.y; x[4 * j + 2] = v.z; x[4 * j + 3] = v.w;
    }
  }
}

// sin and cos of an angle given in fp64: quadrant reduction by pi/2 in fp64,
// then Taylor polynomials on |r| <= pi/4 in fp32 (truncation below 3e-10,
// far under fp32 rounding).
__device__ __forceinline__ void sincos_reduced(double ang, float& s, float& c) {
  const double half_pi = 1.5707963267948966192313216916398;
  const double k = rint(ang / half_pi);
  const float r = (float)(ang - k * half_pi);
  const float r2 = r * r;
  const float sr = r * (1.f + r2 * (-1.f / 6.f + r2 * (1.f / 120.f + r2 * (-1.f / 5040.f +
                   r2 * (1.f / 362880.f + r2 * (-1.f / 39916800.f))))));
  const float cr = 1.f + r2 * (-0.5f + r2 * (1.f / 24.f + r2 * (-1.f / 720.f +
                   r2 * (1.f / 40320.f + r2 * (-1.f / 3628800.f + r2 * (1.f / 479001600.f))))));
  const int q = (int)((long long)k & 3);
  s = q == 0 ? sr : (q == 1 ? cr : (q == 2 ? -sr : -cr));
  c = q == 0 ? cr : (q == 1 ? -sr : (q == 2 ? -cr : sr));
}

// RoPE on interleaved pairs: angle = pos * theta_i ("TurboESM", "2.
// Metodologia" part A: RoPE first, then the orthogonal rotation).
template <int D>
__device__ __forceinline__ void rope_inplace(float (&x)[D], int64_t pos, const double* __restrict__ theta) {
#pragma unroll
  for (int i = 0; i < D / 2; ++i) {
    float s, c;
    sincos_reduced((double)pos * theta[i], s, c);
    const float a = x[2 * i], b = x[2 * i + 1];
    x[2 * i] = a * c - b * s;
    x[2 * i + 1] = a * s + b * c;
  }
}

}  // namespace tqk
