// TurboQuant encode for gfx950, d = 64 or 128: one vector per lane (fp32
// input at d = 64, RoPE keys) or two lanes per vector (fp16 input, and fp32
// input at d = 128; see the layout notes further down).
//
// Per vector ("FibQuant", "1. Enunciato del Problema" and "2.3 Codifica e
// Decodifica"; "Google presenta TurboQuant", "La mecánica geométrica de
// TurboQuant" and "Eliminación del sesgo interno del producto"):
//   (RoPE, keys of a RoPE model)  nu = |x|  ->  y = H_d (D * x)  (in-register
//   butterflies)  ->  z = y / (sqrt(d) nu)  ->  idx_i = #{k : z_i >= t_k}
//   ->  bit-pack at a fixed address
// and for TurboQuant_prod additionally r = z - c[idx], gamma = |r| and the
// sign bits of S r.  S r is a dense (m x d) x (d x 64 tokens) contraction per
// wave, done on the matrix cores with v_mfma_f32_32x32x16_f16 in three
// passes S_hi r_hi + S_hi r_lo + S_lo r_hi (fp16 hi/lo splits of both
// operands, fp32 accumulation), which keeps |error| of (S r)_i near 1e-7.
// The prod path works with r' = 256 r (a power of two, so that the low
// fp16 part of r' stays a normal number); the sign of S r' is that of S r.
//
// Quantizer: codes with 3 or more bits use a uniform grid over z in
// [-1.01, 1.01] (u = a z + b, cell = floor(u)) with at most one threshold
// per cell; a cell's entry holds the threshold inside it (u units) and the
// number of thresholds below the cell, so the code is one table read and
// one compare (the host picks the smallest grid with that property).  The
// result equals #{k : u >= a t_k + b}, the code of z up to fp32 rounding.
// One- and two-bit codes compare directly.
//
// fp16 input: the sign flip is an xor on the packed halves, the norm comes
// from v_dot2 on them, and the first butterfly stage converts and adds in
// one v_fma_mix_f32 per output.
//
// Layout of a wave's tile: lane l owns row 64*tile + l.  The MFMA B operand
// for 32 tokens needs, in lane l, token l%32 and the k-group l/32; the two
// 32-token blocks of a tile are exchanged between wave halves with one
// v_permlane32_swap per pair of packed registers.  The rows of S in the A
// fragments are ordered so that the C registers of lane l hold rows
// 16 (l/32) + 0..15 of the 32-row tile: each lane half collects 16
// consecutive sign bits, and one more swap puts every word on its row.

#include <atomic>
#include <cmath>
#include <cstring>

#include "device_common.hpp"
#include "internal.hpp"

namespace tqk {

constexpr int kEncWaves = 8;
constexpr int kLutMax = 256;
constexpr float kGridRange = 1.01f;

struct EncodeParams {
  const void* x;
  int64_t x_stride;     // elements between consecutive rows of x (d, or more for a channel slice)
  int64_t n_rows;
  uint8_t* idx;
  uint8_t* qjl;
  float* norm;
  float* rnorm;
  CodecArgs codec;
  int64_t seq_len;
  int lut_g;            // grid cells (codes of 3 or more bits)
  float lut_a, lut_b;   // u = z a + b
  uint32_t hflip[64];   // fp16 pairs: xor masks (bits 15, 31) of the sign flip
  double theta[64];
};

template <int D>
struct ProdGeom {
  static constexpr int MT = D / 32;   // 32-row tiles of S
  static constexpr int KS = D / 16;   // 16-wide k steps
  static constexpr int FRAGS = MT * KS;
};

__device__ __forceinline__ uint32_t pack_h2(_Float16 a, _Float16 b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// lo + hi and lo - hi of the two fp16 halves of w, in fp32
__device__ __forceinline__ void mix_butterfly(uint32_t w, float& s, float& d) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(s) : "v"(w));
  asm("v_fma_mix_f32 %0, %1, 1.0, -%1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(d) : "v"(w));
}

// a - (fp16 low half of h) and b - (fp16 high half of h), in fp32 (exact
// when h holds a and b truncated to fp16)
__device__ __forceinline__ void mix_sub(uint32_t h, float a, float b, float& ra, float& rb) {
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(h), "v"(a));
  asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(h), "v"(b));
}

// hi/lo fp16 split of a pair: hi = (a, b) rounded toward zero, lo = rest
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  float ra, rb;
  mix_sub(hi, a, b, ra, rb);
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(ra, rb));
}

template <int D, int CB, bool PROD, typename T, bool ROPE>
__global__ __launch_bounds__(kEncWaves * kWave) void encode_kernel(EncodeParams p) {
  constexpr int NLEV = 1 << CB;
  constexpr int NTH = NLEV - 1;
  constexpr int W = D * CB / 32;          // code words per row
  constexpr int ROW_BYTES = D * CB / 8;
  constexpr int ALIGN = ROW_BYTES % 16 == 0 ? 16 : (ROW_BYTES % 8 == 0 ? 8 : 4);
  constexpr bool USE_LUT = CB >= 3;
  constexpr bool F16 = sizeof(T) == 2 && !ROPE;
  using G = ProdGeom<D>;

  __shared__ float s_cent[16];
  __shared__ float2 s_lut[USE_LUT ? kLutMax : 1];
  __shared__ double s_theta[ROPE ? D / 2 : 1];
  __shared__ uint4 s_frag[PROD ? G::FRAGS * 2 * kWave : 1];

  const int tid = threadIdx.x;
  const EncodeParams* kp = (const EncodeParams*)__builtin_amdgcn_kernarg_segment_ptr();
  const float cscale = PROD ? 256.f : 1.f;
  if (tid < 16) s_cent[tid] = kp->codec.centroids[tid] * cscale;
  if (ROPE && tid < D / 2) s_theta[tid] = kp->theta[tid];
  if constexpr (USE_LUT) {
    // grid cell g: (threshold inside the cell or +inf, thresholds below the
    // cell)
    const float a = p.lut_a, b = p.lut_b;
    for (int g = tid; g < p.lut_g; g += blockDim.x) {
      int base = 0;
      float thr = INFINITY;
#pragma unroll
      for (int k = 0; k < NTH; ++k) {
        const float tu = fmaf(kp->codec.thresholds[k], a, b);
        const int cell = (int)tu;
        base += cell < g ? 1 : 0;
        if (cell == g) thr = tu;
      }
      s_lut[g] = make_float2(thr, __int_as_float(base));
    }
  }

  if constexpr (PROD) {
    // S_hi / S_lo as MFMA A fragments: fragment (mt, ks), lane l holds
    // S[32 mt + perm(l%32)][16 ks + 8 (l/32) + j], j = 0..7, where perm
    // sends the C row 8 (v/4) + 4 h + v%4 of register v in lane half h to
    // row 16 h + v.
    for (int t = tid; t < G::FRAGS * kWave; t += blockDim.x) {
      const int lane = t & 63, f = t >> 6;
      const int mt = f / G::KS, ks = f % G::KS;
      const int rho = lane & 31;
      const int m = 32 * mt + 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
      const int k0 = 16 * ks + 8 * (lane >> 5);
      const float* srow = p.codec.S + (size_t)m * D + k0;
      const float4 s0 = reinterpret_cast<const float4*>(srow)[0];
      const float4 s1 = reinterpret_cast<const float4*>(srow)[1];
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
      _Float16 hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        hi[j] = (_Float16)sv[j];
        lo[j] = (_Float16)(sv[j] - (float)hi[j]);
      }
      s_frag[(2 * f) * kWave + lane] =
          make_uint4(pack_h2(hi[0], hi[1]), pack_h2(hi[2], hi[3]), pack_h2(hi[4], hi[5]), pack_h2(hi[6], hi[7]));
      s_frag[(2 * f + 1) * kWave + lane] =
          make_uint4(pack_h2(lo[0], lo[1]), pack_h2(lo[2], lo[3]), pack_h2(lo[4], lo[5]), pack_h2(lo[6], lo[7]));
    }
  }
  __syncthreads();

  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t ntiles = (p.n_rows + kWave - 1) / kWave;
  const T* __restrict__ xin = reinterpret_cast<const T*>(p.x);
  const float lut_a = p.lut_a, lut_b = p.lut_b;

  for (int64_t tile = (int64_t)blockIdx.x * kEncWaves + wave; tile < ntiles;
       tile += (int64_t)gridDim.x * kEncWaves) {
    const int64_t row = tile * kWave + lane;
    const bool valid = row < p.n_rows;
    float x[D];
    float nu_s, pre_inv = 1.f;
    if constexpr (F16) {
      uint32_t u[D / 2];
      if (valid) {
#pragma unroll
        for (int j = 0; j < D / 8; ++j) {
          const uint4 v = reinterpret_cast<const uint4*>(xin + row * p.x_stride)[j];
          u[4 * j] = v.x; u[4 * j + 1] = v.y; u[4 * j + 2] = v.z; u[4 * j + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < D / 2; ++j) u[j] = 0u;
      }
      typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
      float acc[16];
#pragma unroll
      for (int a = 0; a < 16; ++a) acc[a] = 0.f;
#pragma unroll
      for (int j = 0; j < D / 2; ++j) {
        const h2_t hv = __builtin_bit_cast(h2_t, u[j]);
        acc[j & 15] = __builtin_amdgcn_fdot2(hv, hv, acc[j & 15], false);
      }
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int a = 0; a < w; ++a) acc[a] += acc[a + w];
      // a non-finite input encodes as the zero vector (its norm stays non-finite)
      if (!(acc[0] <= 3.0e38f)) {
#pragma unroll
        for (int j = 0; j < D / 2; ++j) u[j] = 0u;
      }
      nu_s = sqrtf(acc[0]);
#pragma unroll
      for (int j = 0; j < D / 2; ++j) mix_butterfly(u[j] ^ kp->hflip[j], x[2 * j], x[2 * j + 1]);
#pragma unroll
      for (int h = 2; h < D; h <<= 1) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
          if ((i & h) == 0) {
            const float a = x[i], b = x[i + h];
            x[i] = a + b;
            x[i + h] = a - b;
          }
        }
      }
    } else {
      if (valid) {
        load_row<D, T>(xin + row * p.x_stride, x);
      } else {
#pragma unroll
        for (int i = 0; i < D; ++i) x[i] = 0.f;
      }
      if constexpr (ROPE) rope_inplace<D>(x, row % p.seq_len, s_theta);
      // nu = |x|.  When the squares leave the normal fp32 range (only fp32
      // inputs get there) the vector is first scaled exactly by the power of
      // two that brings its largest entry into [0.5, 1).
      float nu2 = sum_squares<D>(x);
      if (!(nu2 >= 0x1p-100f && nu2 <= 0x1p100f)) {
        // a NaN element makes the sum NaN (fmaxf below would skip it)
        const bool has_nan = !(nu2 == nu2);
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) mx = fmaxf(mx, fabsf(x[i]));
        if (has_nan || !(mx <= 3.4e38f)) {
          // a non-finite input encodes as the zero vector; nu2 stays inf or
          // NaN, and so does the stored norm
#pragma unroll
          for (int i = 0; i < D; ++i) x[i] = 0.f;
        } else if (mx > 0.f) {
          int e;
          frexpf(mx, &e);
          const float sc = ldexpf(1.f, -e);
          pre_inv = ldexpf(1.f, e);
#pragma unroll
          for (int i = 0; i < D; ++i) x[i] *= sc;
          nu2 = sum_squares<D>(x);
        }
      }
      nu_s = sqrtf(nu2);
      flip_signs<D>(x, p.codec.flip);
      wht_inreg<D>(x);
    }
    const float nu = nu_s * pre_inv;
    const bool live = nu_s > 0.f && nu_s <= 3.0e38f;
    // z = y * inv;  prod residual r' = 256 z - c'
    const float inv = live ? 1.0f / (sqrtf((float)D) * nu_s) : 0.f;
    const float inv_p = inv * cscale;
    const float ua = lut_a * inv;

    // the quantizer starts once the butterflies are done (interleaving the
    // two only raises the register pressure)
    __builtin_amdgcn_sched_barrier(0);
    uint32_t words[W];
#pragma unroll
    for (int j = 0; j < W; ++j) words[j] = 0u;
    // code of coordinate i (packed into words); prod: returns r'_i
    auto quantize = [&](int i) -> float {
      int c;
      float r = 0.f;
      if constexpr (USE_LUT) {
        const float u = fmaf(x[i], ua, lut_b);
        const float2 e = s_lut[(uint32_t)u];
        c = __float_as_int(e.y) + (u >= e.x ? 1 : 0);
        if constexpr (PROD) r = fmaf(x[i], inv_p, -s_cent[c]);
      } else {
        const float z = x[i] * inv_p;
        c = 0;
#pragma unroll
        for (int k = 0; k < NTH; ++k) c += (z >= p.codec.thresholds[k] * cscale) ? 1 : 0;
        if constexpr (PROD) r = z - s_cent[c];
      }
      const int off = i * CB;
      words[off >> 5] |= (uint32_t)c << (off & 31);
      if ((off & 31) + CB > 32) words[(off >> 5) + 1] |= (uint32_t)c >> (32 - (off & 31));
      return r;
    };

    if constexpr (!PROD) {
#pragma unroll
      for (int i = 0; i < D; ++i) quantize(i);
      if (valid) {
        store_words<W, ALIGN>(p.idx + row * ROW_BYTES, words);
        p.norm[row] = nu;
      }
    } else {
      // 16 coordinates at a time: codes, r' = 256 (z - c[idx]), gamma^2, and
      // the B fragments: X = r'[16ks .. 16ks+7], Y = r'[16ks+8 .. 16ks+15],
      // split hi/lo; after the half-wave swap X holds block 0 (tokens of
      // lanes 0..31) and Y block 1.
      uint32_t b0h[G::KS][4], b1h[G::KS][4], b0l[G::KS][4], b1l[G::KS][4];
      float g2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        float r[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          r[e] = quantize(16 * ks + e);
          g2[e & 3] = fmaf(r[e], r[e], g2[e & 3]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t xh, xl, yh, yl;
          split_pair(r[2 * j], r[2 * j + 1], xh, xl);
          split_pair(r[8 + 2 * j], r[8 + 2 * j + 1], yh, yl);
          swap_halves(xh, yh);
          swap_halves(xl, yl);
          b0h[ks][j] = xh; b1h[ks][j] = yh;
          b0l[ks][j] = xl; b1l[ks][j] = yl;
        }
        // pin the code words here: left alone, the compiler sinks their
        // assembly to the store and keeps every compare mask alive until then
#pragma unroll
        for (int j = 0; j < W; ++j) asm volatile("" : "+v"(words[j]));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (valid) {
        store_words<W, ALIGN>(p.idx + row * ROW_BYTES, words);
        p.norm[row] = nu;
      }
      if (valid) p.rnorm[row] = sqrtf((g2[0] + g2[1]) + (g2[2] + g2[3])) * (1.f / 256.f);

      uint32_t sign_words[4] = {0u, 0u, 0u, 0u};
      const uint32_t half_shift = 16u * (uint32_t)(lane >> 5);
      // one 32-row tile of S at a time (not unrolled: bounds the live
      // registers to the B fragments, one tile's A fragments and 32 sums)
#pragma unroll 1
      for (int mt = 0; mt < G::MT; ++mt) {
        f32x16 c0 = {}, c1 = {};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
          const uint4 ah_u = s_frag[(2 * (mt * G::KS + ks)) * kWave + lane];
          const uint4 al_u = s_frag[(2 * (mt * G::KS + ks) + 1) * kWave + lane];
          const half8_t ah = __builtin_bit_cast(half8_t, ah_u);
          const half8_t al = __builtin_bit_cast(half8_t, al_u);
          const half8_t bh0 = __builtin_bit_cast(half8_t, make_uint4(b0h[ks][0], b0h[ks][1], b0h[ks][2], b0h[ks][3]));
          const half8_t bl0 = __builtin_bit_cast(half8_t, make_uint4(b0l[ks][0], b0l[ks][1], b0l[ks][2], b0l[ks][3]));
          const half8_t bh1 = __builtin_bit_cast(half8_t, make_uint4(b1h[ks][0], b1h[ks][1], b1h[ks][2], b1h[ks][3]));
          const half8_t bl1 = __builtin_bit_cast(half8_t, make_uint4(b1l[ks][0], b1l[ks][1], b1l[ks][2], b1l[ks][3]));
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh0, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh1, c1, 0, 0, 0);
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl0, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl1, c1, 0, 0, 0);
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh0, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh1, c1, 0, 0, 0);
          // keep the next step's A fragments from being hoisted: bounds the
          // live registers to one step's operands
          __builtin_amdgcn_sched_barrier(0);
        }
        // register v of lane half h holds row 16 h + v of the tile: shift the
        // sign bits in from v = 15 down to 0, then bit = [p >= 0] (a result
        // of exactly -0 reads as negative; it needs r = 0)
        uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
        for (int v = 15; v >= 0; --v) {
          w0 = __builtin_amdgcn_alignbit(w0, __float_as_uint(c0[v]), 31);
          w1 = __builtin_amdgcn_alignbit(w1, __float_as_uint(c1[v]), 31);
        }
        w0 = (w0 ^ 0xFFFFu) << half_shift;
        w1 = (w1 ^ 0xFFFFu) << half_shift;
        swap_halves(w0, w1);
        const uint32_t word = w0 | w1;
        sign_words[0] = mt == 0 ? word : sign_words[0];
        sign_words[1] = mt == 1 ? word : sign_words[1];
        sign_words[2] = mt == 2 ? word : sign_words[2];
        sign_words[3] = mt == 3 ? word : sign_words[3];
      }
      if (valid) {
        if constexpr (G::MT == 4)
          *reinterpret_cast<uint4*>(p.qjl + row * (D / 8)) =
              make_uint4(sign_words[0], sign_words[1], sign_words[2], sign_words[3]);
        else
          *reinterpret_cast<uint2*>(p.qjl + row * (D / 8)) = make_uint2(sign_words[0], sign_words[1]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 input without RoPE, and fp32 input at d = 128: two lanes per vector
// (fp32 rows take the path of f32_rotate_half below up to the rotated
// coordinates, then the same quantizer and projection).  Lane l of a wave owns
// token 32 tile + l%32 and the coordinate half h = l/32 (coordinates
// h d/2 .. h d/2 + d/2 - 1), which halves the registers a vector needs and
// lets more waves hide the HBM latency.  The butterfly stages commute; the
// one across the halves (coordinate bit log2(d/2)) runs first, on the
// packed fp16 input: one v_permlane32_swap gives every lane both halves'
// pair, and v_fma_mix_f32 forms x_low + x_high (low lane) or
// x_low - x_high (high lane) in fp32.  The other stages stay in registers.
// For prod, the B operand of the projection takes, in lane l at k step ks,
// the lane's own residuals 8 ks .. 8 ks + 7 (k slot j of lane half h is
// coordinate h d/2 + 8 ks + j; the A fragments of S use the same order),
// so no exchange is needed, and both lane halves hold 16 of the 32 sign
// bits of each 32-row tile.

// Workgroup shape.  prod: the 64 KB of S fragments allow two workgroups
// per CU; eight waves each at two waves per SIMD leave the registers for
// loading the next tile's input while the current one is processed.  mse:
// small workgroups at four waves per SIMD (a prefetch measured no faster).
template <bool PROD, bool F32IN = false>
struct HalfLaunch {
  static constexpr bool kPrefetch = PROD && !F32IN;
  static constexpr int kWaves = PROD ? 8 : 4;
  // (fp32 mse rows hold 64 loaded floats per lane: more than four waves'
  // share of the registers)
  static constexpr int kMinWavesPerEU = PROD || F32IN ? 2 : 4;
};

// v from the low half plus v from the high half, in every lane
__device__ __forceinline__ float cross_sum(float v) {
  uint32_t a = __float_as_uint(v), b = a;
  swap_halves(a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}

// LDS tables of one codec for the two-lanes-per-vector encoder
template <int D, int CB, bool PROD, bool MROT = false, bool F32IN = false>
struct HalfTables {
  static constexpr int FRAGS = (D / 32) * (D / 16);
  float cent[16];
  float2 lut[CB >= 3 ? kLutMax : 1];
  uint4 hmask[MROT ? 1 : D / 8];
  uint4 fmask[F32IN ? D / 4 : 1];       // fp32 input: bit 31 of coordinate i's word set when D_ii = -1
  uint4 hd[MROT ? 2 * (D / 16) * kWave : 1];   // H D as A fragments (rotation on the matrix cores)
  uint4 frag[PROD ? FRAGS * 2 * kWave : 1];
};

// The tables from the codec (all nthr threads of the workgroup take part;
// the caller synchronizes afterwards).  kp: p in the kernel argument
// segment, for indexing its arrays with run-time indices.
template <int D, int CB, bool PROD, bool MROT = false, bool F32IN = false>
__device__ __forceinline__ void half_setup(const EncodeParams& p, const EncodeParams* kp,
                                           HalfTables<D, CB, PROD, MROT, F32IN>& T, int tid, int nthr) {
  constexpr int NLEV = 1 << CB;
  constexpr int NTH = NLEV - 1;
  constexpr int HALF = D / 2;
  constexpr int NP = D / 4;
  constexpr bool USE_LUT = CB >= 3;
  constexpr int KS = D / 16, MT = D / 32, FRAGS = MT * KS;
  (void)MT;
  const float cscale = PROD ? 256.f : 1.f;
  if (tid < 16) T.cent[tid] = kp->codec.centroids[tid] * cscale;
  if (!MROT && tid >= 64 && tid < 64 + NP / 2)
    T.hmask[tid - 64] = make_uint4(kp->hflip[4 * (tid - 64)], kp->hflip[4 * (tid - 64) + 1],
                                   kp->hflip[4 * (tid - 64) + 2], kp->hflip[4 * (tid - 64) + 3]);
  if (F32IN && tid >= 128 && tid < 128 + D / 4) {
    const int i = 4 * (tid - 128);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = ((kp->codec.flip[(i + e) >> 5] >> ((i + e) & 31)) & 1u) << 31;
    T.fmask[tid - 128] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if constexpr (USE_LUT) {
    const float a = p.lut_a, b = p.lut_b;
    for (int g = tid; g < p.lut_g; g += nthr) {
      int base = 0;
      float thr = INFINITY;
#pragma unroll
      for (int k = 0; k < NTH; ++k) {
        const float tu = fmaf(kp->codec.thresholds[k], a, b);
        const int cell = (int)tu;
        base += cell < g ? 1 : 0;
        if (cell == g) thr = tu;
      }
      T.lut[g] = make_float2(thr, __int_as_float(base));
    }
  }
  if constexpr (PROD) {
    // fragment (mt, ks), lane l: row 32 mt + perm(l%32) of S (perm as in the
    // one-vector-per-lane kernel), columns (l/32) d/2 + 8 ks + 0..7
    for (int t = tid; t < FRAGS * kWave; t += nthr) {
      const int lane = t & 63, f = t >> 6;
      const int mt = f / KS, ks = f % KS;
      const int rho = lane & 31;
      const int m = 32 * mt + 16 * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
      const int k0 = (lane >> 5) * HALF + 8 * ks;
      const float* srow = p.codec.S + (size_t)m * D + k0;
      const float4 s0 = reinterpret_cast<const float4*>(srow)[0];
      const float4 s1 = reinterpret_cast<const float4*>(srow)[1];
      // hi / lo fp16 split, four instructions per pair (the set-up of every
      // workgroup converts all of S; measured against rounding each half to
      // nearest element by element: keys alone 45.2 -> 44.6 us, keys and
      // values 58.2 -> 57.8 us per GQA encode call)
      uint32_t hi[4], lo[4];
      split_pair(s0.x, s0.y, hi[0], lo[0]);
      split_pair(s0.z, s0.w, hi[1], lo[1]);
      split_pair(s1.x, s1.y, hi[2], lo[2]);
      split_pair(s1.z, s1.w, hi[3], lo[3]);
      T.frag[(2 * f) * kWave + lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      T.frag[(2 * f + 1) * kWave + lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
  if constexpr (MROT) {
    // fragment (mt, ks), lane l: row sigma(mt, l%32) = (d/2) ((l/4)%2) +
    // 16 mt + 4 ((l%32)/8) + l%4 of H D, columns (d/2) (l/32) + 8 ks + 0..7.
    // With that row order, register v of the product's tile mt lands, in
    // lane half h, on coordinate (d/2) h + 16 mt + v: the input's layout.
    // The bits of 16 mt in a row are set by no other term, and the same bits
    // of a column are those of 16 (ks / 2), so fragment (mt, ks) is fragment
    // (0, ks) times (-1)^popcount(mt & (ks / 2)): the table holds each k step
    // with both signs (half the LDS and half the set-up of one fragment per
    // (mt, ks); measured 61.3 -> 59.8 us per GQA encode call).
    // the flip words through scalar loads (a lane-indexed read of the kernel
    // arguments would be a memory round trip per coordinate)
    const uint32_t fw0 = kp->codec.flip[0], fw1 = kp->codec.flip[1];
    const uint32_t fw2 = D > 64 ? kp->codec.flip[2] : 0u, fw3 = D > 64 ? kp->codec.flip[3] : 0u;
    for (int t = tid; t < 2 * KS * kWave; t += nthr) {
      const int lane = t & 63, f = t >> 6;
      const int ks = f >> 1, sgn = f & 1;
      const int rho = lane & 31;
      const int sig = HALF * ((rho >> 2) & 1) + 4 * (rho >> 3) + (rho & 3);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        uint32_t e[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int pi = HALF * (lane >> 5) + 8 * ks + j + q;
          const int wi = pi >> 5;
          const uint32_t fw = wi == 0 ? fw0 : (wi == 1 ? fw1 : (wi == 2 ? fw2 : fw3));
          const uint32_t neg = ((uint32_t)__popc(sig & pi) + (fw >> (pi & 31)) + sgn) & 1u;
          e[q] = neg ? 0xBC00u : 0x3C00u;   // fp16 -1 / +1
        }
        w[j >> 1] = e[0] | (e[1] << 16);
      }
      T.hd[t] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// largest of v in the low and the high half, in every lane
__device__ __forceinline__ float cross_max(float v) {
  uint32_t a = __float_as_uint(v), b = a;
  swap_halves(a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// fp32 input, two lanes per vector: lane half h loads coordinates
// h d/2 .. h d/2 + d/2 - 1 of its row; the pair forms nu, flips the signs
// and runs every butterfly stage, the one across the halves through
// v_permlane32_swap and the others in registers.  When the squares leave
// the normal fp32 range the row is first scaled exactly by the power of two
// that brings its largest entry into [0.5, 1): the return value is the norm
// of the scaled row and pre_inv the power of two that undoes the scaling.
// A row with an inf or NaN element comes back as the zero vector with a
// non-finite norm (inf, or NaN when an element is NaN).  Both lanes of a
// pair see the same sums and take the same branches.
template <int D>
__device__ __forceinline__ float f32_rotate_half(const EncodeParams& p, const uint4* fmask, int64_t tile,
                                                 float sgn, float (&x)[D / 2], float& pre_inv) {
  constexpr int HALF = D / 2;
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, h = lane >> 5;
  // a buffer descriptor over the (wave-uniform) tile's rows: rows past the
  // end read as zeros
  const int64_t r0 = tile * 32;
  const int64_t left = p.n_rows - r0;
  const uint32_t rows = left <= 0 ? 0u : (left < 32 ? (uint32_t)left : 32u);
  const float* base = reinterpret_cast<const float*>(p.x) + (left > 0 ? r0 * p.x_stride : 0);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)base, (short)0, (int)(rows * (uint32_t)p.x_stride * 4u), 0x00020000);
  const uint32_t off = ((uint32_t)(lane & 31) * (uint32_t)p.x_stride + (uint32_t)(h * HALF)) * 4u;
#pragma unroll
  for (int j = 0; j < HALF / 4; ++j) {
    const u4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * j, 0, 0);
    x[4 * j] = __uint_as_float(v[0]); x[4 * j + 1] = __uint_as_float(v[1]);
    x[4 * j + 2] = __uint_as_float(v[2]); x[4 * j + 3] = __uint_as_float(v[3]);
  }
  float nu2 = cross_sum(sum_squares<HALF>(x));
  pre_inv = 1.f;
  if (!(nu2 >= 0x1p-100f && nu2 <= 0x1p100f)) {
    // a NaN element makes the sum NaN (fmaxf below would skip it)
    const bool has_nan = !(nu2 == nu2);
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) mx = fmaxf(mx, fabsf(x[i]));
    mx = cross_max(mx);
    if (has_nan || !(mx <= 3.4e38f)) {
#pragma unroll
      for (int i = 0; i < HALF; ++i) x[i] = 0.f;
    } else if (mx > 0.f) {
      int e;
      frexpf(mx, &e);
      const float sc = ldexpf(1.f, -e);
      pre_inv = ldexpf(1.f, e);
#pragma unroll
      for (int i = 0; i < HALF; ++i) x[i] *= sc;
      nu2 = cross_sum(sum_squares<HALF>(x));
    }
  }
  // sign flip, then the stage across the halves: the low lane keeps
  // x_i + x_{i + d/2}, the high lane x_i - x_{i + d/2}
#pragma unroll
  for (int j4 = 0; j4 < HALF / 4; ++j4) {
    const uint4 m4 = fmask[h * (HALF / 4) + j4];
    const uint32_t ms[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * j4 + e;
      uint32_t a = __float_as_uint(x[j]) ^ ms[e], b = a;
      swap_halves(a, b);   // a: the low lane's value, b: the high lane's value
      x[j] = fmaf(__uint_as_float(b), sgn, __uint_as_float(a));
    }
  }
#pragma unroll
  for (int hh = 1; hh < HALF; hh <<= 1) {
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      if ((i & hh) == 0) {
        const float a = x[i], b = x[i + hh];
        x[i] = a + b;
        x[i + hh] = a - b;
      }
    }
  }
  return sqrtf(nu2);
}

// Loads the fp16 input of tile t for this lane through a buffer descriptor
// over the tile's rows: 32-bit offsets, and rows past the end (or a tile
// past the end) read as zeros with no branch.  t is wave-uniform.
template <int D>
__device__ __forceinline__ void half_load(const EncodeParams& p, int64_t t, uint32_t (&dst)[D / 4]) {
  constexpr int NP = D / 4;
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const int64_t r0 = t * 32;
  const int64_t left = p.n_rows - r0;
  const uint32_t rows = left <= 0 ? 0u : (left < 32 ? (uint32_t)left : 32u);
  const _Float16* base = reinterpret_cast<const _Float16*>(p.x) + (left > 0 ? r0 * p.x_stride : 0);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)base, (short)0, (int)(rows * (uint32_t)p.x_stride * 2u), 0x00020000);
  const uint32_t off = ((uint32_t)(lane & 31) * (uint32_t)p.x_stride + (uint32_t)(h * (D / 2))) * 2u;
#pragma unroll
  for (int j = 0; j < NP / 4; ++j) {
    const u4v v = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * j, 0, 0);
    dst[4 * j] = v[0]; dst[4 * j + 1] = v[1]; dst[4 * j + 2] = v[2]; dst[4 * j + 3] = v[3];
  }
}

// One wave's tiles: tile, tile + tstride, ...  With PF the input of the
// next tile is loaded while the current one is processed, and nxt holds
// the first tile's input on entry.
template <int D, int CB, bool PROD, bool PF, bool MROT = false, bool F32IN = false>
__device__ __forceinline__ void half_tiles(const EncodeParams& p, const HalfTables<D, CB, PROD, MROT, F32IN>& T,
                                           int64_t tile, int64_t tstride, uint32_t (&nxt)[D / 4]) {
  static_assert(!F32IN || (!PF && !MROT), "fp32 input: no prefetch, butterflies in registers");
  constexpr int NLEV = 1 << CB;
  constexpr int NTH = NLEV - 1;
  constexpr int HALF = D / 2;              // coordinates per lane
  constexpr int NP = D / 4;                // packed fp16 pairs per lane
  constexpr int HW = HALF * CB / 32;       // code words per lane (half a row)
  constexpr int ROW_BYTES = D * CB / 8;
  constexpr int HB = ROW_BYTES / 2;
  constexpr int HALIGN = HB % 16 == 0 ? 16 : (HB % 8 == 0 ? 8 : 4);
  constexpr bool USE_LUT = CB >= 3;
  constexpr int KS = D / 16, MT = D / 32;
  (void)NTH;
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const float sgn = h ? -1.f : 1.f;
  const int64_t ntiles = (p.n_rows + 31) / 32;
  const float lut_a = p.lut_a, lut_b = p.lut_b;
  const float cscale = PROD ? 256.f : 1.f;
  auto load_tile = [&](int64_t t, uint32_t (&dst)[NP]) { half_load<D>(p, t, dst); };
  for (; tile < ntiles; tile += tstride) {
    const int64_t row = tile * 32 + (lane & 31);
    const bool valid = row < p.n_rows;
    float x[HALF];
    float nu_s, nu_out;
    if constexpr (F32IN) {
      // x may come back scaled by a power of two (nu_s is its norm)
      float pre_inv;
      nu_s = f32_rotate_half<D>(p, T.fmask, tile, sgn, x, pre_inv);
      nu_out = nu_s * pre_inv;
    } else {
    uint32_t u[NP];
    if (PF) {
#pragma unroll
      for (int j = 0; j < NP; ++j) u[j] = nxt[j];
    } else {
      half_load<D>(p, tile, u);
    }
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    float acc[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) acc[a] = 0.f;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const h2_t hv = __builtin_bit_cast(h2_t, u[j]);
      acc[j & 7] = __builtin_amdgcn_fdot2(hv, hv, acc[j & 7], false);
    }
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
      for (int a = 0; a < w; ++a) acc[a] += acc[a + w];
    const float nu2 = cross_sum(acc[0]);
    // a non-finite input encodes as the zero vector (its norm stays non-finite)
    if (!(nu2 <= 3.0e38f)) {
#pragma unroll
      for (int j = 0; j < NP; ++j) u[j] = 0u;
    }
    nu_s = sqrtf(nu2);
    nu_out = nu_s;

    if constexpr (MROT) {
      // y = H D x on the matrix cores: B = the lane's own input (k slot j of
      // lane half h at step ks is coordinate (d/2) h + 8 ks + j), A = the
      // H D fragments; fp16 input times +-1 is exact, sums in fp32
      f32x16 acc_y[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_y[mt][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const half8_t bx = __builtin_bit_cast(half8_t, make_uint4(u[4 * ks], u[4 * ks + 1], u[4 * ks + 2], u[4 * ks + 3]));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int sgn = __builtin_popcount(mt & (ks >> 1)) & 1;
          const half8_t ahd = __builtin_bit_cast(half8_t, T.hd[(2 * ks + sgn) * kWave + lane]);
          acc_y[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahd, bx, acc_y[mt], 0, 0, 0);
        }
      }
      if (PF) load_tile(tile + tstride, nxt);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[16 * mt + v] = acc_y[mt][v];
    } else {
      // sign flip, the stage across the halves, and the stage on bit 0
#pragma unroll
      for (int j4 = 0; j4 < NP / 4; ++j4) {
        const uint4 m4 = T.hmask[h * (NP / 4) + j4];
        const uint32_t ms[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * j4 + e;
          uint32_t a = u[j] ^ ms[e], b = a;
          swap_halves(a, b);   // a: the low lane's pair, b: the high lane's pair
          float t0, t1;
          asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,1]" : "=v"(t0) : "v"(b), "v"(sgn), "v"(a));
          asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(t1) : "v"(b), "v"(sgn), "v"(a));
          x[2 * j] = t0 + t1;
          x[2 * j + 1] = t0 - t1;
        }
      }
      if (PF) load_tile(tile + tstride, nxt);
#pragma unroll
      for (int hh = 2; hh < HALF; hh <<= 1) {
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
          if ((i & hh) == 0) {
            const float a = x[i], b = x[i + hh];
            x[i] = a + b;
            x[i + hh] = a - b;
          }
        }
      }
    }
    }
    __builtin_amdgcn_sched_barrier(0);

    const bool live = nu_s > 0.f && nu_s <= 3.0e38f;
    const float inv = live ? 1.0f / (sqrtf((float)D) * nu_s) : 0.f;
    const float inv_p = inv * cscale;
    const float ua = lut_a * inv;
    uint32_t words[HW];
#pragma unroll
    for (int j = 0; j < HW; ++j) words[j] = 0u;
    auto quantize = [&](int i) -> float {
      int c;
      float r = 0.f;
      if constexpr (USE_LUT) {
        const float uu = fmaf(x[i], ua, lut_b);
        const float2 e = T.lut[(uint32_t)uu];
        c = __float_as_int(e.y) + (uu >= e.x ? 1 : 0);
        if constexpr (PROD) r = fmaf(x[i], inv_p, -T.cent[c]);
      } else {
        const float z = x[i] * inv_p;
        c = 0;
#pragma unroll
        for (int k = 0; k < NTH; ++k) c += (z >= p.codec.thresholds[k] * cscale) ? 1 : 0;
        if constexpr (PROD) r = z - T.cent[c];
      }
      const int off = i * CB;
      words[off >> 5] |= (uint32_t)c << (off & 31);
      if ((off & 31) + CB > 32) words[(off >> 5) + 1] |= (uint32_t)c >> (32 - (off & 31));
      return r;
    };
    uint8_t* idx_dst = p.idx + row * ROW_BYTES + h * HB;

    if constexpr (!PROD) {
#pragma unroll
      for (int i = 0; i < HALF; ++i) quantize(i);
      if (valid) {
        store_words<HW, HALIGN>(idx_dst, words);
        if (h == 0) p.norm[row] = nu_out;
      }
    } else {
      uint32_t bh[KS][4], bl[KS][4];
      float g2[2] = {0.f, 0.f};
      // S r' on the matrix cores, two 32-row tiles of S (mp) at a time: the
      // six products of step ks (S_hi r_hi + S_hi r_lo + S_lo r_hi for both
      // tiles)
      auto project = [&](int mp, int ks, f32x16& c0, f32x16& c1) {
        const int f0 = (2 * mp) * KS + ks, f1 = (2 * mp + 1) * KS + ks;
        const half8_t a0h = __builtin_bit_cast(half8_t, T.frag[(2 * f0) * kWave + lane]);
        const half8_t a0l = __builtin_bit_cast(half8_t, T.frag[(2 * f0 + 1) * kWave + lane]);
        const half8_t a1h = __builtin_bit_cast(half8_t, T.frag[(2 * f1) * kWave + lane]);
        const half8_t a1l = __builtin_bit_cast(half8_t, T.frag[(2 * f1 + 1) * kWave + lane]);
        const half8_t rh = __builtin_bit_cast(half8_t, make_uint4(bh[ks][0], bh[ks][1], bh[ks][2], bh[ks][3]));
        const half8_t rl = __builtin_bit_cast(half8_t, make_uint4(bl[ks][0], bl[ks][1], bl[ks][2], bl[ks][3]));
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0h, rh, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1h, rh, c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0h, rl, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1h, rl, c1, 0, 0, 0);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0l, rh, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1l, rh, c1, 0, 0, 0);
      };
      // register v of lane half h holds row 16 h + v of the tile; bit =
      // [p >= 0] (a result of exactly -0 reads as negative; it needs r = 0)
      auto sign_words = [&](const f32x16& c0, const f32x16& c1, uint32_t& s0, uint32_t& s1) {
        uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
        for (int v = 15; v >= 0; --v) {
          w0 = __builtin_amdgcn_alignbit(w0, __float_as_uint(c0[v]), 31);
          w1 = __builtin_amdgcn_alignbit(w1, __float_as_uint(c1[v]), 31);
        }
        w0 = (w0 ^ 0xFFFFu) << (16 * h);
        w1 = (w1 ^ 0xFFFFu) << (16 * h);
        uint32_t a0 = w0, b0 = w0, a1 = w1, b1 = w1;
        swap_halves(a0, b0);
        swap_halves(a1, b1);
        s0 = a0 | b0;
        s1 = a1 | b1;
      };
      uint32_t sw[MT];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          r[e] = quantize(8 * ks + e);
          g2[e & 1] = fmaf(r[e], r[e], g2[e & 1]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) split_pair(r[2 * j], r[2 * j + 1], bh[ks][j], bl[ks][j]);
        // pin the code words and the packed fragments here: left alone, the
        // compiler sinks their assembly to the first use and keeps the
        // compare masks and unpacked fp32 parts alive until then
#pragma unroll
        for (int j = 0; j < HW; ++j) asm volatile("" : "+v"(words[j]));
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(bh[ks][j]), "+v"(bl[ks][j]));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (valid) {
        store_words<HW, HALIGN>(idx_dst, words);
        if (h == 0) p.norm[row] = nu_out;
      }
      const float gamma2 = cross_sum(g2[0] + g2[1]);
      if (valid && h == 0) p.rnorm[row] = sqrtf(gamma2) * (1.f / 256.f);

#pragma unroll 1
      for (int mp = 0; mp < MT / 2; ++mp) {
        f32x16 c0 = {}, c1 = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          project(mp, ks, c0, c1);
          __builtin_amdgcn_sched_barrier(0);
        }
        uint32_t s0, s1;
        sign_words(c0, c1, s0, s1);
#pragma unroll
        for (int t = 0; t < MT / 2; ++t) {
          if (t == mp) {
            sw[2 * t] = s0;
            sw[2 * t + 1] = s1;
          }
        }
      }
      // lane half h stores words h MT/2 .. h MT/2 + MT/2 - 1
      if (valid) {
        uint32_t* qdst = reinterpret_cast<uint32_t*>(p.qjl + row * (D / 8)) + h * (MT / 2);
        if constexpr (MT == 4) {
          *reinterpret_cast<uint2*>(qdst) = make_uint2(h ? sw[2] : sw[0], h ? sw[3] : sw[1]);
        } else {
          *qdst = h ? sw[1] : sw[0];
        }
      }
    }
  }
}

template <int D, int CB, bool PROD, bool F32IN>
__global__ __launch_bounds__((HalfLaunch<PROD, F32IN>::kWaves * kWave), (HalfLaunch<PROD, F32IN>::kMinWavesPerEU)) void encode_half_kernel(EncodeParams p) {
  constexpr int kHalfWaves = HalfLaunch<PROD, F32IN>::kWaves;
  constexpr bool PF = HalfLaunch<PROD, F32IN>::kPrefetch;
  __shared__ HalfTables<D, CB, PROD, false, F32IN> T;
  const int tid = threadIdx.x;
  const EncodeParams* kp = (const EncodeParams*)__builtin_amdgcn_kernarg_segment_ptr();
  const int64_t tstride = (int64_t)gridDim.x * kHalfWaves;
  const int64_t tile = (int64_t)blockIdx.x * kHalfWaves + __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t nxt[D / 4];
  // the first tile's input is in flight during the set-up
  if (PF) half_load<D>(p, tile, nxt);
  half_setup<D, CB, PROD, false, F32IN>(p, kp, T, tid, blockDim.x);
  __syncthreads();
  half_tiles<D, CB, PROD, PF, false, F32IN>(p, T, tile, tstride, nxt);
}

// Keys (prod) and values (mse) of one call in one launch.  Each SIMD runs
// two key waves and one value wave: the value waves' loads and stores
// overlap the key waves' arithmetic.  Waves 0..7 of a workgroup encode key
// tiles, waves 8..11 value tiles (measured against 6 + 6, 4 + 8 and 9 + 3).
// Only the value waves load their next tile ahead: the key waves'
// registers leave no room for it at three waves per SIMD.
struct EncodeKVParams {
  EncodeParams k, v;
};
constexpr int kKVKeyWaves = 8, kKVValWaves = 4;
static_assert(sizeof(EncodeKVParams) <= 4096, "kernel argument segment");

// The value waves rotate on the matrix cores (H D as a +-1 matrix times
// the fp16 input): it moves their butterflies off the vector ALU, which the
// key waves keep busy.  The key waves keep the butterflies (their matrix
// cores already run the S r products).
constexpr bool kKVRotK = false, kKVRotV = true;

template <int D, int CBK, int CBV>
__global__ __launch_bounds__((kKVKeyWaves + kKVValWaves) * kWave, 3) void encode_kv_half_kernel(EncodeKVParams pp) {
  __shared__ HalfTables<D, CBK, true, kKVRotK> TK;
  __shared__ HalfTables<D, CBV, false, kKVRotV> TV;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const EncodeKVParams* kpp = (const EncodeKVParams*)__builtin_amdgcn_kernarg_segment_ptr();
  const bool key_wave = wave < kKVKeyWaves;
  const int64_t vtile = (int64_t)blockIdx.x * kKVValWaves + (wave - kKVKeyWaves);
  uint32_t nxt[D / 4];
  // a value wave's first tile is in flight during the set-up
  if (!key_wave) half_load<D>(pp.v, vtile, nxt);
  half_setup<D, CBK, true, kKVRotK>(pp.k, &kpp->k, TK, tid, blockDim.x);
  half_setup<D, CBV, false, kKVRotV>(pp.v, &kpp->v, TV, tid, blockDim.x);
  __syncthreads();
  if (key_wave)
    half_tiles<D, CBK, true, false, kKVRotK>(pp.k, TK, (int64_t)blockIdx.x * kKVKeyWaves + wave,
                                             (int64_t)gridDim.x * kKVKeyWaves, nxt);
  else
    half_tiles<D, CBV, false, true, kKVRotV>(pp.v, TV, vtile, (int64_t)gridDim.x * kKVValWaves, nxt);
}

template <int D, int CB, bool PROD, bool F32IN>
static hipError_t run_half(const EncodeParams& p, hipStream_t stream) {
  constexpr int kHalfWaves = HalfLaunch<PROD, F32IN>::kWaves;
  // occupancy depends only on the kernel's resources (one code object for
  // every device): computed once, read by any host thread
  static std::atomic<int> per_cu{0};
  if (per_cu.load(std::memory_order_relaxed) == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, encode_half_kernel<D, CB, PROD, F32IN>,
                                                     kHalfWaves * kWave, 0) != hipSuccess || nb < 1)
      nb = 1;
    per_cu.store(nb, std::memory_order_relaxed);
  }
  const int64_t ntiles = (p.n_rows + 31) / 32;
  int64_t blocks = (ntiles + kHalfWaves - 1) / kHalfWaves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu.load(std::memory_order_relaxed);
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((encode_half_kernel<D, CB, PROD, F32IN>), dim3((unsigned)blocks),
                     dim3(kHalfWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool PROD, bool F32IN = false>
static hipError_t pick_half(int cb, const EncodeParams& p, hipStream_t s) {
  switch (cb) {
    case 1: return run_half<D, 1, PROD, F32IN>(p, s);
    case 2: return run_half<D, 2, PROD, F32IN>(p, s);
    case 3: return run_half<D, 3, PROD, F32IN>(p, s);
    case 4: return run_half<D, 4, PROD, F32IN>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int CB, bool PROD, typename T, bool ROPE>
static hipError_t run_encode(const EncodeParams& p, hipStream_t stream) {
  const int64_t ntiles = (p.n_rows + kWave - 1) / kWave;
  int64_t blocks = (ntiles + kEncWaves - 1) / kEncWaves;
  const int64_t cap = (int64_t)device_cu_count() * 4;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((encode_kernel<D, CB, PROD, T, ROPE>), dim3((unsigned)blocks),
                     dim3(kEncWaves * kWave), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool PROD, typename T, bool ROPE>
static hipError_t pick_cb(int cb, const EncodeParams& p, hipStream_t s) {
  switch (cb) {
    case 1: return run_encode<D, 1, PROD, T, ROPE>(p, s);
    case 2: return run_encode<D, 2, PROD, T, ROPE>(p, s);
    case 3: return run_encode<D, 3, PROD, T, ROPE>(p, s);
    case 4: return run_encode<D, 4, PROD, T, ROPE>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t pick_rest(const tq_codec& c, int dtype, bool rope, const EncodeParams& p, hipStream_t s) {
  const bool prod = c.mode == TQ_PROD;
  if (dtype == TQ_F32) {
    if (rope) return hipErrorInvalidValue;  // RoPE inputs are fp16 in this build
    // d = 128: two lanes per vector (one lane would need more than 256
    // registers for the row, its codes and the projection's operands)
    if constexpr (D == 128)
      return prod ? pick_half<D, true, true>(c.code_bits, p, s) : pick_half<D, false, true>(c.code_bits, p, s);
    else
      return prod ? pick_cb<D, true, float, false>(c.code_bits, p, s)
                  : pick_cb<D, false, float, false>(c.code_bits, p, s);
  }
  if (rope) {
    if constexpr (D == 64)
      return prod ? pick_cb<D, true, _Float16, true>(c.code_bits, p, s)
                  : pick_cb<D, false, _Float16, true>(c.code_bits, p, s);
    return hipErrorInvalidValue;
  }
  return prod ? pick_half<D, true>(c.code_bits, p, s) : pick_half<D, false>(c.code_bits, p, s);
}

// Smallest grid (G cells over z in [-1.01, 1.01], one cell of margin on
// each side) in which no two thresholds share a cell, with the cell of a
// threshold computed exactly as the kernel computes it.
static bool build_grid(const tq_codec& c, EncodeParams& p) {
  const int nth = (1 << c.code_bits) - 1;
  for (int G = 32; G <= kLutMax; G *= 2) {
    const float a = (float)((G / 2 - 1) / (double)kGridRange);
    const float b = (float)(G / 2);
    bool ok = true;
    int prev = -1;
    for (int k = 0; k < nth && ok; ++k) {
      const float tu = std::fmaf(c.thresholds[k], a, b);
      if (!(tu >= 0.f && tu < (float)G)) { ok = false; break; }
      const int cell = (int)tu;
      if (cell <= prev) ok = false;
      prev = cell;
    }
    if (ok) {
      p.lut_g = G;
      p.lut_a = a;
      p.lut_b = b;
      return true;
    }
  }
  return false;
}

// Kernel arguments for one codec (false: no quantizer grid fits).
static bool fill_params(const tq_codec& c, const void* x, int64_t n_rows, const RopeHost& rope,
                        const tq_packed& out, EncodeParams& p, int64_t x_stride = 0) {
  p = {};
  p.x = x;
  p.x_stride = x_stride > 0 ? x_stride : c.d;
  // the two-lanes-per-vector kernels address a 32-row tile with 32-bit offsets
  if (p.x_stride > (int64_t)1 << 24) return false;
  p.n_rows = n_rows;
  p.idx = out.idx;
  p.qjl = out.qjl;
  p.norm = out.norm;
  p.rnorm = out.rnorm;
  for (int k = 0; k < 16; ++k) {
    p.codec.centroids[k] = c.centroids[k];
    p.codec.thresholds[k] = c.thresholds[k];
  }
  for (int w = 0; w < 48; ++w) p.codec.flip[w] = c.flip[w];
  for (int j = 0; j < 64 && 2 * j + 1 < c.d; ++j) {
    const uint32_t b0 = (c.flip[(2 * j) >> 5] >> ((2 * j) & 31)) & 1u;
    const uint32_t b1 = (c.flip[(2 * j + 1) >> 5] >> ((2 * j + 1) & 31)) & 1u;
    p.hflip[j] = (b0 << 15) | (b1 << 31);
  }
  p.codec.S = c.S;
  p.codec.d = c.d;
  p.codec.code_bits = c.code_bits;
  p.codec.mode = c.mode;
  p.codec.m = c.m;
  p.seq_len = rope.on ? rope.seq_len : 1;
  if (rope.on) {
    for (int i = 0; i < c.d / 2 && i < 64; ++i)
      p.theta[i] = std::pow((double)rope.base, -2.0 * i / (double)c.d);
  }
  return c.code_bits < 3 || build_grid(c, p);
}

hipError_t launch_encode(const tq_codec& c, const void* x, int dtype, int64_t n_rows,
                         const RopeHost& rope, const tq_packed& out, void* workspace,
                         hipStream_t stream, int64_t x_stride) {
  if (n_rows == 0) return hipSuccess;
  if (c.d == 1536) {
    if (x_stride != 0 && x_stride != c.d) return hipErrorInvalidValue;
    return launch_wide_encode(c, x, dtype, n_rows, out, workspace, stream);
  }
  EncodeParams p;
  if (!fill_params(c, x, n_rows, rope, out, p, x_stride)) return hipErrorInvalidValue;
  if (c.d == 128) return pick_rest<128>(c, dtype, rope.on, p, stream);
  if (c.d == 64) return pick_rest<64>(c, dtype, rope.on, p, stream);
  return hipErrorInvalidValue;
}

template <int D, int CBK, int CBV>
static hipError_t run_kv_half(const EncodeKVParams& pp, hipStream_t stream) {
  // occupancy depends only on the kernel's resources (one code object for
  // every device): computed once, read by any host thread
  static std::atomic<int> per_cu{0};
  constexpr int kThreads = (kKVKeyWaves + kKVValWaves) * kWave;
  if (per_cu.load(std::memory_order_relaxed) == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, encode_kv_half_kernel<D, CBK, CBV>, kThreads, 0) !=
            hipSuccess || nb < 1)
      nb = 1;
    per_cu.store(nb, std::memory_order_relaxed);
  }
  // enough workgroups for every key wave to have a tile, at most what fits
  const int64_t ntiles = (pp.k.n_rows + 31) / 32;
  int64_t blocks = (ntiles + kKVKeyWaves - 1) / kKVKeyWaves;
  const int64_t cap = (int64_t)device_cu_count() * per_cu.load(std::memory_order_relaxed);
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((encode_kv_half_kernel<D, CBK, CBV>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, pp);
  return hipGetLastError();
}

template <int D>
static hipError_t pick_kv(int cbk, int cbv, const EncodeKVParams& pp, hipStream_t s) {
  if constexpr (D == 64) {
    switch (cbk * 8 + cbv) {
      case 1 * 8 + 2: return run_kv_half<D, 1, 2>(pp, s);
      case 1 * 8 + 3: return run_kv_half<D, 1, 3>(pp, s);
      case 1 * 8 + 4: return run_kv_half<D, 1, 4>(pp, s);
    }
  }
  switch (cbk * 8 + cbv) {
    case 2 * 8 + 2: return run_kv_half<D, 2, 2>(pp, s);
    case 2 * 8 + 3: return run_kv_half<D, 2, 3>(pp, s);
    case 2 * 8 + 4: return run_kv_half<D, 2, 4>(pp, s);
    case 3 * 8 + 2: return run_kv_half<D, 3, 2>(pp, s);
    case 3 * 8 + 3: return run_kv_half<D, 3, 3>(pp, s);
    case 3 * 8 + 4: return run_kv_half<D, 3, 4>(pp, s);
  }
  return hipErrorNotSupported;
}

bool encode_kv_fusable(const tq_codec& kc, const tq_codec& vc, int dtype, bool rope) {
  if (dtype != TQ_F16 || rope || kc.d != vc.d || (kc.d != 64 && kc.d != 128)) return false;
  if (kc.mode != TQ_PROD || vc.mode != TQ_MSE) return false;
  // (1-bit key tables at d = 128 would spill at three waves per SIMD)
  const int kmin = kc.d == 128 ? 2 : 1;
  return kc.code_bits >= kmin && kc.code_bits <= 3 && vc.code_bits >= 2 && vc.code_bits <= 4;
}

hipError_t launch_encode_kv(const tq_codec& kc, const tq_codec& vc, const void* k, const void* v,
                            int64_t n_rows, const tq_packed& kout, const tq_packed& vout,
                            hipStream_t stream, int64_t x_stride) {
  if (n_rows == 0) return hipSuccess;
  EncodeKVParams pp;
  if (!fill_params(kc, k, n_rows, RopeHost{}, kout, pp.k, x_stride) ||
      !fill_params(vc, v, n_rows, RopeHost{}, vout, pp.v, x_stride))
    return hipErrorInvalidValue;
  if (kc.d == 128) return pick_kv<128>(kc.code_bits, vc.code_bits, pp, stream);
  return pick_kv<64>(kc.code_bits, vc.code_bits, pp, stream);
}

}  // namespace tqk
