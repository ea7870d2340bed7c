// TurboQuant encode for gfx950, d = 64 or 128: one vector per lane.
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
// r is scaled by 2^8 before the split so that its low part stays a normal
// fp16 number; the sign of S r does not change.
//
// Layout of a wave's tile: lane l owns row 64*tile + l.  The MFMA B operand
// for 32 tokens needs, in lane l, token l%32 and the k-group l/32; the two
// 32-token blocks of a tile are exchanged between wave halves with one
// v_permlane32_swap per packed register, and the sign words are put back on
// their owning lanes the same way.

#include "device_common.hpp"
#include "internal.hpp"

namespace tqk {

constexpr int kEncWaves = 8;

struct EncodeParams {
  const void* x;
  int64_t n_rows;
  uint8_t* idx;
  uint8_t* qjl;
  float* norm;
  float* rnorm;
  CodecArgs codec;
  int64_t seq_len;
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

template <int D, int CB, bool PROD, typename T, bool ROPE>
__global__ __launch_bounds__(kEncWaves * kWave) void encode_kernel(EncodeParams p) {
  constexpr int NLEV = 1 << CB;
  constexpr int NTH = NLEV - 1;
  constexpr int W = D * CB / 32;          // code words per row
  constexpr int ROW_BYTES = D * CB / 8;
  constexpr int ALIGN = ROW_BYTES % 16 == 0 ? 16 : (ROW_BYTES % 8 == 0 ? 8 : 4);
  using G = ProdGeom<D>;

  __shared__ float s_cent[16];
  __shared__ double s_theta[ROPE ? D / 2 : 1];
  __shared__ uint4 s_frag[PROD ? G::FRAGS * 2 * kWave : 1];

  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (tid == k) s_cent[k] = p.codec.centroids[k];
  if constexpr (ROPE) {
#pragma unroll
    for (int k = 0; k < D / 2; ++k)
      if (tid == k) s_theta[k] = p.theta[k];
  }

  if constexpr (PROD) {
    // S_hi / S_lo as MFMA A fragments: fragment (mt, ks), lane l holds
    // S[32 mt + l%32][16 ks + 8 (l/32) + j], j = 0..7.
    for (int t = tid; t < G::FRAGS * kWave; t += blockDim.x) {
      const int lane = t & 63, f = t >> 6;
      const int mt = f / G::KS, ks = f % G::KS;
      const int m = 32 * mt + (lane & 31);
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

  for (int64_t tile = (int64_t)blockIdx.x * kEncWaves + wave; tile < ntiles;
       tile += (int64_t)gridDim.x * kEncWaves) {
    const int64_t row = tile * kWave + lane;
    const bool valid = row < p.n_rows;
    float x[D];
    if (valid) {
      load_row<D, T>(xin + row * D, x);
    } else {
#pragma unroll
      for (int i = 0; i < D; ++i) x[i] = 0.f;
    }
    if constexpr (ROPE) rope_inplace<D>(x, row % p.seq_len, s_theta);

    // nu = |x|.  When the squares leave the normal fp32 range (only fp32
    // inputs get there) the vector is first scaled exactly by the power of
    // two that brings its largest entry into [0.5, 1).
    float nu2 = sum_squares<D>(x);
    float pre_inv = 1.f;
    if (!(nu2 >= 0x1p-100f && nu2 <= 0x1p100f)) {
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) mx = fmaxf(mx, fabsf(x[i]));
      if (mx > 0.f && mx <= 3.4e38f) {
        int e;
        frexpf(mx, &e);
        const float sc = ldexpf(1.f, -e);
        pre_inv = ldexpf(1.f, e);
#pragma unroll
        for (int i = 0; i < D; ++i) x[i] *= sc;
        nu2 = sum_squares<D>(x);
      }
    }
    const float nu_s = sqrtf(nu2);
    const float nu = nu_s * pre_inv;

    flip_signs<D>(x, p.codec.flip);
    wht_inreg<D>(x);
    const float inv = nu_s > 0.f ? 1.0f / (sqrtf((float)D) * nu_s) : 0.f;

    // quantize and pack; x keeps z for the residual
    uint32_t words[W];
#pragma unroll
    for (int j = 0; j < W; ++j) words[j] = 0u;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const float z = x[i] * inv;
      int c = 0;
#pragma unroll
      for (int k = 0; k < NTH; ++k) c += (z >= p.codec.thresholds[k]) ? 1 : 0;
      const int off = i * CB;
      words[off >> 5] |= (uint32_t)c << (off & 31);
      if ((off & 31) + CB > 32) words[(off >> 5) + 1] |= (uint32_t)c >> (32 - (off & 31));
      x[i] = z;
    }
    if (valid) {
      store_words<W, ALIGN>(p.idx + row * ROW_BYTES, words);
      p.norm[row] = nu;
    }

    if constexpr (PROD) {
      // Residual r = z - c[idx] and, 16 coordinates at a time, the B
      // fragments: X = r[16ks .. 16ks+7], Y = r[16ks+8 .. 16ks+15] (scaled by
      // 2^8, split hi/lo); after the half-wave swap X holds block 0 (tokens
      // of lanes 0..31) and Y block 1 (tokens of lanes 32..63).
      uint32_t b0h[G::KS][4], b1h[G::KS][4], b0l[G::KS][4], b1l[G::KS][4];
      float g2[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < G::KS; ++ks) {
        float r[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int i = 16 * ks + e;
          r[e] = x[i] - s_cent[get_code<CB, W>(words, i)];
          g2[e & 3] = fmaf(r[e], r[e], g2[e & 3]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float xa = r[2 * j] * 256.f, xb = r[2 * j + 1] * 256.f;
          const float ya = r[8 + 2 * j] * 256.f, yb = r[8 + 2 * j + 1] * 256.f;
          const _Float16 xah = (_Float16)xa, xbh = (_Float16)xb, yah = (_Float16)ya, ybh = (_Float16)yb;
          uint32_t xh = pack_h2(xah, xbh), yh = pack_h2(yah, ybh);
          uint32_t xl = pack_h2((_Float16)(xa - (float)xah), (_Float16)(xb - (float)xbh));
          uint32_t yl = pack_h2((_Float16)(ya - (float)yah), (_Float16)(yb - (float)ybh));
          swap_halves(xh, yh);
          swap_halves(xl, yl);
          b0h[ks][j] = xh; b1h[ks][j] = yh;
          b0l[ks][j] = xl; b1l[ks][j] = yl;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (valid) p.rnorm[row] = sqrtf((g2[0] + g2[1]) + (g2[2] + g2[3]));

      uint32_t sign_words[4] = {0u, 0u, 0u, 0u};
      const uint32_t half_shift = 4u * (uint32_t)(lane >> 5);
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
        // C layout: lane l holds column l%32, rows 8 (v/4) + 4 (l/32) + v%4
        uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int pos = 8 * (v >> 2) + (v & 3);
          w0 |= (c0[v] >= 0.f ? 1u : 0u) << pos;
          w1 |= (c1[v] >= 0.f ? 1u : 0u) << pos;
        }
        w0 <<= half_shift;
        w1 <<= half_shift;
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
    return prod ? pick_cb<D, true, float, false>(c.code_bits, p, s)
                : pick_cb<D, false, float, false>(c.code_bits, p, s);
  }
  if (rope) {
    if constexpr (D == 64)
      return prod ? pick_cb<D, true, _Float16, true>(c.code_bits, p, s)
                  : pick_cb<D, false, _Float16, true>(c.code_bits, p, s);
    return hipErrorInvalidValue;
  }
  return prod ? pick_cb<D, true, _Float16, false>(c.code_bits, p, s)
              : pick_cb<D, false, _Float16, false>(c.code_bits, p, s);
}

hipError_t launch_encode(const tq_codec& c, const void* x, int dtype, int64_t n_rows,
                         const RopeHost& rope, const tq_packed& out, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  EncodeParams p = {};
  p.x = x;
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
  if (c.d == 128) return pick_rest<128>(c, dtype, rope.on, p, stream);
  if (c.d == 64) return pick_rest<64>(c, dtype, rope.on, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace tqk
