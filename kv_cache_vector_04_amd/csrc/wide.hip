// Wide vectors, d = 1536 = 12 x 128: encode, query preparation and the
// inner-product scan.
//
// Rotation.  Pi u = H (D * u) / sqrt(d) with H = H_12 (x) H_128: H_128 in
// Sylvester order inside each 128-coordinate chunk, H_12 the Paley Hadamard
// matrix of order 12 (first construction, q = 11) across the chunks;
// coordinate i = 128 a + c.  ("Ablazione, Inferenza Statistica e Validazione
// per la Compressione della KV-Cache", "Configurazione Sperimentale": the
// randomized Walsh-Hadamard rotation; 1536 is not a power of two, so the
// order-12 factor is needed.)
//
// Encode (one wavefront per vector).  Lane l holds coordinates
// 128 a + 2 l + e (a < 12, e < 2): coalesced 8-byte loads per chunk, the
// first H_128 stage inside the lane, the other six across lanes, H_12 inside
// the lane over a.  Codes go through LDS bytes into the packed row.  For
// TurboQuant_prod the residual r = z - c[idx] is written as fp16 hi / lo
// planes and the QJL projection S r of a block of vectors is one MFMA
// product ("Google presenta TurboQuant ...", "Eliminación del sesgo interno
// del producto"): P = S R^T with S (1536 x 1536) and R (vectors x 1536) both
// split into fp16 hi + lo, accumulating hi.hi + hi.lo + lo.hi in fp32, and
// the sign bits packed in the epilogue.
//
// Scan.  est(a, j) = nu_j (<q_rot, c[idx_j]> + sqrt(pi/2)/m gamma_j
// <S q_rot, 2 sigma_j - 1>) ("Velocidad y eficiencia de indexación") is a
// product of the fp16 hi / lo query planes (A operand) with operands built
// from the packed bits (B operand): for 1-bit codes and for the QJL bits the
// B values are +-1, exact in fp16; wider codes use a pair table of
// c / c_max split into hi + lo.

#include <cmath>
#include <cstddef>

#include "device_common.hpp"
#include "internal.hpp"

namespace tqk {

constexpr int kWD = 1536;
constexpr int kWA = 12;                  // 128-coordinate chunks

// ---- Paley H_12 -------------------------------------------------------------
// chi: quadratic character mod 11.  H_12 = I + [[0, 1^T], [-1, Q]] with the
// Jacobsthal matrix Q[i][j] = chi(j - i) (i, j < 11).
constexpr int chi11(int a) {
  a %= 11;
  if (a < 0) a += 11;
  if (a == 0) return 0;
  for (int x = 1; x < 11; ++x)
    if ((x * x) % 11 == a) return 1;
  return -1;
}
constexpr int paley12(int a, int b) {
  const int s = a == 0 ? (b == 0 ? 0 : 1) : (b == 0 ? -1 : chi11(b - a));
  return (a == b ? 1 : 0) + s;
}
struct H12Signs {
  int8_t v[kWA][kWA];
};
constexpr H12Signs make_h12() {
  H12Signs t{};
  for (int a = 0; a < kWA; ++a)
    for (int b = 0; b < kWA; ++b) t.v[a][b] = (int8_t)paley12(a, b);
  return t;
}
__device__ constexpr H12Signs kH12 = make_h12();

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define TQ_KARG(P, FIELD) \
  ((const char*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(P, FIELD))

__device__ __forceinline__ uint32_t h2_bits(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// hi / lo fp16 split of two floats: hi = fp16(x), lo = fp16(x - hi)
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  hi = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
  lo = h2_bits(a - (float)ha, b - (float)hb);
}

// ---- transform: norm, rotation, codes, residual planes ----------------------
struct WideXParams {
  const void* x;        // [n][1536] fp16 or fp32
  int64_t n;
  uint8_t* idx;         // rows of 192 * CB bytes
  float* norm;
  float* rnorm;
  _Float16* rh;         // [n][1536] residual (prod) or q_rot (query): hi
  _Float16* rl;         //                                               lo
  float inv_sqrt_d;
  float centroids[16];
  float thresholds[16];
  uint32_t flip[48];
};

enum { kWMse = 0, kWProd = 1, kWQuery = 2 };
constexpr int kXWaves = 4;

template <typename T, int CB, int MODE>
__global__ __launch_bounds__(64 * kXWaves) void wide_transform_kernel(WideXParams p) {
  __shared__ uint32_t s_flip[48];
  __shared__ float s_cent[16];
  __shared__ __align__(16) uint8_t s_code[kXWaves][kWD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 48) s_flip[tid] = reinterpret_cast<const uint32_t*>(TQ_KARG(WideXParams, flip))[tid];
  if (tid < 16) s_cent[tid] = reinterpret_cast<const float*>(TQ_KARG(WideXParams, centroids))[tid];
  __syncthreads();

  for (int64_t row = (int64_t)blockIdx.x * kXWaves + wave; row < p.n;
       row += (int64_t)gridDim.x * kXWaves) {
    float x[kWA][2];
    if constexpr (sizeof(T) == 4) {
      const float2* src = reinterpret_cast<const float2*>(reinterpret_cast<const float*>(p.x) + row * kWD) + lane;
#pragma unroll
      for (int a = 0; a < kWA; ++a) {
        const float2 v = src[64 * a];
        x[a][0] = v.x;
        x[a][1] = v.y;
      }
    } else {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(reinterpret_cast<const _Float16*>(p.x) + row * kWD) + lane;
#pragma unroll
      for (int a = 0; a < kWA; ++a) {
        const uint32_t u = src[64 * a];
        x[a][0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
        x[a][1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
      }
    }
    bool bad = false;
#pragma unroll
    for (int a = 0; a < kWA; ++a) bad |= !__builtin_isfinite(x[a][0]) || !__builtin_isfinite(x[a][1]);
    const bool nonfinite = __ballot(bad) != 0ull;
    auto sum_sq = [&]() {
      float t[kWA];
#pragma unroll
      for (int a = 0; a < kWA; ++a) t[a] = fmaf(x[a][0], x[a][0], x[a][1] * x[a][1]);
      float ss = (((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]))) +
                 ((t[8] + t[9]) + (t[10] + t[11]));
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) ss += __shfl_xor(ss, s);
      return ss;
    };
    float nu = 0.f, nu_x = 0.f;   // the stored norm; the norm of the row z is made from
    if constexpr (MODE != kWQuery) {
      // a non-finite row keeps its sum of squares (inf, or NaN when a NaN is
      // present) as its stored norm
      float ss = sum_sq();
      float pre = 1.f;
      if (!nonfinite && !(ss >= 0x1p-100f && ss <= 0x1p100f)) {
        // squares outside the normal fp32 range (fp32 input only): scale the
        // row exactly by the power of two that brings its largest entry into
        // [0.5, 1), as the d <= 128 encoder does
        float mx = 0.f;
#pragma unroll
        for (int a = 0; a < kWA; ++a) mx = fmaxf(mx, fmaxf(fabsf(x[a][0]), fabsf(x[a][1])));
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
        if (mx > 0.f) {
          int e;
          frexpf(mx, &e);
          const float sc = ldexpf(1.f, -e);
          pre = ldexpf(1.f, e);
#pragma unroll
          for (int a = 0; a < kWA; ++a) {
            x[a][0] *= sc;
            x[a][1] *= sc;
          }
          ss = sum_sq();
        }
      }
      nu_x = sqrtf(ss);
      nu = nu_x * pre;
    }
    // a vector with a non-finite element encodes as the zero vector
    if (nonfinite) {
#pragma unroll
      for (int a = 0; a < kWA; ++a) x[a][0] = x[a][1] = 0.f;
    }
    // D: sign flip of coordinate 128 a + 2 lane + e
#pragma unroll
    for (int a = 0; a < kWA; ++a) {
      const uint32_t w = s_flip[4 * a + (lane >> 4)];
      const int sh = 2 * (lane & 15);
      x[a][0] = __uint_as_float(__float_as_uint(x[a][0]) ^ (((w >> sh) & 1u) << 31));
      x[a][1] = __uint_as_float(__float_as_uint(x[a][1]) ^ (((w >> (sh + 1)) & 1u) << 31));
    }
    // H_128: offset bit 0 inside the lane, bits 1..6 across lanes
#pragma unroll
    for (int a = 0; a < kWA; ++a) {
      const float u = x[a][0], v = x[a][1];
      x[a][0] = u + v;
      x[a][1] = u - v;
    }
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const bool up = (lane & s) != 0;
#pragma unroll
      for (int a = 0; a < kWA; ++a)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float o = __shfl_xor(x[a][e], s);
          x[a][e] = up ? o - x[a][e] : x[a][e] + o;
        }
    }
    // H_12 across the chunks, then the scale
    const float inv = MODE == kWQuery ? p.inv_sqrt_d : (nu_x > 0.f ? p.inv_sqrt_d / nu_x : 0.f);
    float z[kWA][2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int a = 0; a < kWA; ++a) {
        float acc = 0.f;
#pragma unroll
        for (int b = 0; b < kWA; ++b) acc = kH12.v[a][b] > 0 ? acc + x[b][e] : acc - x[b][e];
        z[a][e] = acc * inv;
      }

    if constexpr (MODE == kWQuery) {
      uint32_t* oh = reinterpret_cast<uint32_t*>(p.rh + row * kWD) + lane;
      uint32_t* ol = reinterpret_cast<uint32_t*>(p.rl + row * kWD) + lane;
#pragma unroll
      for (int a = 0; a < kWA; ++a) {
        uint32_t hi, lo;
        split2(z[a][0], z[a][1], hi, lo);
        oh[64 * a] = hi;
        ol[64 * a] = lo;
      }
      continue;
    }

    // idx = #{k : z >= t_k}
    int q[kWA][2];
#pragma unroll
    for (int a = 0; a < kWA; ++a)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        int c = 0;
#pragma unroll
        for (int k = 0; k < (1 << CB) - 1; ++k) c += z[a][e] >= p.thresholds[k] ? 1 : 0;
        q[a][e] = c;
      }

    if constexpr (MODE == kWProd) {
      float r[kWA][2], t[kWA];
#pragma unroll
      for (int a = 0; a < kWA; ++a) {
        r[a][0] = z[a][0] - s_cent[q[a][0]];
        r[a][1] = z[a][1] - s_cent[q[a][1]];
        t[a] = fmaf(r[a][0], r[a][0], r[a][1] * r[a][1]);
      }
      float gg = (((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]))) +
                 ((t[8] + t[9]) + (t[10] + t[11]));
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) gg += __shfl_xor(gg, s);
      uint32_t* oh = reinterpret_cast<uint32_t*>(p.rh + row * kWD) + lane;
      uint32_t* ol = reinterpret_cast<uint32_t*>(p.rl + row * kWD) + lane;
#pragma unroll
      for (int a = 0; a < kWA; ++a) {
        uint32_t hi, lo;
        split2(r[a][0], r[a][1], hi, lo);
        oh[64 * a] = hi;
        ol[64 * a] = lo;
      }
      if (lane == 0) p.rnorm[row] = sqrtf(gg);
    }
    if (lane == 0) p.norm[row] = nu;

    // codes -> LDS bytes -> packed words (word w holds stream bits [32 w, 32 w + 32))
    uint16_t* sc16 = reinterpret_cast<uint16_t*>(s_code[wave]);
#pragma unroll
    for (int a = 0; a < kWA; ++a) sc16[64 * a + lane] = (uint16_t)(q[a][0] | (q[a][1] << 8));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int W = kWD * CB / 32;
    constexpr int SPAN = (32 + CB - 1) / CB + 1;   // codes that can touch one word
    uint32_t* dst = reinterpret_cast<uint32_t*>(p.idx + row * (kWD * CB / 8));
    for (int w = lane; w < W; w += 64) {
      const int b0 = 32 * w;
      const int i0 = b0 / CB;
      uint32_t word = 0u;
#pragma unroll
      for (int j = 0; j < SPAN; ++j) {
        const int i = i0 + j;
        const int off = i * CB - b0;
        if (off < 32 && i < kWD) {
          const uint32_t c = s_code[wave][i];
          word |= off >= 0 ? (c << off) : (c >> (-off));
        }
      }
      dst[w] = word;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---- fp32 -> fp16 hi / lo planes ---------------------------------------------
__global__ __launch_bounds__(256) void split_planes_kernel(const float* __restrict__ src, int64_t n2,
                                                            uint32_t* __restrict__ hi,
                                                            uint32_t* __restrict__ lo) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n2; i += (int64_t)gridDim.x * 256) {
    const float2 v = reinterpret_cast<const float2*>(src)[i];
    uint32_t h, l;
    split2(v.x, v.y, h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

// ---- projection P = S R^T (MFMA) -----------------------------------------------
// Workgroup tile 256 (rows i of S) x 256 (vectors t); 8 waves as 2 (i) x 4 (t),
// each 128 x 64 = 4 x 2 blocks of 32 x 32.  Per 32-wide k stage both
// operands' hi and lo planes pass through LDS (rows padded to 80 bytes so the
// 16-byte fragment reads of 8 consecutive rows hit distinct banks); the next
// stage's global loads are in flight during the products.
struct ProjParams {
  const _Float16* ah;    // S hi [1536][1536]
  const _Float16* al;    // S lo
  const _Float16* bh;    // R hi [nt][1536]
  const _Float16* bl;    // R lo
  int64_t nt;
  uint8_t* qjl;          // EPI 0: sign rows of 192 bytes
  _Float16* ph;          // EPI 1: P hi [nt][1536]
  _Float16* pl;          //        P lo
};

constexpr int kPWI = 2, kPWT = 4;
constexpr int kPBI = 4, kPBT = 2;
constexpr int kPTI = 32 * kPBI * kPWI;   // 256
constexpr int kPTT = 32 * kPBT * kPWT;   // 256
constexpr int kPK = 32;
constexpr int kPStride = kPK + 8;        // halves per LDS row
constexpr int kPThreads = 64 * kPWI * kPWT;
static_assert(kWD % kPTI == 0, "S rows split into whole tiles");
static_assert(kPBI == 4, "one 16-byte store of sign words per vector and wave");
static_assert(2 * (kPTI + kPTT) * kPK / 8 == 8 * kPThreads, "8 pieces of 16 bytes per thread");

template <int EPI>
__global__ __launch_bounds__(kPThreads) void wide_proj_kernel(ProjParams p) {
  __shared__ __align__(16) _Float16 s_a[2][kPTI][kPStride];
  __shared__ __align__(16) _Float16 s_b[2][kPTT][kPStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave % kPWI, wt = wave / kPWI;
  constexpr int NI = kWD / kPTI;
  const int64_t ntt = (p.nt + kPTT - 1) / kPTT;
  const int64_t G = ntt * NI;
  // consecutive workgroups of one XCD (blockIdx = x mod 8) take consecutive
  // tiles, so that the tiles sharing a block of vectors meet in one L2
  int64_t L = blockIdx.x;
  if (G % 8 == 0) L = (int64_t)(blockIdx.x % 8) * (G / 8) + blockIdx.x / 8;
  const int i0 = (int)(L % NI) * kPTI;
  const int64_t t0 = (L / NI) * kPTT;

  // each thread moves pieces q = tid + 512 u (u < 4) of 16 bytes per operand:
  // plane q / 1024, tile row (q % 1024) / 4, part q % 4 of the row's 64 bytes
  const _Float16* ga[4];
  const _Float16* gb[4];
  bool bok[4];
  int loff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = tid + u * kPThreads;
    const int pl = q >> 10, row = (q & 1023) >> 2, part = q & 3;
    ga[u] = (pl ? p.al : p.ah) + (int64_t)(i0 + row) * kWD + 8 * part;
    const int64_t t = t0 + row;
    bok[u] = t < p.nt;
    gb[u] = (pl ? p.bl : p.bh) + (bok[u] ? t : 0) * kWD + 8 * part;
    loff[u] = (pl * kPTI + row) * kPStride + 8 * part;   // same offset in s_a and s_b
  }
  static_assert(kPTI == kPTT, "one LDS offset serves both operands");
  u32x4 ra[4], rb[4];   // native vectors: a struct copy here would land in scratch
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    ra[u] = *reinterpret_cast<const u32x4*>(ga[u]);
    rb[u] = *reinterpret_cast<const u32x4*>(gb[u]);     // row 0 stands in past nt
    if (!bok[u]) rb[u] = u32x4{0u, 0u, 0u, 0u};
  }
  _Float16* la = &s_a[0][0][0];
  _Float16* lb = &s_b[0][0][0];

  f32x16 acc[kPBI][kPBT];
#pragma unroll
  for (int bi = 0; bi < kPBI; ++bi)
#pragma unroll
    for (int bt = 0; bt < kPBT; ++bt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[bi][bt][v] = 0.f;

  for (int k0 = 0; k0 < kWD; k0 += kPK) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<u32x4*>(la + loff[u]) = ra[u];
      *reinterpret_cast<u32x4*>(lb + loff[u]) = rb[u];
    }
    __syncthreads();
    {
      // the next stage (the last stage reloads itself: in bounds, unused)
      const int kn = k0 + kPK < kWD ? k0 + kPK : k0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ra[u] = *reinterpret_cast<const u32x4*>(ga[u] + kn);
        rb[u] = *reinterpret_cast<const u32x4*>(gb[u] + kn);
        if (!bok[u]) rb[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int s = 0; s < kPK / 16; ++s) {
      const int kk = 16 * s + 8 * (lane >> 5);
      half8_t ah[kPBI], al[kPBI], bh[kPBT], bl[kPBT];
#pragma unroll
      for (int bi = 0; bi < kPBI; ++bi) {
        const int r = wi * 32 * kPBI + 32 * bi + (lane & 31);
        ah[bi] = *reinterpret_cast<const half8_t*>(&s_a[0][r][kk]);
        al[bi] = *reinterpret_cast<const half8_t*>(&s_a[1][r][kk]);
      }
#pragma unroll
      for (int bt = 0; bt < kPBT; ++bt) {
        const int r = wt * 32 * kPBT + 32 * bt + (lane & 31);
        bh[bt] = *reinterpret_cast<const half8_t*>(&s_b[0][r][kk]);
        bl[bt] = *reinterpret_cast<const half8_t*>(&s_b[1][r][kk]);
      }
#pragma unroll
      for (int bi = 0; bi < kPBI; ++bi)
#pragma unroll
        for (int bt = 0; bt < kPBT; ++bt) {
          acc[bi][bt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[bi], bh[bt], acc[bi][bt], 0, 0, 0);
          acc[bi][bt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[bi], bl[bt], acc[bi][bt], 0, 0, 0);
          acc[bi][bt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[bi], bh[bt], acc[bi][bt], 0, 0, 0);
        }
      // one k step's fragments live at a time
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // accumulator element v of lane l: column t = l % 32, row 8 (v / 4) + 4 (l / 32) + v % 4
  const int h = lane >> 5;
  const int ib = i0 + wi * 32 * kPBI;
#pragma unroll
  for (int bt = 0; bt < kPBT; ++bt) {
    const int64_t t = t0 + wt * 32 * kPBT + 32 * bt + (lane & 31);
    if constexpr (EPI == 0) {
      uint32_t words[kPBI];
#pragma unroll
      for (int bi = 0; bi < kPBI; ++bi) {
        uint32_t m = 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          m |= (acc[bi][bt][v] >= 0.f ? 1u : 0u) << (8 * (v >> 2) + 4 * h + (v & 3));
        m |= __shfl_xor(m, 32);
        words[bi] = m;
      }
      if (h == 0 && t < p.nt)
        *reinterpret_cast<uint4*>(p.qjl + t * (kWD / 8) + ib / 8) =
            make_uint4(words[0], words[1], words[2], words[3]);
    } else {
      if (t < p.nt) {
#pragma unroll
        for (int bi = 0; bi < kPBI; ++bi)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int i = ib + 32 * bi + 8 * g + 4 * h;
            uint32_t h0, l0, h1, l1;
            split2(acc[bi][bt][4 * g], acc[bi][bt][4 * g + 1], h0, l0);
            split2(acc[bi][bt][4 * g + 2], acc[bi][bt][4 * g + 3], h1, l1);
            *reinterpret_cast<uint2*>(p.ph + t * kWD + i) = make_uint2(h0, h1);
            *reinterpret_cast<uint2*>(p.pl + t * kWD + i) = make_uint2(l0, l1);
          }
      }
    }
  }
}

// ---- scan: est[a][j] over packed rows (MFMA) --------------------------------------
// Workgroup: 32 queries x 512 rows; wave w takes rows 128 w .. 128 w + 127 as
// four 32-row blocks.  Inside a 128-coordinate chunk c, k step s (0..7) and
// lane half h = lane / 32 use coordinates 128 c + 64 h + 8 s + j (j < 8): a
// lane reads 128 contiguous bytes of each query plane and 8 CB contiguous
// bytes of each code row per chunk.
struct WScanParams {
  const _Float16* qh;   // q_rot hi [n_q][1536]
  const _Float16* ql;
  const _Float16* sh;   // S q_rot hi (prod)
  const _Float16* sl;
  const uint8_t* idx;
  const uint8_t* qjl;
  const float* norm;
  const float* rnorm;
  int64_t n;
  int64_t n_q;
  float* out;           // [n_q][n]
  float cscale;         // B operands carry c / cscale
  float qjl_scale;      // sqrt(pi/2) / m
  uint32_t chl[16];     // CB > 1: fp16 hi | lo << 16 of c[j] / cscale
};

constexpr int kSRB = 4;
constexpr int kSWaves = 4;
constexpr int kSRows = 32 * kSRB * kSWaves;

// eight bits -> eight fp16 +-1 (bit set: +1) as four dwords
__device__ __forceinline__ half8_t pm1_frag(uint32_t byte) {
  const uint32_t x = ((~byte) & 0xffu) * 0x8001u;
  uint4 w;
  w.x = ((x << 15) & 0x80008000u) | 0x3C003C00u;
  w.y = ((x << 13) & 0x80008000u) | 0x3C003C00u;
  w.z = ((x << 11) & 0x80008000u) | 0x3C003C00u;
  w.w = ((x << 9) & 0x80008000u) | 0x3C003C00u;
  return __builtin_bit_cast(half8_t, w);
}

template <int CB, bool PROD>
__global__ __launch_bounds__(64 * kSWaves, 2) void wide_scan_kernel(WScanParams p) {
  constexpr int NP = CB > 1 ? (1 << (2 * CB)) : 1;
  __shared__ uint32_t s_ph[NP];
  __shared__ uint32_t s_pl[NP];
  __shared__ u32x4 s_pm[256];       // eight bits -> eight fp16 +-1
  // (the wave index through readfirstlane: a scalar, so that the row bases
  // derived from it stay in scalar registers)
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (CB > 1) {
    const uint32_t* chl = reinterpret_cast<const uint32_t*>(TQ_KARG(WScanParams, chl));
    for (int e = tid; e < NP; e += 64 * kSWaves) {
      const uint32_t a = chl[e & ((1 << CB) - 1)], b = chl[e >> CB];
      s_ph[e] = (a & 0xffffu) | (b << 16);
      s_pl[e] = (a >> 16) | (b & 0xffff0000u);
    }
  }
  for (int e = tid; e < 256; e += 64 * kSWaves) s_pm[e] = __builtin_bit_cast(u32x4, pm1_frag((uint32_t)e));
  __syncthreads();
  // (32-bit index math, then readfirstlane: the divisions run on the vector
  // unit, and their uniform results go back to scalar registers)
  const uint32_t QB = (uint32_t)((p.n_q + 31) / 32);
  const uint32_t b = blockIdx.x;
  uint32_t qb32, rt32;
  if (QB % 8 == 0) {
    // each XCD keeps one eighth of the query planes in its L2
    const uint32_t per = QB / 8, k = b / 8;
    qb32 = (b % 8) * per + k % per;
    rt32 = k / per;
  } else {
    qb32 = b % QB;
    rt32 = b / QB;
  }
  const int64_t qb = (uint32_t)__builtin_amdgcn_readfirstlane((int)qb32);
  const int64_t rt = (uint32_t)__builtin_amdgcn_readfirstlane((int)rt32);
  const int64_t r0 = rt * kSRows + wave * 32 * kSRB;
  constexpr int RB = kWD * CB / 8;
  // Buffer descriptors over the workgroup's rows of the code and sign
  // planes: 32-bit offsets (a lane's row and lane half in the vector
  // offset, which the range check covers), and rows past n read as zero.
  constexpr int kRsrcWord3 = 0x00020000;
  const int64_t wrow = rt * kSRows;
  const uint32_t wrows = (uint32_t)(p.n - wrow < kSRows ? p.n - wrow : kSRows);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.idx + wrow * RB), (short)0, (int)(wrows * RB), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      PROD ? (void*)(p.qjl + wrow * (kWD / 8)) : (void*)p.idx, (short)0, PROD ? (int)(wrows * (kWD / 8)) : 0,
      kRsrcWord3);
  // sign-plane offset of a lane's row and half; the code-plane offset is
  // CB times it
  uint32_t soff[kSRB];
#pragma unroll
  for (int rb = 0; rb < kSRB; ++rb) {
    const uint32_t jr = (uint32_t)(wave * 32 * kSRB + 32 * rb + (lane & 31));
    soff[rb] = jr * (kWD / 8) + 8 * h;
  }
  f32x16 accm[kSRB], accq[kSRB];
#pragma unroll
  for (int rb = 0; rb < kSRB; ++rb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      accm[rb][v] = 0.f;
      accq[rb][v] = 0.f;
    }

  // k steps of 16 coordinates, four to a half chunk of 64: in half chunk hc
  // (chunk c = hc / 2) lane half h covers coordinates
  // 128 c + 64 h + 32 (hc % 2) + [0, 32), 8 per k step.  The workgroup's 32
  // query rows of a half chunk pass through LDS (double buffered, one
  // barrier per half chunk); the next half chunk's query planes and code bits
  // load while the current products run.
  constexpr int NPL = PROD ? 4 : 2;            // query planes
  constexpr int QS = 72;                       // halves per LDS row (64 + 8 pad)
  __shared__ __align__(16) _Float16 s_q[2][NPL][32][QS];
  constexpr int QPIECES = NPL * 32 * 8 / (64 * kSWaves);   // 16-byte pieces per thread
  static_assert(QPIECES == NPL && 64 * kSWaves == 256, "thread t loads piece t of every plane");
  // Buffer descriptors over the workgroup's 32 query rows of each plane
  // (rows past n_q read as zero): thread t loads the 16-byte piece t % 8 of
  // row t / 8 of each plane, at the same 32-bit offset in all of them.
  const uint32_t qrows = (uint32_t)(p.n_q - qb * 32 < 32 ? p.n_q - qb * 32 : 32);
  const _Float16* planes[4] = {p.qh, p.ql, p.sh, p.sl};
  __amdgpu_buffer_rsrc_t rq[NPL];
#pragma unroll
  for (int pl = 0; pl < NPL; ++pl)
    rq[pl] = __builtin_amdgcn_make_buffer_rsrc((void*)(planes[pl] + qb * 32 * kWD), (short)0,
                                               (int)(qrows * kWD * 2), kRsrcWord3);
  const uint32_t qoff = (uint32_t)((((tid >> 3) & 31) * kWD + 64 * ((tid & 7) >> 2) + 8 * (tid & 3)) * 2);
  u32x4 qr[QPIECES];
  auto gload_q = [&](int hc) {
    const int c = hc >> 1, hh = hc & 1;
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
      qr[pl] = __builtin_amdgcn_raw_buffer_load_b128(rq[pl], qoff, (128 * c + 32 * hh) * 2, 0);
  };
  auto lstore_q = [&](int bf) {
#pragma unroll
    for (int u = 0; u < QPIECES; ++u) {
      const int t = tid + u * 64 * kSWaves;
      const int pl = t >> 8, row = (t >> 3) & 31, j = t & 7;
      *reinterpret_cast<u32x4*>(&s_q[bf][pl][row][32 * (j >> 2) + 8 * (j & 3)]) = qr[u];
    }
  };
  uint32_t cw[2][kSRB][CB];         // code bits of a half chunk
  uint32_t sw[2][kSRB];             // sign bits
  auto load_bits = [&](int hc, int bf) {
    const int c = hc >> 1, hh = hc & 1;
#pragma unroll
    for (int rb = 0; rb < kSRB; ++rb) {
      const uint32_t o = CB * soff[rb] + 16 * CB * c + 4 * CB * hh;
      if constexpr (CB == 1) {
        cw[bf][rb][0] = __builtin_amdgcn_raw_buffer_load_b32(rc, o, 0, 0);
      } else if constexpr (CB == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, o, 0, 0);
        cw[bf][rb][0] = v[0]; cw[bf][rb][1] = v[1];
      } else if constexpr (CB == 3) {
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, o, 0, 0);
        cw[bf][rb][0] = v[0]; cw[bf][rb][1] = v[1]; cw[bf][rb][2] = v[2];
      } else {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, o, 0, 0);
        cw[bf][rb][0] = v[0]; cw[bf][rb][1] = v[1]; cw[bf][rb][2] = v[2]; cw[bf][rb][3] = v[3];
      }
      if constexpr (PROD) sw[bf][rb] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff[rb] + 16 * c + 4 * hh, 0, 0);
    }
  };
  auto compute = [&](int s, int bf) {
    half8_t fa[4];
#pragma unroll
    for (int pl = 0; pl < NPL; ++pl)
      fa[pl] = *reinterpret_cast<const half8_t*>(&s_q[bf][pl][lane & 31][32 * h + 8 * s]);
#pragma unroll
    for (int rb = 0; rb < kSRB; ++rb) {
      if constexpr (CB == 1) {
        const half8_t cb = __builtin_bit_cast(half8_t, s_pm[(cw[bf][rb][0] >> (8 * s)) & 0xffu]);
        accm[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[0], cb, accm[rb], 0, 0, 0);
        accm[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[1], cb, accm[rb], 0, 0, 0);
      } else {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int off = (8 * s + 2 * pp) * CB;     // bit offset in this lane's half-chunk bits
          const int w = off >> 5, sh = off & 31;
          uint32_t e = cw[bf][rb][w] >> sh;
          if (sh + 2 * CB > 32) e |= cw[bf][rb][w + 1] << (32 - sh);
          e &= NP - 1;
          hi[pp] = s_ph[e];
          lo[pp] = s_pl[e];
        }
        const half8_t ch = __builtin_bit_cast(half8_t, u32x4{hi[0], hi[1], hi[2], hi[3]});
        const half8_t cl = __builtin_bit_cast(half8_t, u32x4{lo[0], lo[1], lo[2], lo[3]});
        accm[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[0], ch, accm[rb], 0, 0, 0);
        accm[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[1], ch, accm[rb], 0, 0, 0);
        accm[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[0], cl, accm[rb], 0, 0, 0);
      }
      if constexpr (PROD) {
        const half8_t sg = __builtin_bit_cast(half8_t, s_pm[(sw[bf][rb] >> (8 * s)) & 0xffu]);
        accq[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[2], sg, accq[rb], 0, 0, 0);
        accq[rb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[3], sg, accq[rb], 0, 0, 0);
      }
    }
  };
  constexpr int NH = 2 * kWA;       // half chunks
  gload_q(0);
  load_bits(0, 0);
  lstore_q(0);
  __syncthreads();
  auto half = [&](int hc, int bf) {
    if (hc + 1 < NH) {
      gload_q(hc + 1);
      load_bits(hc + 1, bf ^ 1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) compute(s, bf);
    if (hc + 1 < NH) lstore_q(bf ^ 1);
    __syncthreads();
  };
  for (int hc = 0; hc < NH; hc += 2) {
    half(hc, 0);
    half(hc + 1, 1);
  }

  // est = nu (cscale M + sqrt(pi/2)/m gamma Q); element v: query 8 (v/4) + 4 h + v % 4
#pragma unroll
  for (int rb = 0; rb < kSRB; ++rb) {
    const int64_t j = r0 + 32 * rb + (lane & 31);
    if (j >= p.n) continue;
    const float nu = p.norm[j];
    const float g = PROD ? p.rnorm[j] * p.qjl_scale : 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t a = qb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (a < p.n_q) {
        const float m = p.cscale * accm[rb][v];
        p.out[a * p.n + j] = nu * (PROD ? fmaf(g, accq[rb][v], m) : m);
      }
    }
  }
}

// ---- host side ------------------------------------------------------------------
constexpr int64_t kWideChunk = 32768;    // vectors per projection pass of an encode

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
static size_t s_split_bytes() { return align256((size_t)2 * kWD * kWD * sizeof(_Float16)); }

size_t wide_encode_workspace_bytes(const tq_codec& c, int64_t n_rows) {
  if (c.d != kWD || c.mode != TQ_PROD || n_rows <= 0) return 0;
  const int64_t ch = n_rows < kWideChunk ? n_rows : kWideChunk;
  return s_split_bytes() + align256((size_t)ch * kWD * 2 * sizeof(_Float16));
}

size_t wide_scan_workspace_bytes(int64_t n_q) {
  return s_split_bytes() + align256((size_t)n_q * kWD * 4 * sizeof(_Float16));
}

static unsigned grid_for(int64_t items, int64_t per_block, int cap) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return (unsigned)(g < 1 ? 1 : g);
}

static void fill_xparams(WideXParams& p, const tq_codec& c) {
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)kWD));
  for (int k = 0; k < 16; ++k) {
    p.centroids[k] = c.centroids[k];
    p.thresholds[k] = c.thresholds[k];
  }
  for (int w = 0; w < 48; ++w) p.flip[w] = c.flip[w];
}

template <typename T, int MODE>
static hipError_t run_transform(int cb, const WideXParams& p, hipStream_t s) {
  const unsigned grid = grid_for(p.n, kXWaves, device_cu_count() * 8);
  const dim3 blk(64 * kXWaves);
  switch (cb) {
    case 1: hipLaunchKernelGGL((wide_transform_kernel<T, 1, MODE>), dim3(grid), blk, 0, s, p); break;
    case 2: hipLaunchKernelGGL((wide_transform_kernel<T, 2, MODE>), dim3(grid), blk, 0, s, p); break;
    case 3: hipLaunchKernelGGL((wide_transform_kernel<T, 3, MODE>), dim3(grid), blk, 0, s, p); break;
    case 4: hipLaunchKernelGGL((wide_transform_kernel<T, 4, MODE>), dim3(grid), blk, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t transform_dt(int dtype, int cb, const WideXParams& p, hipStream_t s) {
  return dtype == TQ_F16 ? run_transform<_Float16, MODE>(cb, p, s) : run_transform<float, MODE>(cb, p, s);
}

static hipError_t split_s(const float* S, _Float16* hi, _Float16* lo, hipStream_t s) {
  const int64_t n2 = (int64_t)kWD * kWD / 2;
  hipLaunchKernelGGL(split_planes_kernel, dim3(grid_for(n2, 256, 4096)), dim3(256), 0, s, S, n2,
                     reinterpret_cast<uint32_t*>(hi), reinterpret_cast<uint32_t*>(lo));
  return hipGetLastError();
}

template <int EPI>
static hipError_t run_proj(const ProjParams& p, hipStream_t s) {
  const int64_t tiles = ((p.nt + kPTT - 1) / kPTT) * (kWD / kPTI);
  hipLaunchKernelGGL((wide_proj_kernel<EPI>), dim3((unsigned)tiles), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wide_encode(const tq_codec& c, const void* x, int dtype, int64_t n_rows,
                              const tq_packed& out, void* workspace, hipStream_t stream) {
  if (c.d != kWD) return hipErrorInvalidValue;
  WideXParams p = {};
  fill_xparams(p, c);
  const size_t row_bytes = (size_t)kWD * c.code_bits / 8;
  const size_t esz = dtype == TQ_F16 ? 2 : 4;
  if (c.mode != TQ_PROD) {
    p.x = x;
    p.n = n_rows;
    p.idx = out.idx;
    p.norm = out.norm;
    return transform_dt<kWMse>(dtype, c.code_bits, p, stream);
  }
  _Float16* sh = reinterpret_cast<_Float16*>(workspace);
  _Float16* sl = sh + (size_t)kWD * kWD;
  _Float16* rh = reinterpret_cast<_Float16*>(reinterpret_cast<uint8_t*>(workspace) + s_split_bytes());
  const int64_t ch = n_rows < kWideChunk ? n_rows : kWideChunk;
  _Float16* rl = rh + (size_t)ch * kWD;
  hipError_t e = split_s(c.S, sh, sl, stream);
  if (e != hipSuccess) return e;
  for (int64_t r0 = 0; r0 < n_rows; r0 += ch) {
    const int64_t n = (n_rows - r0) < ch ? (n_rows - r0) : ch;
    p.x = reinterpret_cast<const uint8_t*>(x) + (size_t)r0 * kWD * esz;
    p.n = n;
    p.idx = out.idx + (size_t)r0 * row_bytes;
    p.norm = out.norm + r0;
    p.rnorm = out.rnorm + r0;
    p.rh = rh;
    p.rl = rl;
    if ((e = transform_dt<kWProd>(dtype, c.code_bits, p, stream)) != hipSuccess) return e;
    ProjParams q = {};
    q.ah = sh; q.al = sl; q.bh = rh; q.bl = rl;
    q.nt = n;
    q.qjl = out.qjl + (size_t)r0 * (kWD / 8);
    if ((e = run_proj<0>(q, stream)) != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int CB, bool PROD>
static hipError_t run_wscan(const WScanParams& p, hipStream_t s) {
  const int64_t blocks = ((p.n_q + 31) / 32) * ((p.n + kSRows - 1) / kSRows);
  hipLaunchKernelGGL((wide_scan_kernel<CB, PROD>), dim3((unsigned)blocks), dim3(64 * kSWaves), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wide_scan(const tq_codec& c, const void* q, int q_dtype, int64_t n_q,
                            const tq_packed& x, int64_t n, float* scores, void* workspace,
                            hipStream_t stream) {
  if (c.d != kWD) return hipErrorInvalidValue;
  _Float16* sh = reinterpret_cast<_Float16*>(workspace);
  _Float16* sl = sh + (size_t)kWD * kWD;
  _Float16* qh = reinterpret_cast<_Float16*>(reinterpret_cast<uint8_t*>(workspace) + s_split_bytes());
  _Float16* ql = qh + (size_t)n_q * kWD;
  _Float16* qsh = ql + (size_t)n_q * kWD;
  _Float16* qsl = qsh + (size_t)n_q * kWD;
  const bool prod = c.mode == TQ_PROD;
  // q_rot = Pi q (not normalised), as hi / lo planes
  WideXParams p = {};
  fill_xparams(p, c);
  p.x = q;
  p.n = n_q;
  p.rh = qh;
  p.rl = ql;
  hipError_t e = transform_dt<kWQuery>(q_dtype, 1, p, stream);
  if (e != hipSuccess) return e;
  if (prod) {
    // S q_rot through the projection product, stored as hi / lo planes
    if ((e = split_s(c.S, sh, sl, stream)) != hipSuccess) return e;
    ProjParams pp = {};
    pp.ah = sh; pp.al = sl; pp.bh = qh; pp.bl = ql;
    pp.nt = n_q;
    pp.ph = qsh;
    pp.pl = qsl;
    if ((e = run_proj<1>(pp, stream)) != hipSuccess) return e;
  }
  WScanParams s = {};
  s.qh = qh; s.ql = ql; s.sh = qsh; s.sl = qsl;
  s.idx = x.idx; s.qjl = x.qjl; s.norm = x.norm; s.rnorm = x.rnorm;
  s.n = n; s.n_q = n_q;
  s.out = scores;
  const int levels = 1 << c.code_bits;
  float cmax = 0.f;
  for (int k = 0; k < levels; ++k) cmax = std::fmax(cmax, std::fabs(c.centroids[k]));
  if (!(cmax > 0.f)) return hipErrorInvalidValue;
  s.cscale = cmax;
  s.qjl_scale = prod ? (float)(std::sqrt(M_PI / 2.0) / c.m) : 0.f;
  for (int k = 0; k < levels; ++k) {
    const float v = c.centroids[k] / cmax;
    const _Float16 hv = (_Float16)v;
    const _Float16 lv = (_Float16)(v - (float)hv);
    s.chl[k] = (uint32_t)__builtin_bit_cast(uint16_t, hv) | ((uint32_t)__builtin_bit_cast(uint16_t, lv) << 16);
  }
  if (c.code_bits == 1 && !(c.centroids[0] == -cmax && c.centroids[1] == cmax))
    return hipErrorInvalidValue;   // 1-bit operands are +-1: the table must be symmetric
  switch (c.code_bits * 2 + (prod ? 1 : 0)) {
    case 2: return run_wscan<1, false>(s, stream);
    case 3: return run_wscan<1, true>(s, stream);
    case 4: return run_wscan<2, false>(s, stream);
    case 5: return run_wscan<2, true>(s, stream);
    case 6: return run_wscan<3, false>(s, stream);
    case 7: return run_wscan<3, true>(s, stream);
    case 8: return run_wscan<4, false>(s, stream);
    case 9: return run_wscan<4, true>(s, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tqk
