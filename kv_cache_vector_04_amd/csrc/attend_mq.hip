// Attention from packed codes with many query rows per KV head (the
// bidirectional protein-model case: every position attends to every
// position), d = 64.  "TurboESM", "2. Metodologia" part E: unpack, correct
// and attend with an online softmax in one pass; "Google presenta
// TurboQuant", "Eliminación del sesgo interno del producto" for the score
//   s_j = scale nu_j ( <q_rot, c_K[idx_j]> + sqrt(pi/2)/m gamma_j <Sq, 2 sigma_j - 1> ).
//
// A workgroup of 8 waves owns 256 query rows of one (batch, KV head) and
// walks the whole key range in 64-token tiles.  Per tile the codes are
// dequantized once into LDS and shared by all 256 rows:
//   K: nu_j scale c_K[idx] as fp16 hi + lo, [token][coordinate];
//   signs: +-f_j with f_j = nu_j scale sqrt(pi/2)/m gamma_j, as hi + lo;
//   V: nu^V_j c_V[idx] as hi + lo, transposed to [coordinate][token].
// Both products run on the matrix cores (v_mfma_f32_32x32x16_f16) with fp32
// accumulation and the hi / lo splits (hi.hi + hi.lo + lo.hi):
//   scores, transposed: S^T[token][query] = K q + signs Sq, so that a lane
//     holds one query's scores for 32 tokens and the softmax reductions stay
//     in the lane (plus one exchange between lane halves);
//   values: O^T[coordinate][query] += V^T P^T with the weights P taken
//     straight from the score registers: the value tile's token columns are
//     stored in the order that matches the score layout (bits 2 and 3 of
//     the token index swapped).
// At the end each lane divides by the softmax sum and applies
// o = D_V H (O / L) / sqrt(d): butterflies over its 32 coordinates in
// registers plus one exchange between lane halves.

#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"
#include "qprep.hpp"

namespace tqk {

constexpr int kMqWaves = 8;
constexpr int kMqThreads = kMqWaves * kWave;
constexpr int kMqRows = 32 * kMqWaves;   // query rows per workgroup
constexpr int kMqTile = 64;              // tokens per tile
constexpr int kMqStr = 72;               // halves per LDS row (64 + 8: conflict-free 16-byte reads)

struct MqParams {
  const uint8_t* kidx;
  const uint8_t* kqjl;
  const float* knorm;
  const float* krnorm;
  const uint8_t* vidx;
  const float* vnorm;
  const void* q;         // [rows][64], fp16 or fp32
  int q_f16;
  int rope;
  int32_t pos0;
  const float* S;        // 64 x 64 row-major
  float* out;            // [rows][64]
  float* scores_out;     // optional [rows][ctx]
  int64_t ctx;
  int hq, hkv, n_q, G, nqb;
  float scale, qjl_scale, inv_sqrt_d;
  float kcent[16];
  float vcent[16];
  uint32_t vflip[2];
  uint32_t kflip[2];
  double theta[32];      // RoPE: base^(-2i/64)
};

typedef uint32_t mq_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mq_h16(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// hi / lo fp16 pair of one float, as two 16-bit patterns
__device__ __forceinline__ void mq_split(float x, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = (_Float16)x;
  hi = (uint32_t)__builtin_bit_cast(uint16_t, h);
  lo = mq_h16(x - (float)h);
}

// value of lane l ^ 32 (the other half of the wave)
__device__ __forceinline__ float mq_partner(float x, int h) {
  uint32_t a = __float_as_uint(x), b = a;
  swap_halves(a, b);
  return __uint_as_float(h ? a : b);
}

template <int CBK, int CBV>
__global__ __launch_bounds__(kMqThreads, 2) void attend_mq_kernel(MqParams p) {
  constexpr int D = 64;
  constexpr int KRW = D * CBK / 32;      // words per key row
  constexpr int VRW = D * CBV / 32;      // words per value row
  constexpr int CPT = kMqTile * D / kMqThreads;   // key coordinates dequantized per thread
  constexpr int TPT = kMqTile * D / kMqThreads;   // value tokens dequantized per thread
  static_assert(CPT % 8 == 0 && CPT <= 16 && TPT % 8 == 0, "16-byte LDS stores");
  // two buffers of each: the products of tile i read one while tile i + 1
  // is dequantized into the other
  __shared__ __align__(16) _Float16 s_kh[2][kMqTile][kMqStr];
  __shared__ __align__(16) _Float16 s_kl[2][kMqTile][kMqStr];
  __shared__ __align__(16) _Float16 s_sh[2][kMqTile][kMqStr];
  __shared__ __align__(16) _Float16 s_sl[2][kMqTile][kMqStr];
  __shared__ __align__(16) _Float16 s_vh[2][D][kMqStr];
  __shared__ __align__(16) _Float16 s_vl[2][D][kMqStr];
  __shared__ uint32_t s_kraw[2][kMqTile][KRW + 1];   // a spare word per row: codes read two words
  __shared__ uint32_t s_sraw[2][kMqTile][2];
  __shared__ uint32_t s_vraw[2][kMqTile][VRW + 1];
  __shared__ float s_fk[2][kMqTile], s_fs[2][kMqTile], s_nv[2][kMqTile];
  __shared__ float s_kc[16], s_vc[16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int bg = blockIdx.x / p.nqb, qb = blockIdx.x % p.nqb;
  const int g = bg % p.hkv, b = bg / p.hkv;
  const int rows = p.G * p.n_q;                              // query rows of this KV head
  const int r = qb * kMqRows + wave * 32 + l32;              // this lane's query row
  const bool rok = r < rows;
  const int64_t row_base = ((int64_t)b * p.hq + (int64_t)g * p.G) * p.n_q;
  const int64_t kv_base = (int64_t)bg * p.ctx;

  // ---- query preparation, in registers: lane (row r, h) holds coordinates
  // 16 ks + 8 h + j (the B-operand layout of the products below) ----
  // S as fp16 hi / lo in key-tile buffer 1 (free until the second tile)
  for (int i = tid; i < D * D / 4; i += kMqThreads) {
    const float4 v = reinterpret_cast<const float4*>(p.S)[i];
    const int row = (4 * i) / D, col = (4 * i) % D;
    uint32_t h0, l0, h1, l1, h2, l2, h3, l3;
    mq_split(v.x, h0, l0);
    mq_split(v.y, h1, l1);
    mq_split(v.z, h2, l2);
    mq_split(v.w, h3, l3);
    *reinterpret_cast<uint2*>(&s_kh[1][row][col]) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
    *reinterpret_cast<uint2*>(&s_kl[1][row][col]) = make_uint2(l0 | (l1 << 16), l2 | (l3 << 16));
  }
  mq_u32x4 fq[4][4];     // [k step][q_hi, q_lo, Sq_hi, Sq_lo]
  {
    float x[4][8];
    const int64_t row = row_base + (rok ? r : 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 16 * ks + 8 * h;
      if (p.q_f16) {
        const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const _Float16*>(p.q) + row * D + c0);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[ks][2 * e] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] & 0xffffu));
          x[ks][2 * e + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[e] >> 16));
        }
      } else {
        const float4 x0 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.q) + row * D + c0)[0];
        const float4 x1 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.q) + row * D + c0)[1];
        x[ks][0] = x0.x; x[ks][1] = x0.y; x[ks][2] = x0.z; x[ks][3] = x0.w;
        x[ks][4] = x1.x; x[ks][5] = x1.y; x[ks][6] = x1.z; x[ks][7] = x1.w;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) x[ks][j] = rok ? x[ks][j] : 0.f;
      // RoPE on the interleaved pairs (c, c + 1), c even, at position pos0 + r % n_q
      if (p.rope) {
        const int64_t pos = (int64_t)p.pos0 + (r % p.n_q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sn, cs;
          sincos_reduced((double)pos * p.theta[(c0 >> 1) + e], sn, cs);
          const float a = x[ks][2 * e], bq = x[ks][2 * e + 1];
          x[ks][2 * e] = a * cs - bq * sn;
          x[ks][2 * e + 1] = a * sn + bq * cs;
        }
      }
      // sign flip D_K
      const uint32_t fw = p.kflip[c0 >> 5] >> (c0 & 31);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[ks][j] = __uint_as_float(__float_as_uint(x[ks][j]) ^ (((fw >> j) & 1u) << 31));
    }
    // H_64: coordinate bits 0-2 = j, 3 = h (across lane halves), 4-5 = ks
#pragma unroll
    for (int m = 1; m < 8; m <<= 1)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((j & m) == 0) {
            const float a = x[ks][j], c = x[ks][j | m];
            x[ks][j] = a + c;
            x[ks][j | m] = a - c;
          }
#pragma unroll
    for (int m = 1; m < 4; m <<= 1)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        if ((ks & m) == 0)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float a = x[ks][j], c = x[ks | m][j];
            x[ks][j] = a + c;
            x[ks | m][j] = a - c;
          }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float o = mq_partner(x[ks][j], h);
        x[ks][j] = (h ? (o - x[ks][j]) : (x[ks][j] + o)) * p.inv_sqrt_d;
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) mq_split(x[ks][j], hi[j], lo[j]);
      fq[ks][0] = mq_u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                           hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
      fq[ks][1] = mq_u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                           lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
    }
  }
  __syncthreads();       // S in LDS
  {
    // Sq^T = S q_rot: rows = output coordinates 32 bi + 8 (v / 4) + 4 h + v % 4
    f32x16 C[2];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
      for (int v = 0; v < 16; ++v) C[bi][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const half8_t ah = *reinterpret_cast<const half8_t*>(&s_kh[1][32 * bi + l32][16 * ks + 8 * h]);
        const half8_t al = *reinterpret_cast<const half8_t*>(&s_kl[1][32 * bi + l32][16 * ks + 8 * h]);
        const half8_t qh = __builtin_bit_cast(half8_t, fq[ks][0]);
        const half8_t ql = __builtin_bit_cast(half8_t, fq[ks][1]);
        C[bi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, qh, C[bi], 0, 0, 0);
        C[bi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, ql, C[bi], 0, 0, 0);
        C[bi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, qh, C[bi], 0, 0, 0);
      }
    }
    // Exchange coordinate bit 2 (the lane half of C) with bit 3 (the lane
    // half of the operand layout): one half swap per register pair
    // (v, v + 4), v % 8 < 4.  After it, lane half h holds coordinates with
    // bit 3 = h: element j = 4 e + (v % 4) of k step 2 bi + v / 8 comes from
    // register v + 4 e of the pair.
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((v & 4) == 0) {
          uint32_t a = __float_as_uint(C[bi][v]), c = __float_as_uint(C[bi][v + 4]);
          swap_halves(a, c);
          C[bi][v] = __uint_as_float(a);
          C[bi][v + 4] = __uint_as_float(c);
        }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int bi = ks >> 1, v0 = 8 * (ks & 1);
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) mq_split(C[bi][v0 + 4 * (j >> 2) + (j & 3)], hi[j], lo[j]);
      fq[ks][2] = mq_u32x4{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16),
                           hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16)};
      fq[ks][3] = mq_u32x4{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16),
                           lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16)};
    }
  }
  if (tid < 16) {
    s_kc[tid] = p.kcent[tid];
    s_vc[tid] = p.vcent[tid];
  }

  f32x16 O[2];           // O^T: coordinates 32 cb + 8 (v / 4) + 4 h + v % 4, column = query
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[cb][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // raw codes and norms of a tile, loaded into registers one tile ahead
  // (tokens past the end: zero codes, zero norms)
  constexpr int KPT = (kMqTile * KRW + kMqThreads - 1) / kMqThreads;   // key words per thread
  constexpr int VPT = (kMqTile * VRW + kMqThreads - 1) / kMqThreads;   // value words per thread
  uint32_t rk[KPT], rv[VPT], rs = 0u;
  float rn0 = 0.f, rn1 = 0.f, rn2 = 0.f;
  auto load_raw = [&](int64_t tile) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int i = tid + u * kMqThreads;
      const int tok = i / KRW, w = i % KRW;
      const int64_t t = tile + tok;
      rk[u] = (i < kMqTile * KRW && t < p.ctx)
                  ? reinterpret_cast<const uint32_t*>(p.kidx)[(kv_base + t) * KRW + w] : 0u;
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int i = tid + u * kMqThreads;
      const int tok = i / VRW, w = i % VRW;
      const int64_t t = tile + tok;
      rv[u] = (i < kMqTile * VRW && t < p.ctx)
                  ? reinterpret_cast<const uint32_t*>(p.vidx)[(kv_base + t) * VRW + w] : 0u;
    }
    if (tid < 2 * kMqTile) {
      const int64_t t = tile + (tid >> 1);
      rs = t < p.ctx ? reinterpret_cast<const uint32_t*>(p.kqjl)[(kv_base + t) * 2 + (tid & 1)] : 0u;
    } else if (tid < 3 * kMqTile) {
      const int64_t t = tile + (tid - 2 * kMqTile);
      const bool ok = t < p.ctx;
      rn0 = ok ? p.knorm[kv_base + t] : 0.f;
      rn1 = ok ? p.krnorm[kv_base + t] : 0.f;
      rn2 = ok ? p.vnorm[kv_base + t] : 0.f;
    }
  };
  // raw tile data lives in slot t % 2 and tile t's operands in buffer t % 2
  auto store_raw = [&](int rb) {
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
      const int i = tid + u * kMqThreads;
      if (i < kMqTile * KRW) s_kraw[rb][i / KRW][i % KRW] = rk[u];
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int i = tid + u * kMqThreads;
      if (i < kMqTile * VRW) s_vraw[rb][i / VRW][i % VRW] = rv[u];
    }
    if (tid < 2 * kMqTile) {
      s_sraw[rb][tid >> 1][tid & 1] = rs;
    } else if (tid < 3 * kMqTile) {
      const int tok = tid - 2 * kMqTile;
      const float nk = rn0 * p.scale;
      s_fk[rb][tok] = nk;
      s_fs[rb][tok] = nk * rn1 * p.qjl_scale;
      s_nv[rb][tok] = rn2;
    }
  };
  auto dequant = [&](int rb) {
    // dequantize: thread -> (token, CPT coordinates) for K and signs
    {
      const int tok = tid / (kMqTile / CPT), c0 = CPT * (tid % (kMqTile / CPT));
      const float fk = s_fk[rb][tok], fs = s_fs[rb][tok];
      uint32_t kh[CPT / 2], kl[CPT / 2];
#pragma unroll
      for (int j = 0; j < CPT; j += 2) {
        uint32_t code[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int bit = (c0 + j + e) * CBK;
          const int w = bit >> 5, sh = bit & 31;
          // both words, joined by one funnel shift (no lane-dependent branch)
          const uint32_t x = __builtin_amdgcn_alignbit(s_kraw[rb][tok][w + 1], s_kraw[rb][tok][w], sh);
          code[e] = x & ((1u << CBK) - 1u);
        }
        uint32_t h0, l0, h1, l1;
        mq_split(s_kc[code[0]] * fk, h0, l0);
        mq_split(s_kc[code[1]] * fk, h1, l1);
        kh[j >> 1] = h0 | (h1 << 16);
        kl[j >> 1] = l0 | (l1 << 16);
      }
      uint32_t fh, fl;
      mq_split(fs, fh, fl);
      const uint32_t sb = (s_sraw[rb][tok][c0 >> 5] >> (c0 & 31)) & ((1u << CPT) - 1u);
      uint32_t sh2[CPT / 2], sl2[CPT / 2];
#pragma unroll
      for (int j = 0; j < CPT; j += 2) {
        const uint32_t n0 = ((sb >> j) & 1u) ? 0u : 0x8000u;        // sign bit of -f
        const uint32_t n1 = ((sb >> (j + 1)) & 1u) ? 0u : 0x8000u;
        sh2[j >> 1] = (fh ^ n0) | ((fh ^ n1) << 16);
        sl2[j >> 1] = (fl ^ n0) | ((fl ^ n1) << 16);
      }
#pragma unroll
      for (int q4 = 0; q4 < CPT / 8; ++q4) {
        *reinterpret_cast<mq_u32x4*>(&s_kh[rb][tok][c0 + 8 * q4]) =
            mq_u32x4{kh[4 * q4], kh[4 * q4 + 1], kh[4 * q4 + 2], kh[4 * q4 + 3]};
        *reinterpret_cast<mq_u32x4*>(&s_kl[rb][tok][c0 + 8 * q4]) =
            mq_u32x4{kl[4 * q4], kl[4 * q4 + 1], kl[4 * q4 + 2], kl[4 * q4 + 3]};
        *reinterpret_cast<mq_u32x4*>(&s_sh[rb][tok][c0 + 8 * q4]) =
            mq_u32x4{sh2[4 * q4], sh2[4 * q4 + 1], sh2[4 * q4 + 2], sh2[4 * q4 + 3]};
        *reinterpret_cast<mq_u32x4*>(&s_sl[rb][tok][c0 + 8 * q4]) =
            mq_u32x4{sl2[4 * q4], sl2[4 * q4 + 1], sl2[4 * q4 + 2], sl2[4 * q4 + 3]};
      }
    }
    // values: thread -> (coordinate tid % 64, columns TPT (tid / 64) ... + TPT - 1);
    // column col holds token col with bits 2 and 3 swapped
    {
      const int c = tid & 63, col0 = TPT * (tid >> 6);
      const int bit = c * CBV, w = bit >> 5, sh = bit & 31;
      uint32_t vh[TPT / 2], vl[TPT / 2];
#pragma unroll
      for (int j = 0; j < TPT; j += 2) {
        float val[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int col = col0 + j + e;
          const int tok = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
          const uint32_t x = __builtin_amdgcn_alignbit(s_vraw[rb][tok][w + 1], s_vraw[rb][tok][w], sh);
          val[e] = s_vc[x & ((1u << CBV) - 1u)] * s_nv[rb][tok];
        }
        uint32_t h0, l0, h1, l1;
        mq_split(val[0], h0, l0);
        mq_split(val[1], h1, l1);
        vh[j >> 1] = h0 | (h1 << 16);
        vl[j >> 1] = l0 | (l1 << 16);
      }
#pragma unroll
      for (int q4 = 0; q4 < TPT / 8; ++q4) {
        *reinterpret_cast<mq_u32x4*>(&s_vh[rb][c][col0 + 8 * q4]) =
            mq_u32x4{vh[4 * q4], vh[4 * q4 + 1], vh[4 * q4 + 2], vh[4 * q4 + 3]};
        *reinterpret_cast<mq_u32x4*>(&s_vl[rb][c][col0 + 8 * q4]) =
            mq_u32x4{vl[4 * q4], vl[4 * q4 + 1], vl[4 * q4 + 2], vl[4 * q4 + 3]};
      }
    }
  };
  load_raw(0);
  store_raw(0);
  if (kMqTile < p.ctx) load_raw(kMqTile);
  __syncthreads();
  dequant(0);
  if (kMqTile < p.ctx) store_raw(1);
  if (2 * kMqTile < p.ctx) load_raw(2 * kMqTile);
  __syncthreads();

  int cur = 0;
  for (int64_t tile = 0; tile < p.ctx; tile += kMqTile, cur ^= 1) {
    // the next tile's operands, beside this tile's products.  Unconditional,
    // so that it shares a basic block with the score products and the
    // compiler interleaves the two (measured 2164 -> 2113 us per ESM-2-shaped
    // layer call); past the last tile it dequantizes stale raw words into the
    // buffer that is not read again.
    dequant(cur ^ 1);
    // ---- scores, transposed: rows = 32 tokens of block bk, column = query ----
    f32x16 S[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
#pragma unroll
      for (int v = 0; v < 16; ++v) S[bk][v] = 0.f;
      const int trow = 32 * bk + l32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int k0 = 16 * ks + 8 * h;
        const half8_t akh = *reinterpret_cast<const half8_t*>(&s_kh[cur][trow][k0]);
        const half8_t akl = *reinterpret_cast<const half8_t*>(&s_kl[cur][trow][k0]);
        const half8_t ash = *reinterpret_cast<const half8_t*>(&s_sh[cur][trow][k0]);
        const half8_t asl = *reinterpret_cast<const half8_t*>(&s_sl[cur][trow][k0]);
        const half8_t qh = __builtin_bit_cast(half8_t, fq[ks][0]);
        const half8_t ql = __builtin_bit_cast(half8_t, fq[ks][1]);
        const half8_t sqh = __builtin_bit_cast(half8_t, fq[ks][2]);
        const half8_t sql = __builtin_bit_cast(half8_t, fq[ks][3]);
        S[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(akh, qh, S[bk], 0, 0, 0);
        S[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(akh, ql, S[bk], 0, 0, 0);
        S[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(akl, qh, S[bk], 0, 0, 0);
        S[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ash, sqh, S[bk], 0, 0, 0);
        S[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ash, sql, S[bk], 0, 0, 0);
        S[bk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(asl, sqh, S[bk], 0, 0, 0);
      }
    }
    // token of S[bk][v]: tile + 32 bk + 8 (v / 4) + 4 h + v % 4
    float mt = -INFINITY;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t t = tile + 32 * bk + 8 * (v >> 2) + 4 * h + (v & 3);
        if (t >= p.ctx) S[bk][v] = -INFINITY;
        mt = fmaxf(mt, S[bk][v]);
      }
    if (p.scores_out != nullptr && rok) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t t = tile + 32 * bk + 8 * (v >> 2) + 4 * h + (v & 3);
          if (t < p.ctx) p.scores_out[(row_base + r) * p.ctx + t] = S[bk][v];
        }
    }
    mt = fmaxf(mt, mq_partner(mt, h));
    const float mn = fmaxf(m_run, mt);                 // finite: the tile has a valid token
    const float alpha = __expf(m_run - mn);            // 0 on the first tile
    m_run = mn;
    float ls = 0.f;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        S[bk][v] = __expf(S[bk][v] - mn);
        ls += S[bk][v];
      }
    l_run = fmaf(l_run, alpha, ls);
    if (alpha != 1.f) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[cb][v] *= alpha;
    }

    // ---- values: O^T += V^T P^T, 16 tokens per product ----
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int bk = ks >> 1, v0 = 8 * (ks & 1);
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t h0, l0, h1, l1;
        mq_split(S[bk][v0 + 2 * j], h0, l0);
        mq_split(S[bk][v0 + 2 * j + 1], h1, l1);
        ph[j] = h0 | (h1 << 16);
        pl[j] = l0 | (l1 << 16);
      }
      const half8_t bph = __builtin_bit_cast(half8_t, mq_u32x4{ph[0], ph[1], ph[2], ph[3]});
      const half8_t bpl = __builtin_bit_cast(half8_t, mq_u32x4{pl[0], pl[1], pl[2], pl[3]});
      const int col = 32 * bk + 16 * (ks & 1) + 8 * h;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const half8_t avh = *reinterpret_cast<const half8_t*>(&s_vh[cur][32 * cb + l32][col]);
        const half8_t avl = *reinterpret_cast<const half8_t*>(&s_vl[cur][32 * cb + l32][col]);
        O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(avh, bph, O[cb], 0, 0, 0);
        O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(avh, bpl, O[cb], 0, 0, 0);
        O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(avl, bph, O[cb], 0, 0, 0);
      }
    }
    // tile + 2 into the raw slot the previous dequantization freed (not read
    // in this pass), tile + 3 in flight
    if (tile + 2 * kMqTile < p.ctx) store_raw(cur);
    if (tile + 3 * kMqTile < p.ctx) load_raw(tile + 3 * kMqTile);
    __syncthreads();     // buffer cur^1 written, buffer cur and raw slot cur^1 read
  }

  // ---- o = D_V H (O / L) / sqrt(d) for this lane's query ----
  const float L = l_run + mq_partner(l_run, h);
  const float inv = 1.f / L;
  float x[2][16];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) x[cb][v] = O[cb][v] * inv;
  // coordinate bits: 0, 1 = v & 3; 2 = h; 3, 4 = v >> 2; 5 = cb
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {       // v bits (coordinate bits 0, 1, 3, 4)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((v & m) == 0) {
          const float a = x[cb][v], c = x[cb][v | m];
          x[cb][v] = a + c;
          x[cb][v | m] = a - c;
        }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {           // cb (coordinate bit 5)
    const float a = x[0][v], c = x[1][v];
    x[0][v] = a + c;
    x[1][v] = a - c;
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)           // h (coordinate bit 2), across lane halves
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float o = mq_partner(x[cb][v], h);
      x[cb][v] = h ? (o - x[cb][v]) : (x[cb][v] + o);
    }
  if (rok) {
    float* dst = p.out + (row_base + r) * D;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int i0 = 32 * cb + 8 * v4 + 4 * h;
        float o4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + e;
          const uint32_t bit = (p.vflip[i >> 5] >> (i & 31)) & 1u;
          const float o = x[cb][4 * v4 + e] * p.inv_sqrt_d;
          o4[e] = bit ? -o : o;
        }
        *reinterpret_cast<float4*>(dst + i0) = make_float4(o4[0], o4[1], o4[2], o4[3]);
      }
  }
}

bool mq_path(int n_q, int hq, int hkv, int d) {
  return d == 64 && !decode_path(n_q, hq, hkv);
}

size_t mq_workspace_bytes(int batch, int n_q, int hq) {
  (void)batch; (void)n_q; (void)hq;
  return 0;      // the query preparation runs inside the kernel
}

template <int CBK, int CBV>
static hipError_t run_mq(const MqParams& p, unsigned blocks, hipStream_t s) {
  hipLaunchKernelGGL((attend_mq_kernel<CBK, CBV>), dim3(blocks), dim3(kMqThreads), 0, s, p);
  return hipGetLastError();
}

template <int CBK>
static hipError_t mq_pick_v(int cbv, const MqParams& p, unsigned blocks, hipStream_t s) {
  switch (cbv) {
    case 1: return run_mq<CBK, 1>(p, blocks, s);
    case 2: return run_mq<CBK, 2>(p, blocks, s);
    case 3: return run_mq<CBK, 3>(p, blocks, s);
    case 4: return run_mq<CBK, 4>(p, blocks, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attend_mq(const tq_codec& kc, const tq_codec& vc, const void* q, int q_dtype,
                            int batch, int n_q, int hq, int hkv, const RopeHost& rope,
                            const tq_packed& k, const tq_packed& v, int64_t ctx, float scale,
                            float* out, float* scores_out, void* workspace, hipStream_t stream) {
  constexpr int D = 64;
  (void)workspace;
  if (kc.d != D) return hipErrorInvalidValue;
  MqParams p = {};
  p.kidx = k.idx; p.kqjl = k.qjl; p.knorm = k.norm; p.krnorm = k.rnorm;
  p.vidx = v.idx; p.vnorm = v.norm;
  p.q = q;
  p.q_f16 = q_dtype == TQ_F16;
  p.rope = rope.on ? 1 : 0;
  p.pos0 = rope.on ? rope.pos0 : 0;
  for (int i = 0; i < D / 2; ++i)
    p.theta[i] = rope.on ? std::pow((double)rope.base, -2.0 * i / (double)D) : 0.0;
  p.S = kc.S;
  p.kflip[0] = kc.flip[0];
  p.kflip[1] = kc.flip[1];
  p.out = out; p.scores_out = scores_out;
  p.ctx = ctx; p.hq = hq; p.hkv = hkv; p.n_q = n_q; p.G = hq / hkv;
  p.nqb = (p.G * n_q + kMqRows - 1) / kMqRows;
  p.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
  p.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / kc.m);
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)D));
  for (int i = 0; i < 16; ++i) { p.kcent[i] = kc.centroids[i]; p.vcent[i] = vc.centroids[i]; }
  p.vflip[0] = vc.flip[0];
  p.vflip[1] = vc.flip[1];
  const unsigned blocks = (unsigned)((int64_t)batch * hkv * p.nqb);
  switch (kc.code_bits) {
    case 1: return mq_pick_v<1>(vc.code_bits, p, blocks, stream);
    case 2: return mq_pick_v<2>(vc.code_bits, p, blocks, stream);
    case 3: return mq_pick_v<3>(vc.code_bits, p, blocks, stream);
    case 4: return mq_pick_v<4>(vc.code_bits, p, blocks, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tqk
