// Decode attention from packed codes on the matrix cores, d = 128, up to four
// query rows per workgroup (the G query heads of one KV head at one
// position).
//
// "TurboESM", "2. Metodologia" part E (one pass over the codes: unpack,
// correct, attend with an online softmax); "Google presenta TurboQuant",
// "Eliminación del sesgo interno del producto" (the unbiased estimate):
//   s_j = scale nu_j ( <q', c_K[idx_j]> + sqrt(pi/2)/m gamma_j <S q', 2 sigma_j - 1> )
//   o   = Pi_V^T sum_j softmax(s)_j nu^V_j c_V[idx^V_j]
//
// Scores as an integer product of the code bits.  The key table is odd
// (c[L-1-k] = -c[k]), so in the +-1 variables s_p = 2 b_p - 1 of the code
// bits it is a sum of odd monomials: c = sum_p alpha_p s_p (+ alpha_3
// s_0 s_1 s_2 for 3-bit codes; four cubic terms for 4-bit codes).  Hence
//   <q', c[idx]> = 2 sum_S alpha_S sum_i q'_i b^S_i - c[L-1] sum_i q'_i
// with b^S the code bits (linear terms) or their xor (cubic terms), and
//   <S q', 2 sigma - 1> = 2 sum_i (S q')_i sigma_i - sum_i (S q')_i.
// Both bit sums are products of a 0/1 matrix (16 tokens x the bits of their
// rows) with fixed query columns, which v_mfma_i32_16x16x64_i8 computes
// exactly: A holds the raw packed words masked to one bit per byte
// (w & (0x01010101 << j): byte value 2^j b, or -128 b for j = 7), B holds the
// query column times 2^-j (negated for j = 7) as four int8 limbs of a per-row power-of-two fixed point (rows
// (limb, query row) of the 16 columns).  Products of the stream's raw bits
// cover the linear terms without unpacking the codes; the cubic terms come
// from xors of shifted words.
//
// Value sum as rank-one updates on the matrix cores: v_mfma_f32_4x4x1f32
// with A = the softmax weights of one token (4 query rows) and B = the
// centroid value of one coordinate, 16 blocks of (token, 4 coordinates) per
// instruction, accumulating over the tokens in fp32.
//
// Softmax: online, per wave, with a lazily raised reference maximum (the
// accumulators are rescaled only when a tile's maximum exceeds the
// reference by more than 8, so weights stay below e^8).  The waves merge in
// LDS and the workgroup writes (acc, max, sum) per row for the log-sum-exp
// merge kernel, which applies Pi_V^T once per row.

#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"

namespace tqk {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMD = 128;        // head dimension of this kernel
constexpr int kMRows = 4;       // query rows per workgroup (= the merge record rows)
constexpr int kMGroup = 16;     // tokens per wave step

template <int CBK>
struct KeyMfma {
  static constexpr int NL = 2 * CBK;                                  // linear-term products
  static constexpr int NC = CBK == 3 ? 2 : (CBK == 4 ? 8 : 0);        // cubic-term products
  static constexpr int NQ = 2;                                        // QJL products
  static constexpr int NM = NL + NC + NQ;
};

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Whole-wave reductions: DPP inside each 16-lane row (quad xor 1, quad
// xor 2, half-row mirror, row mirror), then the four rows through scalar
// reads; every lane gets the result.
__device__ __forceinline__ float wave_max64(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_sum64(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

// Maximum over the 16 lanes of each row: four maxima with a DPP-permuted
// operand (quad xor 1, quad xor 2, half-row mirror, row mirror).  Written
// out because fmaxf on a DPP move compiles to the move, the maximum and one
// or two canonicalizing maxima per stage.  Two wait states before each DPP
// read of a VGPR written by the previous VALU instruction.
__device__ __forceinline__ float row16_max(float v) {
  asm("s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf"
      : "+v"(v));
  return v;
}

// The smallest power of two F with m / F <= 127 (1 for m = 0).
__device__ __forceinline__ float limb_scale(float m) {
  if (!(m > 0.f)) return 1.f;
  int e;
  frexpf(m * (1.f / 127.f), &e);
  return ldexpf(1.f, e);
}

// The four int8 limbs of v, |v| <= 127: v = a0 + a1/128 + a2/128^2 + a3/128^3
// (up to 2^-22) with a0 = rint(v) and |a_k| <= 64 after it; every step is
// exact in fp32.  Returned as bytes 0..3 of a word.
__device__ __forceinline__ uint32_t limbs_of(float v) {
  uint32_t out = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = rintf(v);
    out |= ((uint32_t)(int)a & 0xffu) << (8 * k);
    v = (v - a) * 128.f;
  }
  return out;
}

// One wave step's loads: the key words of the lane's 32 coordinates of
// token t = lane % 16, its QJL word and norms, and the lane's value bits of
// tokens 4 (lane / 16) + i, i = 0..3.
template <int CBK, int CBV>
struct StepRegs {
  static constexpr bool VSTR = (8 * CBV) % 32 != 0 && CBV == 3;   // value bits may straddle words
  uint32_t kw[CBK];
  uint32_t qw;
  float nk, gk, nv;      // norms of token lane % 16
  uint32_t v0[4], v1[4];
};

}  // namespace

struct MfmaDecodeArgs {
  const void* q;
  int q_f16;
  const uint8_t* kidx;
  const uint8_t* kqjl;
  const float* knorm;
  const float* krnorm;
  const uint8_t* vidx;
  const float* vnorm;
  const float* S;
  float* scores_out;
  float* part;            // [bgc][split][kMRows][D + 2]
  int64_t ctx;
  int hq, hkv, n_q, G, nchunks, splits;
  int64_t split_len;
  float scale, qjl_scale, inv_sqrt_d;
  int rope;
  int32_t pos0;
  float alpha[8];         // key table in odd monomials: b0..b(CB-1), then the cubic terms
  float alpha_max;        // max |alpha|
  float ktop;             // c_K[L - 1] = sum of the alphas
  float vcent[16];
  uint32_t kflip[4];
  double theta[64];
};

template <int CBK, int CBV, int W>
__global__ __launch_bounds__(W * 64) void decode_mfma_kernel(MfmaDecodeArgs p) {
  constexpr int D = kMD;
  constexpr int THREADS = W * 64;
  using KM = KeyMfma<CBK>;
  constexpr int NL = KM::NL, NC = KM::NC, NM = KM::NM;
  constexpr int KROW = D * CBK / 8;
  constexpr int VROW = D * CBV / 8;
  constexpr int KP = 4;                        // k-parts of S q' (threads 0..511)
  constexpr int KL = D / KP;
  static_assert(THREADS >= KP * D, "S q' split");
  static_assert(W >= kMRows, "one wave per query row in the set-up");

  __shared__ float s_q[kMRows][D];             // q' = Pi RoPE(q)
  __shared__ float s_sq[kMRows][D];            // S q'
  __shared__ __align__(16) float s_big[W * kMRows * (D + 2) > KP * kMRows * D
                                           ? W * kMRows * (D + 2) : KP * kMRows * D];
  __shared__ __align__(16) uint4 s_lb[NM][64]; // B operands: query limbs
  __shared__ float s_F[kMRows], s_T[kMRows], s_U[kMRows];
  __shared__ float s_Fi[kMRows], s_Gi[kMRows];   // 1 / s_F and the QJL limb scale (powers of two)
  __shared__ float s_ws[16];                   // per-wave max |S q'| and sum
  __shared__ float s_vc[16];
  __shared__ float s_alpha[8];                 // key table in odd monomials
  __shared__ __align__(16) float s_wt[W * 64];   // per-wave weight transpose

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int bgc = blockIdx.x;
  const int split = blockIdx.y;
  const int bg = bgc / p.nchunks, chunk = bgc % p.nchunks;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int qr_total = p.G * p.n_q;
  const int lr0 = chunk * kMRows;
  const int nrows = (qr_total - lr0) < kMRows ? (qr_total - lr0) : kMRows;
  const int64_t row_base = ((int64_t)b * p.hq + (int64_t)g * p.G) * p.n_q + lr0;
  const int64_t t0 = (int64_t)split * p.split_len;
  int64_t t1 = t0 + p.split_len;
  if (t1 > p.ctx) t1 = p.ctx;
  const int64_t kv_base = (int64_t)bg * p.ctx;
  const int ng = (int)((t1 - t0 + kMGroup - 1) / kMGroup);

  // lane roles: key bits (row = token t, k-slice lg), score columns
  // (n = 4 lam + r: limb lam of query row r), value blocks (token slot lg,
  // coordinates 8 (lane % 16) .. + 7)
  const int lg = lane >> 4, lt = lane & 15;
  const int rr = lt & 3;

  // Buffer descriptors over this (batch, KV head)'s ctx rows of each plane:
  // 32-bit offsets, and rows past ctx read as zero (no clamping; tokens past
  // the range end are masked out of the softmax)
  const uint32_t nctx = (uint32_t)p.ctx;
  constexpr int kRsrcWord3 = 0x00020000;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.kidx + kv_base * KROW), (short)0, (int)(nctx * KROW), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.kqjl + kv_base * (D / 8)), (short)0, (int)(nctx * (D / 8)), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.vidx + kv_base * VROW), (short)0, (int)(nctx * VROW), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rnk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.knorm + kv_base), (short)0, (int)(nctx * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rgk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.krnorm + kv_base), (short)0, (int)(nctx * 4), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rnv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.vnorm + kv_base), (short)0, (int)(nctx * 4), kRsrcWord3);
  typedef uint32_t u2v __attribute__((ext_vector_type(2)));
  typedef uint32_t u3v __attribute__((ext_vector_type(3)));
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const int vbit = 8 * CBV * lt;
  const int vdw = vbit >> 5;

  // per-lane byte offsets inside a step; the step's own offset is
  // wave-uniform and goes in the scalar offset of each load
  const int ko_b = lt * KROW + 4 * CBK * lg;
  const int qo_b = lt * (D / 8) + 4 * lg;
  const int no_b = 4 * lt;
  const int vo_b = 4 * lg * VROW + 4 * vdw;

  auto load_step = [&](int gi, StepRegs<CBK, CBV>& R) {
    const int tb0 = __builtin_amdgcn_readfirstlane((int)(t0 + (int64_t)gi * kMGroup));
    // a whole group of rows inside [0, ctx): the step offset goes in the
    // scalar offset.  The group at the range's end may run past ctx: there
    // every offset is a vector offset, so the descriptor's range check (which
    // does not cover the scalar offset) turns the rows past ctx into zeros.
    const bool whole = tb0 + kMGroup <= (int)nctx;
    const int tb = whole ? tb0 : 0;
    const int vb = whole ? 0 : tb0;
    const int ko_l = ko_b + vb * KROW, qo_l = qo_b + vb * (D / 8), no_l = no_b + vb * 4;
    const int vo_l = vo_b + vb * VROW;
    if constexpr (CBK == 1) {
      R.kw[0] = __builtin_amdgcn_raw_buffer_load_b32(rk, ko_l, tb * KROW, 0);
    } else if constexpr (CBK == 2) {
      const u2v v = __builtin_amdgcn_raw_buffer_load_b64(rk, ko_l, tb * KROW, 0);
      R.kw[0] = v.x; R.kw[1] = v.y;
    } else if constexpr (CBK == 3) {
      const u3v v = __builtin_amdgcn_raw_buffer_load_b96(rk, ko_l, tb * KROW, 0);
      R.kw[0] = v.x; R.kw[1] = v.y; R.kw[2] = v.z;
    } else {
      const u4v v = __builtin_amdgcn_raw_buffer_load_b128(rk, ko_l, tb * KROW, 0);
      R.kw[0] = v.x; R.kw[1] = v.y; R.kw[2] = v.z; R.kw[3] = v.w;
    }
    R.qw = __builtin_amdgcn_raw_buffer_load_b32(rq, qo_l, tb * (D / 8), 0);
    R.nk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rnk, no_l, tb * 4, 0));
    R.gk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rgk, no_l, tb * 4, 0));
    R.nv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rnv, no_l, tb * 4, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int so = (tb + i) * VROW;
      if constexpr (StepRegs<CBK, CBV>::VSTR) {
        // the last word of a row is never straddled: a load past the row's
        // end only reads the next row's first word (or zero past ctx)
        const u2v v = __builtin_amdgcn_raw_buffer_load_b64(rv, vo_l, so, 0);
        R.v0[i] = v.x;
        R.v1[i] = v.y;
      } else {
        R.v0[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo_l, so, 0);
      }
    }
  };

  // ---- set-up ----
  // Loads in the order they are needed, none waited on before the next one
  // is issued: the query rows (wave 0), the S rows of S q' (cached after the
  // first workgroups), and only once the query rows are rotated, the first
  // steps' codes: one step after each of the first two set-up barriers and
  // the rest once the set-up is done.  A CU holds a limited number of loads
  // in flight, and while its waves' codes stream in at the CU's share of HBM
  // bandwidth a wave that issues one more load waits at that instruction,
  // and with it the set-up arithmetic behind it; spread out, the requests
  // overlap the set-up without holding it back (measured: 24.1 -> 23.3 us
  // per GQA call against all three steps requested after the rotation; all
  // after the set-up, 24.0 us).  Issued before the rotation, the codes of
  // every workgroup would queue in front of the query rows.  Each step
  // refills its slot, NBUF steps ahead, once it is done with it.  Kernel
  // arguments read at a per-lane index would be memory loads on this chain:
  // the code tables reach LDS through scalar reads instead.
  // Wave 0 rotates all four query rows: lane (row r = lane / 16, j = lane % 16)
  // holds coordinates 8 j .. 8 j + 7 of row r.
  // steps in flight per wave (measured: 2 and 4 slower than 3; 4-bit key
  // tables leave room for 2)
  constexpr int NBUF = CBK == 4 ? 2 : 3;
  StepRegs<CBK, CBV> ring[NBUF] = {};
  // A step past the wave's last one reloads that last step (cached; the
  // data goes unused): every pass issues the same loads, so the wait before
  // a step counts only the loads older than its own, not all in flight.
  const int last_step = wave < ng ? wave + ((ng - 1 - wave) / W) * W : wave;
  auto load_clamped = [&](int g, StepRegs<CBK, CBV>& R) { load_step(g < ng ? g : last_step, R); };

  const int qr = lane >> 4, qj = lane & 15;
  uint4 qraw0 = make_uint4(0u, 0u, 0u, 0u), qraw1 = qraw0;
  if (wave == 0 && qr < nrows) {
    // the lane's 8 coordinates: 16 bytes of fp16 or 32 bytes of fp32
    const int64_t off = (row_base + qr) * D + 8 * qj;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(p.q) + off * (p.q_f16 ? 2 : 4));
    qraw0 = src[0];
    qraw1 = src[p.q_f16 ? 0 : 1];   // (unused for fp16: a second read of the first 16 bytes)
  }
  const MfmaDecodeArgs* kp = (const MfmaDecodeArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  // RoPE angles of the lane's four coordinate pairs, loaded beside the query
  double th[4] = {0.0, 0.0, 0.0, 0.0};
  if (wave == 0 && p.rope) {
#pragma unroll
    for (int c = 0; c < 4; ++c) th[c] = kp->theta[4 * qj + c];
  }
  // S rows for S q': thread -> (coordinate si, k-part sp)
  // (with exactly KP D threads every thread loads: no branch, so the wait
  // for the query rows does not also wait for these loads)
  const int si = tid % D, sp = tid / D;
  const bool sq_thread = THREADS == KP * D || tid < KP * D;
  float4 srow[KL / 4];
  if (sq_thread) {
    const float4* S4 = reinterpret_cast<const float4*>(p.S + (size_t)si * D + sp * KL);
#pragma unroll
    for (int j = 0; j < KL / 4; ++j) srow[j] = S4[j];
  }
  if (tid == 64) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s_vc[i] = p.vcent[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) s_alpha[i] = p.alpha[i];
  }
  if (wave == 0) {
    float x[8];
    if (p.q_f16) {
      const uint32_t u[4] = {qraw0.x, qraw0.y, qraw0.z, qraw0.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        x[2 * c] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[c] & 0xffffu));
        x[2 * c + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u[c] >> 16));
      }
    } else {
      x[0] = __uint_as_float(qraw0.x); x[1] = __uint_as_float(qraw0.y);
      x[2] = __uint_as_float(qraw0.z); x[3] = __uint_as_float(qraw0.w);
      x[4] = __uint_as_float(qraw1.x); x[5] = __uint_as_float(qraw1.y);
      x[6] = __uint_as_float(qraw1.z); x[7] = __uint_as_float(qraw1.w);
    }
    if (p.rope) {
      // interleaved pairs (2 p, 2 p + 1), p = 4 j + c
      const int64_t pos = (int64_t)p.pos0 + ((lr0 + qr) % p.n_q);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float sn, cs;
        sincos_reduced((double)pos * th[c], sn, cs);
        const float a0 = x[2 * c], b0 = x[2 * c + 1];
        x[2 * c] = a0 * cs - b0 * sn;
        x[2 * c + 1] = a0 * sn + b0 * cs;
      }
    }
    const int fq = qj >> 2;
    const uint32_t kfw = fq == 0 ? p.kflip[0] : (fq == 1 ? p.kflip[1] : (fq == 2 ? p.kflip[2] : p.kflip[3]));
    const uint32_t fw = (kfw >> (8 * (qj & 3))) & 0xffu;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      x[c] = __uint_as_float(__float_as_uint(x[c]) ^ (((fw >> c) & 1u) << 31));
    // butterflies on coordinate bits 0..2 inside the lane
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if ((c & h) == 0) {
          const float u0 = x[c], u1 = x[c + h];
          x[c] = u0 + u1;
          x[c + h] = u0 - u1;
        }
    // bits 3..6 across the lanes of the row (lane bits 0..3), by DPP:
    // quad xor 1, quad xor 2, xor 4 (row_ror 4 or 12), xor 8 (row_ror 8)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float w = dppf<0xB1>(x[c]);
      x[c] = (qj & 1) ? (w - x[c]) : (x[c] + w);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float w = dppf<0x4E>(x[c]);
      x[c] = (qj & 2) ? (w - x[c]) : (x[c] + w);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float w4 = dppf<0x124>(x[c]), w12 = dppf<0x12C>(x[c]);
      x[c] = (qj & 4) ? (w4 - x[c]) : (x[c] + w12);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float w = dppf<0x128>(x[c]);
      x[c] = (qj & 8) ? (w - x[c]) : (x[c] + w);
    }
    float mq = 0.f, tq = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      x[c] *= p.inv_sqrt_d;
      mq = fmaxf(mq, fabsf(x[c]));
      tq += x[c];
    }
    *reinterpret_cast<float4*>(&s_q[qr][8 * qj]) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(&s_q[qr][8 * qj + 4]) = make_float4(x[4], x[5], x[6], x[7]);
    // row statistics over the 16 lanes of the row
    mq = fmaxf(mq, dppf<0xB1>(mq));
    mq = fmaxf(mq, dppf<0x4E>(mq));
    mq = fmaxf(mq, dppf<0x141>(mq));
    mq = fmaxf(mq, dppf<0x140>(mq));
    tq += dppf<0xB1>(tq);
    tq += dppf<0x4E>(tq);
    tq += dppf<0x141>(tq);
    tq += dppf<0x140>(tq);
    if (qj == 0) {
      // the inverse of a power of two (exact); the scan takes F = 1 / it
      const float fs = limb_scale(2.f * p.alpha_max * mq);
      s_F[qr] = 1.f / fs;
      s_Fi[qr] = fs;
      s_T[qr] = p.ktop * tq;
    }
  }
  __syncthreads();
  load_clamped(wave, ring[0]);

  // B operands: for product u, lane (g, n = 4 lam + r), dword s, byte e the
  // limb lam of (2 coef x 2^-j) / F_r, where the byte pairs with bit j of
  // byte e of the A dword (see the key-bit masks in the scan below).  One
  // item t = (u, g, r, s, e) writes that byte of all four limb lanes.  The
  // code-bit products need only q', so they are built while the S rows are
  // still arriving; the QJL products follow S q'.
  uint8_t* lb8 = reinterpret_cast<uint8_t*>(&s_lb[0][0]);
  auto limb_item = [&](int t) {
    const int e = t & 3, s = (t >> 2) & 3, r = (t >> 4) & 3, gg = (t >> 6) & 3, u = t >> 8;
    int j, coord;
    float x;
    bool qjl = false;
    if (u < NL) {
      const int up = 4 * u + s, a = up >> 3;
      j = up & 7;
      const int P = 32 * a + 8 * e + j;
      coord = 32 * gg + P / CBK;
      x = s_alpha[P % CBK] * s_q[r][coord];
    } else if (u < NL + NC) {
      if constexpr (CBK == 3) {
        j = 4 * (u - NL) + s;
        const int P = 8 * e + j, a = P % 3;
        coord = 32 * gg + (P + 32 * a) / 3;
        x = s_alpha[3] * s_q[r][coord];
      } else {
        const int up = 4 * (u - NL) + s, a = up >> 3;
        j = up & 7;
        const int P = 8 * e + j;
        coord = 32 * gg + 8 * a + (P >> 2);
        x = s_alpha[4 + (P & 3)] * s_q[r][coord];
      }
    } else {
      j = 4 * (u - NL - NC) + s;
      coord = 32 * gg + 8 * e + j;
      x = s_sq[r][coord];
      qjl = true;
    }
    // the A byte of bit 7 reads as int8 -128: the sign moves into B
    const float invF = qjl ? 1.f / limb_scale(2.f * fmaxf(s_ws[4 * r], s_ws[4 * r + 2])) : s_F[r];
    const uint32_t l4 = limbs_of(ldexpf(j == 7 ? -2.f * x : 2.f * x, -j) * invF);
#pragma unroll
    for (int la = 0; la < 4; ++la)
      lb8[(u * 64 + 16 * gg + 4 * la + r) * 16 + 4 * s + e] = (uint8_t)(l4 >> (8 * la));
  };
  constexpr int NKC = (NL + NC) * 256;   // items of the code-bit products
#pragma unroll
  for (int k = 0; k < (NKC + THREADS - 1) / THREADS; ++k) {
    const int t = tid + k * THREADS;
    if (t < NKC) limb_item(t);
  }

  // S q' partial sums over this thread's k-part
  if (sq_thread) {
    float a[kMRows] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KL / 4; ++j) {
      const int k = sp * KL + 4 * j;
#pragma unroll
      for (int r = 0; r < kMRows; ++r) {
        a[r] = fmaf(s_q[r][k], srow[j].x, a[r]);
        a[r] = fmaf(s_q[r][k + 1], srow[j].y, a[r]);
        a[r] = fmaf(s_q[r][k + 2], srow[j].z, a[r]);
        a[r] = fmaf(s_q[r][k + 3], srow[j].w, a[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kMRows; ++r) s_big[(sp * kMRows + r) * D + si] = a[r];
  }
  __syncthreads();
  load_clamped(wave + W, ring[1]);
  // S q' rows; each of waves 0..7 (two per row) also leaves its 64 values'
  // max |.| and sum, combined in a fixed order below
  if (tid < kMRows * D) {
    const int r = tid / D, i = tid % D;
    float a = 0.f;
#pragma unroll
    for (int q = 0; q < KP; ++q) a += s_big[(q * kMRows + r) * D + i];
    s_sq[r][i] = a;
    const float mu = wave_max64(fabsf(a));
    const float tu = wave_sum64(a);
    if (lane == 0) {
      s_ws[2 * wave] = mu;
      s_ws[2 * wave + 1] = tu;
    }
  }
  __syncthreads();
  for (int t = NKC + tid; t < NM * 256; t += THREADS) limb_item(t);
  if (tid < kMRows) {
    s_Gi[tid] = limb_scale(2.f * fmaxf(s_ws[4 * tid], s_ws[4 * tid + 2]));
    s_U[tid] = s_ws[4 * tid + 1] + s_ws[4 * tid + 3];
  }
  __syncthreads();
#pragma unroll
  for (int k = 2; k < NBUF; ++k) load_clamped(wave + k * W, ring[k]);

  uint4 bop[NM];
#pragma unroll
  for (int u = 0; u < NM; ++u) bop[u] = s_lb[u][lane];
  // per-lane score constants: after the products, lane (g, n) holds limb g
  // of query rows 0..3 for token n; the limb's weight times each row's
  // scale, and each row's constant term, carried by limb 0 only
  const float limb_w = ldexpf(1.f, -7 * lg);
  float xw[kMRows], yw[kMRows], xc[kMRows], yc[kMRows];
#pragma unroll
  for (int r = 0; r < kMRows; ++r) {
    xw[r] = limb_w * s_Fi[r];     // exact: powers of two
    yw[r] = limb_w * s_Gi[r];
    xc[r] = lg == 0 ? -s_T[r] : 0.f;
    yc[r] = lg == 0 ? -s_U[r] : 0.f;
  }
  // the value weights of each wave pass through LDS from the score layout
  // (lane (row g, token n)) to the value layout (lane (token slot lg, ...,
  // row lane % 4) holding tokens 4 lg + i)
  float* s_wave_w = s_wt + wave * 64;
  const int wt_put = (lt >> 2) * 16 + lg * 4 + (lt & 3);
  const int wt_get = lg * 16 + rr * 4;
  const float sc = p.scale, qs = p.qjl_scale;
  const uint32_t t1u = (uint32_t)t1;
  const float* vc_lds = s_vc;

  // ---- scan ----
  float m_ref = -INFINITY, l_run = 0.f;
  v4f acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = v4f{0.f, 0.f, 0.f, 0.f};
  const int voff = vbit & 31;

  // key bits times query limbs: integer bit sums of one step's 16 tokens
  auto keys = [&](const StepRegs<CBK, CBV>& R, v4i& cacc, v4i& qacc) {
    // scores: bit products of the 16 tokens' key rows with the query limbs
    // two accumulator chains for the code bits (summed below), one for QJL
    v4i cacc2 = {0, 0, 0, 0};
    cacc = v4i{0, 0, 0, 0};
    qacc = v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      uint32_t a4[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int up = 4 * u + s;
        a4[s] = R.kw[up >> 3] & (0x01010101u << (up & 7));
      }
      const v4i av = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3]};
      const v4i bv = {(int)bop[u].x, (int)bop[u].y, (int)bop[u].z, (int)bop[u].w};
      if (u & 1)
        cacc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, av, cacc2, 0, 0, 0);
      else
        cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, av, cacc, 0, 0, 0);
    }
    if constexpr (CBK == 3) {
      // xor of each code's three bits at the code's first bit, the three
      // words' code starts (positions = word index mod 3) folded into one
      const uint32_t w0 = R.kw[0], w1 = R.kw[1], w2 = R.kw[2];
      const uint32_t t0w = w0 ^ __builtin_amdgcn_alignbit(w1, w0, 1) ^ __builtin_amdgcn_alignbit(w1, w0, 2);
      const uint32_t t1w = w1 ^ __builtin_amdgcn_alignbit(w2, w1, 1) ^ __builtin_amdgcn_alignbit(w2, w1, 2);
      const uint32_t t2w = w2 ^ (w2 >> 1) ^ (w2 >> 2);
      const uint32_t cw = (t0w & 0x49249249u) | (t1w & 0x92492492u) | (t2w & 0x24924924u);
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const v4i av = {(int)(cw & (0x01010101u << (4 * u))), (int)(cw & (0x01010101u << (4 * u + 1))),
                        (int)(cw & (0x01010101u << (4 * u + 2))), (int)(cw & (0x01010101u << (4 * u + 3)))};
        const v4i bv = {(int)bop[NL + u].x, (int)bop[NL + u].y, (int)bop[NL + u].z, (int)bop[NL + u].w};
        if (u & 1)
          cacc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, av, cacc2, 0, 0, 0);
        else
          cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, av, cacc, 0, 0, 0);
      }
    } else if constexpr (CBK == 4) {
      uint32_t cw[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t w = R.kw[a];
        const uint32_t x1 = w ^ (w >> 1) ^ (w >> 2);    // nibble bit 0: b0^b1^b2, bit 1: b1^b2^b3
        const uint32_t x2 = w ^ (w >> 1) ^ (w >> 3);    // bit 0: b0^b1^b3
        const uint32_t x3 = w ^ (w >> 2) ^ (w >> 3);    // bit 0: b0^b2^b3
        cw[a] = (x1 & 0x33333333u) | ((x2 & 0x11111111u) << 2) | ((x3 & 0x11111111u) << 3);
      }
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        uint32_t a4[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int up = 4 * u + s;
          a4[s] = cw[up >> 3] & (0x01010101u << (up & 7));
        }
        const v4i av = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3]};
        const v4i bv = {(int)bop[NL + u].x, (int)bop[NL + u].y, (int)bop[NL + u].z, (int)bop[NL + u].w};
        if (u & 1)
          cacc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, av, cacc2, 0, 0, 0);
        else
          cacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, av, cacc, 0, 0, 0);
      }
    }
    cacc += cacc2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t qw = R.qw;
      const v4i av = {(int)(qw & (0x01010101u << (4 * u))), (int)(qw & (0x01010101u << (4 * u + 1))),
                      (int)(qw & (0x01010101u << (4 * u + 2))), (int)(qw & (0x01010101u << (4 * u + 3)))};
      const v4i bv = {(int)bop[NL + NC + u].x, (int)bop[NL + NC + u].y, (int)bop[NL + NC + u].z,
                      (int)bop[NL + NC + u].w};
      qacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, av, qacc, 0, 0, 0);
    }

  };

  // scores, online softmax with a lazily raised reference maximum, and the
  // tokens' value weights
  auto scores = [&](int gi, const StepRegs<CBK, CBV>& R, const v4i& cacc, const v4i& qacc,
                    float (&w)[4]) {
    const uint32_t tb = (uint32_t)(t0 + (int64_t)gi * kMGroup);
    const bool whole = tb + kMGroup <= t1u;      // wave-uniform
    // weight the limbs (lane group g = limb), then a reduce-scatter over
    // the four lane groups: group g ends with query row g of token n = lt
    float X[4], Y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      X[r] = fmaf((float)cacc[r], xw[r], xc[r]);
      Y[r] = fmaf((float)qacc[r], yw[r], yc[r]);
    }
    auto scatter = [](float (&v)[4]) {
      // lanes l, l ^ 32: the lower half keeps rows 0, 1, the upper rows 2, 3
      auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[0]), __float_as_uint(v[2]), false, false);
      auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[1]), __float_as_uint(v[3]), false, false);
      const float r02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      const float r13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
      // lanes l, l ^ 16: group g keeps row g
      auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(r02), __float_as_uint(r13), false, false);
      return __uint_as_float(c[0]) + __uint_as_float(c[1]);
    };
    const float Xs = scatter(X), Ys = scatter(Y);
    float sv = (R.nk * sc) * fmaf(qs * R.gk, Ys, Xs);
    const bool valid = whole || tb + lt < t1u;
    sv = valid ? sv : -INFINITY;
    if (p.scores_out != nullptr && lg < nrows && valid)
      p.scores_out[(row_base + lg) * p.ctx + tb + lt] = sv;

    // online softmax, lane group g = query row g
    const float mt = row16_max(sv);
    const bool bump = mt > m_ref + 8.f;
    if (__ballot(bump) != 0ull) {
      const float m_new = bump ? mt : m_ref;
      const float al = m_new == m_ref ? 1.f : __expf(m_ref - m_new);
      m_ref = m_new;
      l_run *= al;
      const float a0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 0));
      const float a1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 16));
      const float a2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 32));
      const float a3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 48));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e][0] *= a0;
        acc[e][1] *= a1;
        acc[e][2] *= a2;
        acc[e][3] *= a3;
      }
    }
    const float pe = valid ? __expf(sv - m_ref) : 0.f;
    l_run += pe;
    s_wave_w[wt_put] = pe * R.nv;
    // LDS operations of one wave complete in order: the read below sees the
    // write above (and the next step's write follows this read)
    __builtin_amdgcn_wave_barrier();
    const float4 w4 = *reinterpret_cast<const float4*>(s_wave_w + wt_get);
    w[0] = w4.x; w[1] = w4.y; w[2] = w4.z; w[3] = w4.w;
  };

  // value sum: rank-one updates of the accumulators with the weights w.
  // For 4-bit values each accumulator takes its four tokens' updates back to
  // back (measured: 21.4 -> 21.1 us per GQA call against the token-major
  // order, same bits); for 3-bit values the token-major order is 0.3 us
  // faster per Llama-shaped call.
  auto values = [&](const StepRegs<CBK, CBV>& R, const float (&w)[4]) {
    uint32_t bits[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (StepRegs<CBK, CBV>::VSTR)
        bits[i] = __builtin_amdgcn_alignbit(R.v1[i], R.v0[i], voff);
      else
        bits[i] = R.v0[i] >> voff;
    }
    if constexpr (CBV == 4) {
      // the eight codes' byte offsets into the table: even codes from the
      // low nibbles, odd codes from the high nibbles, one byte each
      uint32_t ev[4], od[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ev[i] = (bits[i] & 0x0F0F0F0Fu) << 2;
        od[i] = (bits[i] >> 2) & 0x3C3C3C3Cu;
        // opaque to the optimizer, which would otherwise fold each byte
        // extraction back into a shift and a mask of bits (two instructions
        // per code instead of one)
        asm("" : "+v"(ev[i]), "+v"(od[i]));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t off = __builtin_amdgcn_ubfe((e & 1) ? od[i] : ev[i], 8 * (e >> 1), 8);
          const float c = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(vc_lds) + off);
          acc[e] = __builtin_amdgcn_mfma_f32_4x4x1f32(w[i], c, acc[e], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = vc_lds[(bits[i] >> (CBV * e)) & ((1u << CBV) - 1u)];
          acc[e] = __builtin_amdgcn_mfma_f32_4x4x1f32(w[i], c, acc[e], 0, 0, 0);
        }
    }
  };

  // Software pipeline over a wave's steps: the key products of the next
  // step are issued beside the value sum of the current one (independent
  // work for the matrix cores and the vector ALU), then the next step's
  // softmax runs.  NBUF register sets rotate (ring[0], ring[1], ...); a set
  // is refilled NBUF steps ahead once its value sum is issued.
  {
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    v4i cacc, qacc;
    // the wave's steps are wave, wave + W, ...: nst of them; step i sits in
    // slot i % NBUF.  Whole rounds of NBUF steps first (every pass issues
    // the same loads), then the rest.
    const int nst = wave < ng ? (ng - 1 - wave) / W + 1 : 0;
    if (nst > 0) {
      keys(ring[0], cacc, qacc);
      scores(wave, ring[0], cacc, qacc, w);
    }
    int it = 0;
    for (; it + NBUF <= nst; it += NBUF) {
#pragma unroll
      for (int k = 0; k < NBUF; ++k) {
        const int gc = wave + (it + k) * W;
        // Waves w and w + W / 2 share a SIMD, and the older one issues first
        // whenever both can: left alone, it finishes its steps well before
        // its partner, which then runs alone.  The younger wave takes the
        // higher priority once a quarter of its steps are done (measured:
        // 24.1 -> 23.6 us per GQA call, about 1 us less per Llama-shaped
        // layer; from the first step, no gain).
        if (wave >= W / 2 && it + k == nst / 4) __builtin_amdgcn_s_setprio(1);
        // next step's products (on stale registers past the end: unused)
        keys(ring[(k + 1) % NBUF], cacc, qacc);
        values(ring[k], w);
        load_clamped(gc + NBUF * W, ring[k]);
        if (it + k + 1 < nst) scores(gc + W, ring[(k + 1) % NBUF], cacc, qacc, w);
      }
    }
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k) {
      if (it + k < nst) {
        const int gc = wave + (it + k) * W;
        keys(ring[(k + 1) % NBUF], cacc, qacc);
        values(ring[k], w);
        if (it + k + 1 < nst) scores(gc + W, ring[(k + 1) % NBUF], cacc, qacc, w);
      }
    }
  }

  // ---- merge the lane rows, then the waves; write this range's record ----
  // Reduce-scatter of the 32 accumulators (index f = 4 e + m) over the four
  // 16-lane rows: each lane swap sums two accumulators across a pair of
  // rows at once and keeps one of them per row, so 16-lane row G ends with
  // the totals of query row m = 2 (G & 1) + G / 2, coordinates 8 lt + e.
  float r1[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    // lanes 0..31 keep f = 2 j, lanes 32..63 f = 2 j + 1
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[j >> 1][2 * (j & 1)]),
                                                    __float_as_uint(acc[j >> 1][2 * (j & 1) + 1]), false, false);
    r1[j] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  float tot[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    // rows 0 and 2 keep r1[2 e], rows 1 and 3 r1[2 e + 1]
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(r1[2 * e]), __float_as_uint(r1[2 * e + 1]),
                                                    false, false);
    tot[e] = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  const int mrow = 2 * ((lane >> 4) & 1) + (lane >> 5);
  // l_run: lane group g holds query row g's sums per token slot; sum the row
  l_run += dppf<0xB1>(l_run);
  l_run += dppf<0x4E>(l_run);
  l_run += dppf<0x141>(l_run);
  l_run += dppf<0x140>(l_run);
  __syncthreads();   // s_big (S q' partials) is free: wave merge space
  constexpr int REC = D + 2;
  float* mrg = s_big;   // [wave][row][D + 2]
#pragma unroll
  for (int e = 0; e < 8; ++e) mrg[(wave * kMRows + mrow) * REC + 8 * lt + e] = tot[e];
  if (lt == 0) {
    mrg[(wave * kMRows + lg) * REC + D] = m_ref;
    mrg[(wave * kMRows + lg) * REC + D + 1] = l_run;
  }
  __syncthreads();
  const int64_t rec0 = ((int64_t)bgc * p.splits + split) * kMRows;
  for (int t = tid; t < kMRows * D; t += THREADS) {
    const int r = t / D, i = t % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, mrg[(w * kMRows + r) * REC + D]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = mrg[(w * kMRows + r) * REC + D];
      const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
      a = fmaf(mrg[(w * kMRows + r) * REC + i], f, a);
      L = fmaf(mrg[(w * kMRows + r) * REC + D + 1], f, L);
    }
    float* rec = p.part + (rec0 + r) * REC;
    rec[i] = a;
    if (i == 0) {
      rec[D] = M;
      rec[D + 1] = L;
    }
  }
}

// ---------------------------------------------------------------------------

#ifndef TQ_DECODE_MFMA_WAVES
#define TQ_DECODE_MFMA_WAVES 8
#endif
constexpr int kMfmaWaves = TQ_DECODE_MFMA_WAVES;

// Odd-monomial coefficients of a code table: alpha_S = 2^-CB sum_k c[k]
// prod_{p in S} (2 b_p(k) - 1), for S the single bits, then (3 bits) {0,1,2}
// or (4 bits) {0,1,2}, {1,2,3}, {0,1,3}, {0,2,3}.  False when the table is
// not odd (an even term above rounding), which this kernel cannot express.
bool mfma_key_alphas(const float* c, int cb, float* alpha, float* amax) {
  const int L = 1 << cb;
  auto coef = [&](unsigned set) {
    double s = 0.0;
    for (int k = 0; k < L; ++k) {
      double chi = 1.0;
      for (int b = 0; b < cb; ++b)
        if ((set >> b) & 1u) chi *= ((k >> b) & 1) ? 1.0 : -1.0;
      s += (double)c[k] * chi;
    }
    return s / L;
  };
  double mx = 0.0;
  for (int k = 0; k < L; ++k) mx = std::fmax(mx, std::fabs((double)c[k]));
  for (unsigned set = 0; set < (unsigned)L; ++set)
    if (__builtin_popcount(set) % 2 == 0 && std::fabs(coef(set)) > 1e-6 * mx) return false;
  int n = 0;
  for (int b = 0; b < cb; ++b) alpha[n++] = (float)coef(1u << b);
  if (cb == 3) alpha[n++] = (float)coef(7u);
  if (cb == 4) {
    alpha[n++] = (float)coef(0x7u);
    alpha[n++] = (float)coef(0xEu);
    alpha[n++] = (float)coef(0xBu);
    alpha[n++] = (float)coef(0xDu);
  }
  double am = 0.0;
  for (int i = 0; i < n; ++i) am = std::fmax(am, std::fabs((double)alpha[i]));
  for (int i = n; i < 8; ++i) alpha[i] = 0.f;
  *amax = (float)am;
  return true;
}

template <int CBK, int CBV>
static hipError_t run_mfma(const MfmaDecodeArgs& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_mfma_kernel<CBK, CBV, kMfmaWaves>), grid, dim3(kMfmaWaves * 64), 0, s, p);
  return hipGetLastError();
}

template <int CBK>
static hipError_t mfma_pick_v(int cbv, const MfmaDecodeArgs& p, dim3 grid, hipStream_t s) {
  switch (cbv) {
    case 1: return run_mfma<CBK, 1>(p, grid, s);
    case 2: return run_mfma<CBK, 2>(p, grid, s);
    case 3: return run_mfma<CBK, 3>(p, grid, s);
    case 4: return run_mfma<CBK, 4>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

bool decode_mfma_supported(const tq_codec& kc, const tq_codec& vc) {
  if (kc.d != kMD || vc.d != kMD || kc.m != kMD) return false;
  if (kc.code_bits < 1 || kc.code_bits > 4 || vc.code_bits < 1 || vc.code_bits > 4) return false;
  float alpha[8], amax;
  return mfma_key_alphas(kc.centroids, kc.code_bits, alpha, &amax);
}

hipError_t launch_decode_mfma(const tq_codec& kc, const tq_codec& vc, const void* q, int q_dtype,
                              int n_q, int hq, int hkv, const RopeHost& rope, const tq_packed& k,
                              const tq_packed& v, int64_t ctx, float scale, float* scores_out,
                              float* part, int nchunks, int splits, int64_t split_len, dim3 grid,
                              hipStream_t stream) {
  MfmaDecodeArgs p = {};
  p.q = q;
  p.q_f16 = q_dtype == TQ_F16;
  p.kidx = k.idx; p.kqjl = k.qjl; p.knorm = k.norm; p.krnorm = k.rnorm;
  p.vidx = v.idx; p.vnorm = v.norm;
  p.S = kc.S;
  p.scores_out = scores_out;
  p.part = part;
  p.ctx = ctx; p.hq = hq; p.hkv = hkv; p.n_q = n_q; p.G = hq / hkv;
  p.nchunks = nchunks; p.splits = splits; p.split_len = split_len;
  p.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)kMD));
  p.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / kc.m);
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)kMD));
  p.rope = rope.on ? 1 : 0;
  p.pos0 = rope.on ? rope.pos0 : 0;
  if (!mfma_key_alphas(kc.centroids, kc.code_bits, p.alpha, &p.alpha_max)) return hipErrorInvalidValue;
  p.ktop = kc.centroids[(1 << kc.code_bits) - 1];
  for (int i = 0; i < 16; ++i) p.vcent[i] = vc.centroids[i];
  for (int w = 0; w < 4; ++w) p.kflip[w] = kc.flip[w];
  if (rope.on)
    for (int i = 0; i < kMD / 2; ++i) p.theta[i] = std::pow((double)rope.base, -2.0 * i / (double)kMD);
  switch (kc.code_bits) {
    case 1: return mfma_pick_v<1>(vc.code_bits, p, grid, stream);
    case 2: return mfma_pick_v<2>(vc.code_bits, p, grid, stream);
    case 3: return mfma_pick_v<3>(vc.code_bits, p, grid, stream);
    case 4: return mfma_pick_v<4>(vc.code_bits, p, grid, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tqk
