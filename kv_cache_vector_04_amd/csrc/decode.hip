// Decode attention straight from packed codes, few query rows per KV head
// (GQA decode: the G query heads of one KV head at one position).
//
// "TurboESM", "2. Metodologia" part E (one pass: unpack, correct, attend
// with an online softmax, no dequantized copy); "Google presenta TurboQuant",
// "Eliminación del sesgo interno del producto" (the unbiased estimate):
//   s_j = scale nu_j ( <q_rot, c_K[idx_j]> + sqrt(pi/2)/m gamma_j <Sq, 2 sigma_j - 1> )
//   o   = Pi_V^T sum_j softmax(s)_j nu^V_j c_V[idx^V_j]
//
// decode_kernel: a workgroup (8 waves) owns one (batch, KV head), up to 4
// query rows of it and one token range.  Set-up, all in LDS: the query rows
// are rotated (q' = RoPE(q), q_rot = H (D_K q') / sqrt(d)), S is staged with
// a padded stride for Sq = S q_rot, and three lookup tables are built that
// replace per-coordinate multiplies in the scan:
//   LK[f][v] = sum over the gk coordinates of field f of q_rot[i] c_K[code_i]
//              (float4: the 4 rows), one entry per value v of a gk-code field;
//   LQ[p][v] = sum_{b : bit b of v} Sq[8p + b]  (float4), per QJL byte value;
//   LV[v]    = (c_V[v & mask], c_V[v >> CBV])  (float2), per pair of V codes.
// Scan: scores with one token per lane (d/gk + m/8 table reads, float4 adds);
// value sum with lane (cg, ts) owning coordinates 8cg..8cg+7 of tokens
// ts + TS t (32 accumulators: 8 coordinates x 4 rows), fed by softmax
// weights passed through LDS.  Running max per wave, running sums per lane.
// The next tile's codes are loaded while the current one is processed.
// The waves merge in LDS and the workgroup writes (acc, max, sum) per row.
// merge_kernel: per query row, log-sum-exp merge of the token ranges and
// o = D_V * H acc / sqrt(d), once per row (the rotation is linear).

#include <cmath>

#include "device_common.hpp"
#include "internal.hpp"

namespace tqk {

// Waves per workgroup: 12 (3 per SIMD).
template <int CBV>
struct DecWaves {
  static constexpr int kWaves = 12;
  static constexpr int kThreads = kWaves * kWave;
};
constexpr int kDecRows = 4;

struct DecodeParams {
  const void* q;          // [batch][hq][n_q][D]
  int q_f16;
  const uint8_t* kidx;
  const uint8_t* kqjl;
  const float* knorm;
  const float* krnorm;
  const uint8_t* vidx;
  const float* vnorm;
  const float* S;         // m x D row-major
  float* scores_out;      // optional [batch][hq][n_q][ctx]
  float* part;            // [bg][chunk][split][kDecRows][D + 2]
  int64_t ctx;
  int batch, hq, hkv, n_q, G, nchunks, splits;
  int64_t split_len;
  float scale;
  float qjl_scale;
  float inv_sqrt_d;
  int rope;
  int32_t pos0;
  float kcent[16];
  float vcent[16];
  uint32_t kflip[48];
  double theta[64];
};

template <int CB>
struct KGroup {
  // coordinates per K table field
  static constexpr int gk = CB == 1 ? 8 : (CB == 4 ? 1 : 2);
  static constexpr int bits = gk * CB;
  static constexpr int entries = 1 << bits;
};

template <int W>
__device__ __forceinline__ uint32_t field_bits(const uint32_t (&w)[W], int off, int nbits) {
  const int word = off >> 5, sh = off & 31;
  uint32_t v;
  if (sh + nbits <= 32) {
    v = w[word] >> sh;
  } else {
    v = __builtin_amdgcn_alignbit(w[word + 1], w[word], sh);
  }
  return nbits == 32 ? v : (v & ((1u << nbits) - 1u));
}

__device__ __forceinline__ float4 f4add(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

__device__ __forceinline__ float4 f4fma(float4 a, float s, float4 c) {
  return make_float4(fmaf(a.x, s, c.x), fmaf(a.y, s, c.y), fmaf(a.z, s, c.z), fmaf(a.w, s, c.w));
}

// Cross-lane moves inside each row of 16 lanes (DPP, no LDS traffic):
// quad xor 1, quad xor 2, half-row mirror, row mirror.  After the four steps
// every lane of a row holds the row's reduction; the four rows are combined
// through scalar reads of one lane each, so every lane gets the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

template <int D, int CBK, int CBV>
struct DecGeom {
  using KG = KGroup<CBK>;
  static constexpr int NF = D / KG::gk;          // K table fields per row
  static constexpr int NE = KG::entries;
  static constexpr int NB = D / 8;               // QJL bytes per row (m = D)
  static constexpr int WK = D * CBK / 32;
  static constexpr int KROW = D * CBK / 8;
  static constexpr int KALIGN = KROW % 16 == 0 ? 16 : 8;
  static constexpr int VW = D * CBV / 32;
  static constexpr int VROW = D * CBV / 8;
  static constexpr int NVE = 1 << (2 * CBV);
  static constexpr int CG = D / 8;               // 8-coordinate groups of a V row
  static constexpr int TS = kWave / CG;          // token subgroups per wave
  static constexpr int TPL = kWave / TS;         // tokens per lane per tile
  // LDS carve-up (bytes)
  static constexpr int LK_B = NF * NE * 16;
  static constexpr int LQ_B = NB * 256 * 16;
  static constexpr int kDecWaves = DecWaves<CBV>::kWaves;
  static constexpr int kDecThreads = DecWaves<CBV>::kThreads;
  static constexpr int MRG_B = kDecWaves * kDecRows * (D + 2) * 4;   // wave merge
  static constexpr int SQP_B = kDecThreads * 16;                      // Sq partials
  static constexpr int TAB0_B = (LK_B + LQ_B) > SQP_B ? (LK_B + LQ_B) : SQP_B;
  static constexpr int TAB_B = TAB0_B > MRG_B ? TAB0_B : MRG_B;
  static constexpr int LV_B = NVE * 8;
  static constexpr int W_B = kDecWaves * kWave * 16;
  static constexpr int NIB_B = NB * 2 * 16 * 16;  // nibble sums, set-up only
  static constexpr int WN_B = W_B > NIB_B ? W_B : NIB_B;
};

// One tile of a wave's token range: the key codes one lane needs.
template <int WK, int NB4>
struct TileRegs {
  uint32_t kw[WK];
  uint32_t sb[NB4];
  float nuk, gk, nuv;
};

template <int D, int CBK, int CBV>
__global__ __launch_bounds__(DecWaves<CBV>::kThreads) void decode_kernel(DecodeParams p) {
  constexpr int kDecWaves = DecWaves<CBV>::kWaves;
  constexpr int kDecThreads = DecWaves<CBV>::kThreads;
  using Gm = DecGeom<D, CBK, CBV>;
  using KG = typename Gm::KG;
  constexpr int NF = Gm::NF, NE = Gm::NE, NB = Gm::NB, WK = Gm::WK, KROW = Gm::KROW;
  constexpr int VW = Gm::VW, VROW = Gm::VROW, NVE = Gm::NVE, CG = Gm::CG, TS = Gm::TS;
  constexpr int TPL = Gm::TPL;
  static_assert(CG * TS == kWave, "lane layout");

  __shared__ __align__(16) unsigned char s_tab[Gm::TAB_B];   // LK | LQ  (Sq partials in set-up)
  __shared__ __align__(16) float2 s_lv[NVE];
  __shared__ __align__(16) unsigned char s_wn[Gm::WN_B];     // weights (nibble sums in set-up)
  __shared__ __align__(16) float4 s_qT[D];                    // q_rot, 4 rows per coordinate
  __shared__ __align__(16) float4 s_sT[D];                    // Sq, 4 rows per coordinate
  __shared__ float s_tot[kDecRows];
  __shared__ float s_kc[16], s_vc[16];
  // 3-bit value codes: the lane groups' 24 bits straddle words, so each
  // wave stages its tile's value rows here instead of holding two words per
  // token in registers
  // (where LDS allows: the 64 KB key table of 1- and 3-bit keys at d = 128
  // leaves no room, and those variants keep the two-word registers)
  constexpr bool VST = CBV == 3 && (D == 64 || CBK % 2 == 0);
  // the other 3-bit variants load their value words after the scores, four
  // tokens at a time (all sixteen tokens' two words through the scores
  // spill at this register budget)
  constexpr bool VCHUNK = CBV == 3 && !VST;
  constexpr int VSTR = VW + 1;
  __shared__ uint32_t s_vst[VST ? kDecWaves * kWave * VSTR : 1];

  float4* s_lk = reinterpret_cast<float4*>(s_tab);
  float4* s_lq = reinterpret_cast<float4*>(s_tab + Gm::LK_B);
  float4* s_w = reinterpret_cast<float4*>(s_wn);               // [wave][lane]
  float4* s_nib = reinterpret_cast<float4*>(s_wn);             // [byte][half][16]

  const int tid = threadIdx.x;
  // the wave index is uniform: scalar, so the token loop below is too
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int bgc = blockIdx.x;                    // (batch * hkv) * nchunks + chunk
  const int split = blockIdx.y;
  const int bg = bgc / p.nchunks, chunk = bgc % p.nchunks;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int qr_total = p.G * p.n_q;
  const int lr0 = chunk * kDecRows;
  const int nrows = (qr_total - lr0) < kDecRows ? (qr_total - lr0) : kDecRows;
  const int64_t row_base = ((int64_t)b * p.hq + (int64_t)g * p.G) * p.n_q + lr0;
  const int64_t t0 = (int64_t)split * p.split_len;
  int64_t t1 = t0 + p.split_len;
  if (t1 > p.ctx) t1 = p.ctx;
  const int64_t kv_base = (int64_t)bg * p.ctx;
  const int cg = lane % CG, ts = lane / CG;
  const int vbit0 = cg * 8 * CBV;
  const int vw0 = vbit0 >> 5;
  const int vw1 = (vw0 + 1) < VW ? (vw0 + 1) : (VW - 1);
  const bool vstraddle = (vbit0 & 31) + 8 * CBV > 32;

  auto load_tile = [&](int64_t tile, TileRegs<WK, NB / 4>& R) {
    const int64_t tok = tile + lane;
    const int64_t kr = kv_base + (tok < t1 ? tok : t0);
    load_words<WK, Gm::KALIGN>(p.kidx + kr * KROW, R.kw);
    load_words<NB / 4, (NB % 16 == 0) ? 16 : 8>(p.kqjl + kr * NB, R.sb);
    R.nuk = p.knorm[kr] * p.scale;
    R.gk = p.krnorm[kr] * p.qjl_scale;
    R.nuv = p.vnorm[kr];
  };

  // first tile's key codes in flight during the set-up
  TileRegs<WK, NB / 4> cur;
  const int64_t first = t0 + (int64_t)wave * kWave;
  if (first < t1) load_tile(first, cur);

  // ---- set-up ----
  // S rows for Sq, straight into registers: thread -> (coordinate i, k-part)
  constexpr int KP = (kDecThreads / D) >= 8 ? 8 : ((kDecThreads / D) >= 4 ? 4 : 2);  // k-parts
  constexpr int KL = D / KP;                      // k per part
  const int si = tid % D, spart = tid / D;
  const bool sq_thread = spart < KP;
  float4 srow[KL / 4];
  if (sq_thread) {
    const float4* S4 = reinterpret_cast<const float4*>(p.S + (size_t)si * D + spart * KL);
#pragma unroll
    for (int j = 0; j < KL / 4; ++j) srow[j] = S4[j];
  }
  const DecodeParams* kp = (const DecodeParams*)__builtin_amdgcn_kernarg_segment_ptr();
  if (tid < 16) {
    s_kc[tid] = kp->kcent[tid];
    s_vc[tid] = kp->vcent[tid];
  }
  // q' = RoPE(q), sign flip and the natural-order butterflies: wave r < 4
  // rotates query row r in registers, lane l holding coordinates C l + c
  // (C = d / 64): the stages on coordinate bits below log2 C stay in the
  // lane, the others exchange with lane l ^ 2^(bit - log2 C)
  constexpr int C = D / kWave;
  if (wave < kDecRows) {
    const int r = wave;
    float x[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int i = C * lane + c;
      float v = 0.f;
      if (r < nrows) {
        const int64_t off = (row_base + r) * D + i;
        v = p.q_f16 ? (float)reinterpret_cast<const _Float16*>(p.q)[off]
                    : reinterpret_cast<const float*>(p.q)[off];
      }
      x[c] = v;
    }
    if (p.rope) {
      // interleaved pairs (2 pr, 2 pr + 1) rotated by pos * theta_pr
      const int64_t pos = (int64_t)p.pos0 + ((lr0 + r) % p.n_q);
      if constexpr (C == 2) {
        float sn, cs;
        sincos_reduced((double)pos * kp->theta[lane], sn, cs);
        const float a = x[0], bb = x[1];
        x[0] = a * cs - bb * sn;
        x[1] = a * sn + bb * cs;
      } else {
        const int i = lane;
        float sn, cs;
        sincos_reduced((double)pos * kp->theta[i >> 1], sn, cs);
        const float o = __shfl_xor(x[0], 1);
        const float a = (i & 1) ? o : x[0], bb = (i & 1) ? x[0] : o;
        x[0] = (i & 1) ? (a * sn + bb * cs) : (a * cs - bb * sn);
      }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int i = C * lane + c;
      if ((kp->kflip[i >> 5] >> (i & 31)) & 1u) x[c] = -x[c];
    }
#pragma unroll
    for (int hb = 1; hb < C; hb <<= 1)
#pragma unroll
      for (int c = 0; c < C; ++c)
        if ((c & hb) == 0) {
          const float a = x[c], bb = x[c + hb];
          x[c] = a + bb;
          x[c + hb] = a - bb;
        }
#pragma unroll
    for (int lb = 1; lb < kWave; lb <<= 1) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float o = __shfl_xor(x[c], lb);
        x[c] = (lane & lb) ? (o - x[c]) : (x[c] + o);
      }
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
      reinterpret_cast<float*>(s_qT)[4 * (C * lane + c) + r] = x[c] * p.inv_sqrt_d;
  }
  __syncthreads();                                  // q_rot and the centroids in LDS
  // Sq partial sums over this thread's k-part (into the weight buffer, free
  // until the scan); the other threads build the key and value tables
  float4* s_sqp = reinterpret_cast<float4*>(s_wn);
  static_assert(KP * D * 16 <= Gm::WN_B, "Sq partials fit the weight buffer");
  if (sq_thread) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KL / 4; ++j) {
      const int k = spart * KL + 4 * j;
      a = f4fma(s_qT[k], srow[j].x, a);
      a = f4fma(s_qT[k + 1], srow[j].y, a);
      a = f4fma(s_qT[k + 2], srow[j].z, a);
      a = f4fma(s_qT[k + 3], srow[j].w, a);
    }
    s_sqp[spart * D + si] = a;
  }
  {
    // LK: lanes over table values, all threads (the Sq threads join after
    // their partial sums)
    for (int t = tid; t < NF * NE; t += kDecThreads) {
      const int v = t % NE, f = t / NE;
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int e = 0; e < KG::gk; ++e)
        a = f4fma(s_qT[f * KG::gk + e], s_kc[(v >> (e * CBK)) & ((1 << CBK) - 1)], a);
      s_lk[t] = a;
    }
  }
  for (int t = tid; t < NVE; t += kDecThreads)
    s_lv[t] = make_float2(s_vc[t & ((1 << CBV) - 1)], s_vc[t >> CBV]);
  __syncthreads();                                  // Sq partials, LK, LV
  if (tid < D) {
    float4 a = s_sqp[tid];
#pragma unroll
    for (int q = 1; q < KP; ++q) a = f4add(a, s_sqp[q * D + tid]);
    s_sT[tid] = a;
  }
  __syncthreads();                                  // Sq
  // tot[r] = sum_i Sq[r][i]: one wave per row
  if (wave < kDecRows) {
    float t = 0.f;
    for (int i = lane; i < D; i += kWave) t += reinterpret_cast<const float*>(s_sT)[4 * i + wave];
    t = wave_sum(t);
    if (lane == 0) s_tot[wave] = t;
  }
  // nibble sums of Sq for the QJL byte table: (byte pb, half h, nibble n)
  for (int t = tid; t < NB * 32; t += kDecThreads) {
    const int pb = t >> 5, h = (t >> 4) & 1, n = t & 15;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((n >> e) & 1) a = f4add(a, s_sT[8 * pb + 4 * h + e]);
    s_nib[t] = a;
  }
  __syncthreads();                                  // nibble sums, tot
  for (int t = tid; t < NB * 256; t += kDecThreads) {
    const int pb = t >> 8, v = t & 255;
    s_lq[t] = f4add(s_nib[pb * 32 + (v & 15)], s_nib[pb * 32 + 16 + (v >> 4)]);
  }
  __syncthreads();
  const float4 tot = make_float4(s_tot[0], s_tot[1], s_tot[2], s_tot[3]);

  // ---- scan of the token range ----
  float m_run[kDecRows], l_run[kDecRows];
  float acc[kDecRows][8];
#pragma unroll
  for (int r = 0; r < kDecRows; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }
  const float4* __restrict__ lk = s_lk;
  const float4* __restrict__ lq = s_lq;

  for (int64_t tile = first; tile < t1; tile += (int64_t)kDecWaves * kWave) {
    const TileRegs<WK, NB / 4> R = cur;
    const int64_t next = tile + (int64_t)kDecWaves * kWave;
    if (next < t1) load_tile(next, cur);
    const int64_t tok = tile + lane;
    const bool valid = tok < t1;
    // this tile's value codes (used after the scores)
    uint32_t vwr[VCHUNK ? 1 : TPL][2];
    uint32_t vrow[VST ? VW : 1];   // 3-bit codes: the lane's own token row, staged to LDS
    if constexpr (VST) {
      const int64_t vt = valid ? tok : t0;
      load_words<VW, (VROW % 16 == 0) ? 16 : 8>(p.vidx + (kv_base + vt) * VROW, vrow);
    } else if constexpr (!VCHUNK) {
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        int64_t vt = tile + (int64_t)u * TS + ts;
        vt = vt < t1 ? vt : t0;
        const uint32_t* vr = reinterpret_cast<const uint32_t*>(p.vidx + (kv_base + vt) * VROW);
        vwr[u][0] = vr[vw0];
        vwr[u][1] = vstraddle ? vr[vw1] : 0u;
      }
    }

    // four independent accumulation chains per table
    float4 msa[4] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f),
                     make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t v = field_bits<WK>(R.kw, f * KG::bits, KG::bits);
      msa[f & 3] = f4add(msa[f & 3], lk[f * NE + v]);
      // bound the table reads in flight (each holds 4 registers)
      if ((f & 15) == 15) __builtin_amdgcn_sched_barrier(0);
    }
    float4 qsa[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
    for (int pb = 0; pb < NB; ++pb) {
      const uint32_t v = (R.sb[pb >> 2] >> (8 * (pb & 3))) & 255u;
      qsa[pb & 1] = f4add(qsa[pb & 1], lq[pb * 256 + v]);
    }
    const float4 ms = f4add(f4add(msa[0], msa[1]), f4add(msa[2], msa[3]));
    const float4 qs = f4add(qsa[0], qsa[1]);
    float s[kDecRows];
    s[0] = R.nuk * fmaf(R.gk, 2.f * qs.x - tot.x, ms.x);
    s[1] = R.nuk * fmaf(R.gk, 2.f * qs.y - tot.y, ms.y);
    s[2] = R.nuk * fmaf(R.gk, 2.f * qs.z - tot.z, ms.z);
    s[3] = R.nuk * fmaf(R.gk, 2.f * qs.w - tot.w, ms.w);
    if (p.scores_out != nullptr && valid) {
#pragma unroll
      for (int r = 0; r < kDecRows; ++r)
        if (r < nrows) p.scores_out[(row_base + r) * p.ctx + tok] = s[r];
    }
    float pw[kDecRows];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
      const float sv = valid ? s[r] : -INFINITY;
      const float mt = wave_max(sv);
      const float mn = fmaxf(m_run[r], mt);
      const float alpha = __expf(m_run[r] - mn);
      m_run[r] = mn;
      const float e = valid ? __expf(sv - mn) : 0.f;
      l_run[r] = fmaf(l_run[r], alpha, e);
      pw[r] = e * R.nuv;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[r][k] *= alpha;
    }
    s_w[wave * kWave + lane] = make_float4(pw[0], pw[1], pw[2], pw[3]);
    if constexpr (VST) {
#pragma unroll
      for (int w = 0; w < VW; ++w) s_vst[(wave * kWave + lane) * VSTR + w] = vrow[w];
    }
    // LDS operations of one wave complete in order: the weights (and rows)
    // written above are visible to the reads below without a workgroup barrier.
    __builtin_amdgcn_wave_barrier();
    // weight of token u times the pair table entries of its four code pairs
    auto accum = [&](int u, uint32_t bits) {
      const float4 w = s_w[wave * kWave + u * TS + ts];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t pv = (bits >> (2 * CBV * e)) & (NVE - 1);
        const float2 c2 = s_lv[pv];
        acc[0][2 * e] = fmaf(w.x, c2.x, acc[0][2 * e]);
        acc[0][2 * e + 1] = fmaf(w.x, c2.y, acc[0][2 * e + 1]);
        acc[1][2 * e] = fmaf(w.y, c2.x, acc[1][2 * e]);
        acc[1][2 * e + 1] = fmaf(w.y, c2.y, acc[1][2 * e + 1]);
        acc[2][2 * e] = fmaf(w.z, c2.x, acc[2][2 * e]);
        acc[2][2 * e + 1] = fmaf(w.z, c2.y, acc[2][2 * e + 1]);
        acc[3][2 * e] = fmaf(w.w, c2.x, acc[3][2 * e]);
        acc[3][2 * e + 1] = fmaf(w.w, c2.y, acc[3][2 * e + 1]);
      }
    };
    if constexpr (VCHUNK) {
      constexpr int VC = 4;
      auto load_v = [&](int u0, uint32_t (&dst)[VC][2]) {
#pragma unroll
        for (int q = 0; q < VC; ++q) {
          int64_t vt = tile + (int64_t)(u0 + q) * TS + ts;
          vt = vt < t1 ? vt : t0;
          const uint32_t* vr = reinterpret_cast<const uint32_t*>(p.vidx + (kv_base + vt) * VROW);
          dst[q][0] = vr[vw0];
          dst[q][1] = vstraddle ? vr[vw1] : 0u;
        }
      };
      uint32_t vnext[VC][2];
      load_v(0, vnext);
#pragma unroll 1
      for (int c = 0; c < TPL / VC; ++c) {
        uint32_t vc4[VC][2];
#pragma unroll
        for (int q = 0; q < VC; ++q) {
          vc4[q][0] = vnext[q][0];
          vc4[q][1] = vnext[q][1];
        }
        if (c + 1 < TPL / VC) load_v((c + 1) * VC, vnext);
#pragma unroll
        for (int q = 0; q < VC; ++q)
          accum(c * VC + q, vstraddle ? __builtin_amdgcn_alignbit(vc4[q][1], vc4[q][0], vbit0 & 31)
                                      : (vc4[q][0] >> (vbit0 & 31)));
      }
    } else {
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        uint32_t bits;
        if constexpr (VST) {
          const uint32_t* vr = s_vst + (wave * kWave + u * TS + ts) * VSTR;
          bits = __builtin_amdgcn_alignbit(vr[vw1], vr[vw0], vbit0 & 31);
        } else {
          bits = vstraddle ? __builtin_amdgcn_alignbit(vwr[u][1], vwr[u][0], vbit0 & 31)
                           : (vwr[u][0] >> (vbit0 & 31));
        }
        accum(u, bits);
        if ((u & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the waves, write this range's (acc, max, sum) per row ----
#pragma unroll
  for (int r = 0; r < kDecRows; ++r) {
    l_run[r] = wave_sum(l_run[r]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma unroll
      for (int off = CG; off < kWave; off <<= 1) acc[r][k] += __shfl_xor(acc[r][k], off);
    }
  }
  __syncthreads();   // tables are no longer read: reuse them as merge space
  constexpr int REC = D + 2;
  float* mrg = reinterpret_cast<float*>(s_tab);   // [wave][row][D + 2]
  if (ts == 0) {
#pragma unroll
    for (int r = 0; r < kDecRows; ++r)
#pragma unroll
      for (int k = 0; k < 8; ++k) mrg[(wave * kDecRows + r) * REC + 8 * cg + k] = acc[r][k];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
      mrg[(wave * kDecRows + r) * REC + D] = m_run[r];
      mrg[(wave * kDecRows + r) * REC + D + 1] = l_run[r];
    }
  }
  __syncthreads();
  const int64_t rec0 = ((int64_t)bgc * p.splits + split) * kDecRows;
  for (int t = tid; t < kDecRows * D; t += kDecThreads) {
    const int r = t / D, i = t % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, mrg[(w * kDecRows + r) * REC + D]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = mrg[(w * kDecRows + r) * REC + D];
      const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
      a = fmaf(mrg[(w * kDecRows + r) * REC + i], f, a);
      L = fmaf(mrg[(w * kDecRows + r) * REC + D + 1], f, L);
    }
    float* rec = p.part + (rec0 + r) * REC;
    rec[i] = a;
    if (i == 0) {
      rec[D] = M;
      rec[D + 1] = L;
    }
  }
}

struct MergeParams {
  const float* part;
  float* out;
  int hq, hkv, n_q, G, nchunks, splits;
  int wht_len;            // d, or 64 for the two halves of a split codec
  float inv_sqrt_d;       // 1 / sqrt(wht_len)
  uint32_t vflip[48];
};

// Log-sum-exp merge of the token ranges of one query row, then
// o = D_V * (H a) / sqrt(d) (for a split codec H is H_64 on each half).
// Thread i owns coordinate i.  A pass over kMergeBatch records issues all of
// its loads before it waits (one memory round trip): each thread's value of
// every record, and in lane u of each wave the (max, sum) pair of record u,
// whose weight the other lanes then read from that lane.  The butterflies
// run inside the wave (DPP and lane swaps); only the stage across the two
// waves of d = 128 goes through LDS.
constexpr int kMergeBatch = 32;

// One butterfly stage of stride hh < 64 inside the wave: the lane with
// bit hh of its index clear keeps x + x', the other x' - x (x' the
// partner's value, the partner's index lower).
__device__ __forceinline__ float wave_butterfly(float x, int lane, int hh) {
  switch (hh) {
    case 1: {
      const float o = dpp_f<0xB1>(x);            // quad_perm [1, 0, 3, 2]
      return (lane & 1) ? (o - x) : (x + o);
    }
    case 2: {
      const float o = dpp_f<0x4E>(x);            // quad_perm [2, 3, 0, 1]
      return (lane & 2) ? (o - x) : (x + o);
    }
    case 4: {
      // row_ror 4 reads lane l - 4 of the row, row_ror 12 lane l + 4
      const float lo = dpp_f<0x124>(x), hi = dpp_f<0x12C>(x);
      return (lane & 4) ? (lo - x) : (x + hi);
    }
    case 8: {
      const float o = dpp_f<0x128>(x);           // row_ror 8: lane l ^ 8
      return (lane & 8) ? (o - x) : (x + o);
    }
    case 16: {
      // [0]: the value of the lower row of the pair, [1]: of the upper row
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
      return (lane & 16) ? (a - b) : (a + b);
    }
    default: {
      // [0]: the value of the lower half, [1]: of the upper half
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
      const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
      return (lane & 32) ? (a - b) : (a + b);
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void merge_kernel(MergeParams p) {
  constexpr int REC = D + 2;
  constexpr int NB = kMergeBatch;
  __shared__ float s_v[D];
  const int i = threadIdx.x, lane = i & 63;
  const int64_t row = blockIdx.x;                 // (b, h, a)
  const int a = (int)(row % p.n_q);
  const int64_t bh = row / p.n_q;
  const int h = (int)(bh % p.hq);
  const int b = (int)(bh / p.hq);
  const int g = h / p.G;
  const int lr = (h - g * p.G) * p.n_q + a;
  const int chunk = lr / kDecRows, r = lr % kDecRows;
  const int64_t bgc = ((int64_t)b * p.hkv + g) * p.nchunks + chunk;
  const float* base = p.part + (bgc * p.splits * kDecRows + r) * REC;
  const int64_t stride = (int64_t)kDecRows * REC;
  float M = -INFINITY, L = 0.f, v = 0.f;
  for (int s0 = 0; s0 < p.splits; s0 += NB) {
    const int ns = (p.splits - s0) < NB ? (p.splits - s0) : NB;
    // records past the last one re-read the last (and are weighted 0)
    float x[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) x[u] = base[(int64_t)(s0 + (u < ns ? u : ns - 1)) * stride + i];
    const float* mine = base + (int64_t)(s0 + (lane < ns ? lane : ns - 1)) * stride;
    float mu = mine[D], lu = mine[D + 1];
    if (lane >= ns) {
      mu = -INFINITY;
      lu = 0.f;
    }
    const float Mc = fmaxf(M, wave_max(mu));
    const float f = mu == -INFINITY ? 0.f : __expf(mu - Mc);
    const float rescale = M == -INFINITY ? 0.f : __expf(M - Mc);
    L = fmaf(L, rescale, wave_sum(lu * f));
    v *= rescale;
#pragma unroll
    for (int u = 0; u < NB; ++u)
      v = fmaf(x[u], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), u)), v);
    M = Mc;
  }
  v /= L;
#pragma unroll
  for (int hh = 1; hh < (D < 64 ? D : 64); hh <<= 1)
    if (hh < p.wht_len) v = wave_butterfly(v, lane, hh);
  if (D == 128 && p.wht_len == 128) {
    s_v[i] = v;
    __syncthreads();
    const float o = s_v[i ^ 64];
    v = (i & 64) ? (o - v) : (v + o);
  }
  const uint32_t bit = (p.vflip[i >> 5] >> (i & 31)) & 1u;
  v *= p.inv_sqrt_d;
  p.out[row * D + i] = bit ? -v : v;
}

// ---------------------------------------------------------------------------

static void plan_decode(int batch, int n_q, int hq, int hkv, int64_t ctx, int& nchunks,
                        int& splits, int64_t& split_len) {
  const int G = hq / hkv;
  nchunks = (G * n_q + kDecRows - 1) / kDecRows;
  const int64_t groups = (int64_t)batch * hkv * nchunks;
  const int64_t tiles = (ctx + kWave - 1) / kWave;
  const int cus = device_cu_count();
  int64_t want = (cus + groups - 1) / groups;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  split_len = ((ctx + want - 1) / want + kWave - 1) / kWave * kWave;
  splits = (int)((ctx + split_len - 1) / split_len);
}

bool decode_path(int n_q, int hq, int hkv) {
  return (hq / hkv) * n_q <= 16;
}

size_t decode_workspace_bytes(int batch, int n_q, int hq, int hkv, int64_t ctx, int d) {
  int nchunks, splits;
  int64_t split_len;
  plan_decode(batch, n_q, hq, hkv, ctx, nchunks, splits, split_len);
  const size_t groups = (size_t)batch * hkv * nchunks;
  return groups * splits * kDecRows * (d + 2) * sizeof(float);
}

template <int D, int CBK, int CBV>
static hipError_t run_decode(const DecodeParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<D, CBK, CBV>), grid, dim3(DecWaves<CBV>::kThreads), 0, s, p);
  return hipGetLastError();
}

template <int D, int CBK>
static hipError_t dec_pick_v(int cbv, const DecodeParams& p, dim3 grid, hipStream_t s) {
  switch (cbv) {
    case 1: return run_decode<D, CBK, 1>(p, grid, s);
    case 2: return run_decode<D, CBK, 2>(p, grid, s);
    case 3: return run_decode<D, CBK, 3>(p, grid, s);
    case 4: return run_decode<D, CBK, 4>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t dec_pick_k(int cbk, int cbv, const DecodeParams& p, dim3 grid, hipStream_t s) {
  switch (cbk) {
    case 1: return dec_pick_v<D, 1>(cbv, p, grid, s);
    case 2: return dec_pick_v<D, 2>(cbv, p, grid, s);
    case 3: return dec_pick_v<D, 3>(cbv, p, grid, s);
    case 4: return dec_pick_v<D, 4>(cbv, p, grid, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const tq_codec& kc, const tq_codec& vc, const void* q, int q_dtype,
                         int batch, int n_q, int hq, int hkv, const RopeHost& rope,
                         const tq_packed& k, const tq_packed& v, int64_t ctx, float scale,
                         float* out, float* scores_out, void* workspace, hipStream_t stream) {
  const int d = kc.d;
  int nchunks, splits;
  int64_t split_len;
  plan_decode(batch, n_q, hq, hkv, ctx, nchunks, splits, split_len);
  const size_t groups = (size_t)batch * hkv * nchunks;
  DecodeParams p = {};
  p.q = q;
  p.q_f16 = q_dtype == TQ_F16;
  p.kidx = k.idx; p.kqjl = k.qjl; p.knorm = k.norm; p.krnorm = k.rnorm;
  p.vidx = v.idx; p.vnorm = v.norm;
  p.S = kc.S;
  p.scores_out = scores_out;
  p.part = reinterpret_cast<float*>(workspace);
  p.ctx = ctx; p.batch = batch; p.hq = hq; p.hkv = hkv; p.n_q = n_q; p.G = hq / hkv;
  p.nchunks = nchunks; p.splits = splits; p.split_len = split_len;
  p.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)d));
  p.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / kc.m);
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)d));
  p.rope = rope.on ? 1 : 0;
  p.pos0 = rope.on ? rope.pos0 : 0;
  for (int i = 0; i < 16; ++i) { p.kcent[i] = kc.centroids[i]; p.vcent[i] = vc.centroids[i]; }
  for (int w = 0; w < 48; ++w) p.kflip[w] = kc.flip[w];
  if (rope.on)
    for (int i = 0; i < d / 2 && i < 64; ++i)
      p.theta[i] = std::pow((double)rope.base, -2.0 * i / (double)d);
  const dim3 grid((unsigned)groups, (unsigned)splits);
  hipError_t e;
  if (d == 128 && decode_mfma_supported(kc, vc))
    e = launch_decode_mfma(kc, vc, q, q_dtype, n_q, hq, hkv, rope, k, v, ctx, scale, scores_out,
                           p.part, nchunks, splits, split_len, grid, stream);
  else if (d == 128) e = dec_pick_k<128>(kc.code_bits, vc.code_bits, p, grid, stream);
  else if (d == 64) e = dec_pick_k<64>(kc.code_bits, vc.code_bits, p, grid, stream);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  MergeParams mp = {};
  mp.part = p.part;
  mp.out = out;
  mp.hq = hq; mp.hkv = hkv; mp.n_q = n_q; mp.G = hq / hkv; mp.nchunks = nchunks;
  mp.splits = splits;
  mp.wht_len = d;
  mp.inv_sqrt_d = p.inv_sqrt_d;
  for (int w = 0; w < 48; ++w) mp.vflip[w] = vc.flip[w];
  const unsigned rows = (unsigned)((int64_t)batch * hq * n_q);
  if (d == 128)
    hipLaunchKernelGGL((merge_kernel<128>), dim3(rows), dim3(128), 0, stream, mp);
  else
    hipLaunchKernelGGL((merge_kernel<64>), dim3(rows), dim3(64), 0, stream, mp);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Attention from outlier-split codes.  Keys and values are each two d = 64
// codecs over the channel halves [0, 64) (hi) and [64, 128) (lo), so with
// q_h the query's half h:
//   s_j = scale sum_h nu_hj ( <Pi_h q_h, c_Kh[idx_hj]> +
//                             sqrt(pi/2)/64 gamma_hj <S_h Pi_h q_h, 2 sigma_hj - 1> )
//   o_h = Pi_Vh^T sum_j softmax(s)_j nu^V_hj c_Vh[idx^V_hj]
// The layout of decode_kernel, with: the query rotation stopped before the
// butterfly stage across the halves (H_64 on each half, per-half flips,
// 1/8); S block-diagonal; one key table per half at its own width; the QJL
// byte table over the 16 bytes of the two halves (8 each) summed per half;
// two weights per token (one per half's value norm); lanes 0..7 of each
// 16-lane group accumulate hi coordinates, 8..15 lo ones, at their half's
// code width.  The merge kernel applies H_64 per half.

struct DecodeSplitParams {
  const void* q;
  int q_f16;
  const uint8_t* kidx[2];
  const uint8_t* kqjl[2];
  const float* knorm[2];
  const float* krnorm[2];
  const uint8_t* vidx[2];
  const float* vnorm[2];
  const float* S[2];           // 64 x 64 row-major per half
  float* scores_out;
  float* part;
  int64_t ctx;
  int batch, hq, hkv, n_q, G, nchunks, splits;
  int64_t split_len;
  float scale;
  float qjl_scale;             // sqrt(pi/2) / 64
  float kcent[2][16];
  float vcent[2][16];
  uint32_t kflip[4];           // bit i: channel i (hi 0..63, lo 64..127)
};

template <int CBKH, int CBKL, int CBVH, int CBVL>
struct SplitGeom {
  using KH = KGroup<CBKH>;
  using KL = KGroup<CBKL>;
  static constexpr int D = 128, HD = 64;
  static constexpr int NFH = HD / KH::gk, NFL = HD / KL::gk;
  static constexpr int NEH = KH::entries, NEL = KL::entries;
  static constexpr int WKH = HD * CBKH / 32, WKL = HD * CBKL / 32;
  static constexpr int KROWH = HD * CBKH / 8, KROWL = HD * CBKL / 8;
  static constexpr int NB = 16;                  // QJL bytes per token, 8 per half
  static constexpr int VROWH = HD * CBVH / 8, VROWL = HD * CBVL / 8;
  static constexpr int NVEH = 1 << (2 * CBVH), NVEL = 1 << (2 * CBVL);
  static constexpr int CG = D / 8, TS = kWave / CG, TPL = kWave / TS;
  // 8 waves (2 per SIMD): the two halves' tables, sums and weights need
  // more than the 168 registers of 3 waves per SIMD
  static constexpr int kWaves = 8, kThreads = kWaves * kWave;
  static constexpr int LKH_B = NFH * NEH * 16, LKL_B = NFL * NEL * 16;
  static constexpr int LQ_B = NB * 256 * 16;
  static constexpr int MRG_B = kWaves * kDecRows * (D + 2) * 4;
  static constexpr int TAB0_B = LKH_B + LKL_B + LQ_B;
  static constexpr int TAB_B = TAB0_B > MRG_B ? TAB0_B : MRG_B;
  static constexpr int KP = 4;                   // S column parts per half
  static constexpr int W_B = kWaves * kWave * 2 * 16;
  static constexpr int NIB_B = NB * 2 * 16 * 16;
  static constexpr int SQP_B = KP * D * 16;
  static constexpr int WN0_B = W_B > NIB_B ? W_B : NIB_B;
  static constexpr int WN_B = WN0_B > SQP_B ? WN0_B : SQP_B;
};

template <int CBKH, int CBKL>
struct SplitTile {
  uint32_t kh[SplitGeom<CBKH, CBKL, 2, 2>::WKH];
  uint32_t kl[SplitGeom<CBKH, CBKL, 2, 2>::WKL];
  uint32_t sb[4];
  float nkh, nkl, gh, gl, nvh, nvl;
};

constexpr int kSplitThreads = 8 * kWave;

template <int CBKH, int CBKL, int CBVH, int CBVL>
__global__ __launch_bounds__(kSplitThreads) void decode_split_kernel(DecodeSplitParams p) {
  using Gm = SplitGeom<CBKH, CBKL, CBVH, CBVL>;
  static_assert(Gm::kThreads == kSplitThreads, "launch bounds");
  using KH = typename Gm::KH;
  using KL = typename Gm::KL;
  constexpr int D = Gm::D, HD = Gm::HD, kW = Gm::kWaves, kT = Gm::kThreads;
  constexpr int NFH = Gm::NFH, NFL = Gm::NFL, NEH = Gm::NEH, NEL = Gm::NEL, NB = Gm::NB;
  constexpr int CG = Gm::CG, TS = Gm::TS, TPL = Gm::TPL;

  __shared__ __align__(16) unsigned char s_tab[Gm::TAB_B];   // LK hi | LK lo | LQ
  __shared__ __align__(16) float2 s_lv[Gm::NVEH + Gm::NVEL];
  __shared__ __align__(16) unsigned char s_wn[Gm::WN_B];     // weights / set-up scratch
  __shared__ __align__(16) float4 s_qT[D];
  __shared__ __align__(16) float4 s_sT[D];
  __shared__ float s_tot[2][kDecRows];
  __shared__ float s_kc[2][16], s_vc[2][16];

  float4* s_lkh = reinterpret_cast<float4*>(s_tab);
  float4* s_lkl = reinterpret_cast<float4*>(s_tab + Gm::LKH_B);
  float4* s_lq = reinterpret_cast<float4*>(s_tab + Gm::LKH_B + Gm::LKL_B);
  float4* s_w = reinterpret_cast<float4*>(s_wn);               // [wave][lane][half]
  float4* s_nib = reinterpret_cast<float4*>(s_wn);

  const int tid = threadIdx.x;
  // the wave index is uniform: scalar, so the token loop below is too
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int bgc = blockIdx.x;
  const int split = blockIdx.y;
  const int bg = bgc / p.nchunks, chunk = bgc % p.nchunks;
  const int b = bg / p.hkv, g = bg % p.hkv;
  const int qr_total = p.G * p.n_q;
  const int lr0 = chunk * kDecRows;
  const int nrows = (qr_total - lr0) < kDecRows ? (qr_total - lr0) : kDecRows;
  const int64_t row_base = ((int64_t)b * p.hq + (int64_t)g * p.G) * p.n_q + lr0;
  const int64_t t0 = (int64_t)split * p.split_len;
  int64_t t1 = t0 + p.split_len;
  if (t1 > p.ctx) t1 = p.ctx;
  const int64_t kv_base = (int64_t)bg * p.ctx;
  // value lanes: 8-coordinate group cg of the row, half vh, its code width
  const int cg = lane % CG, ts = lane / CG;
  const int vh = cg >> 3, cgl = cg & 7;
  const int cbv = vh ? CBVL : CBVH;
  const int vbit0 = cgl * 8 * cbv;
  const int vw0 = vbit0 >> 5;
  const int vwords = 2 * cbv;
  const int vw1 = (vw0 + 1) < vwords ? (vw0 + 1) : (vwords - 1);
  const bool vstraddle = (vbit0 & 31) + 8 * cbv > 32;
  const uint32_t vrow = vh ? Gm::VROWL : Gm::VROWH;
  // the lane's value plane from this range's first token: one 64-bit base,
  // then 32-bit offsets (a range is under 2^26 tokens of at most 32 bytes)
  const uint32_t* vbase =
      reinterpret_cast<const uint32_t*>((vh ? p.vidx[1] : p.vidx[0]) + (kv_base + t0) * vrow) + vw0;
  const int lvoff = vh ? Gm::NVEH : 0;
  const uint32_t vmask = (1u << (2 * cbv)) - 1u;

  // the ten planes of the key side from this range's first token (uniform
  // bases), addressed with one 32-bit token offset per lane
  const int64_t rb = kv_base + t0;
  const uint8_t* const kih = p.kidx[0] + rb * Gm::KROWH;
  const uint8_t* const kil = p.kidx[1] + rb * Gm::KROWL;
  const uint2* const kqh = reinterpret_cast<const uint2*>(p.kqjl[0] + rb * 8);
  const uint2* const kql = reinterpret_cast<const uint2*>(p.kqjl[1] + rb * 8);
  const float* const nkh = p.knorm[0] + rb;
  const float* const nkl = p.knorm[1] + rb;
  const float* const gkh = p.krnorm[0] + rb;
  const float* const gkl = p.krnorm[1] + rb;
  const float* const nvh = p.vnorm[0] + rb;
  const float* const nvl = p.vnorm[1] + rb;
  auto load_tile = [&](int64_t tile, SplitTile<CBKH, CBKL>& R) {
    const int64_t tok = tile + lane;
    const uint32_t rel = tok < t1 ? (uint32_t)(tok - t0) : 0u;
    load_words<Gm::WKH, (Gm::KROWH % 16 == 0) ? 16 : 8>(kih + rel * Gm::KROWH, R.kh);
    load_words<Gm::WKL, (Gm::KROWL % 16 == 0) ? 16 : 8>(kil + rel * Gm::KROWL, R.kl);
    const uint2 sh = kqh[rel];
    const uint2 sl = kql[rel];
    R.sb[0] = sh.x; R.sb[1] = sh.y; R.sb[2] = sl.x; R.sb[3] = sl.y;
    R.nkh = nkh[rel] * p.scale;
    R.nkl = nkl[rel] * p.scale;
    R.gh = gkh[rel] * p.qjl_scale;
    R.gl = gkl[rel] * p.qjl_scale;
    R.nvh = nvh[rel];
    R.nvl = nvl[rel];
  };

  SplitTile<CBKH, CBKL> cur;
  const int64_t first = t0 + (int64_t)wave * kWave;
  if (first < t1) load_tile(first, cur);

  // ---- set-up ----
  // S rows for Sq: thread -> (row si, column part spart of si's half)
  constexpr int KP = Gm::KP, KLN = HD / KP;
  const int si = tid % D, spart = tid / D;
  const bool sq_thread = spart < KP;
  const int sh_half = si / HD;
  float4 srow[KLN / 4];
  if (sq_thread) {
    const float4* S4 = reinterpret_cast<const float4*>(p.S[sh_half] + (size_t)(si % HD) * HD + spart * KLN);
#pragma unroll
    for (int j = 0; j < KLN / 4; ++j) srow[j] = S4[j];
  }
  const DecodeSplitParams* kp = (const DecodeSplitParams*)__builtin_amdgcn_kernarg_segment_ptr();
  if (tid < 32) {
    s_kc[tid >> 4][tid & 15] = kp->kcent[tid >> 4][tid & 15];
    s_vc[tid >> 4][tid & 15] = kp->vcent[tid >> 4][tid & 15];
  }
  // q_h -> H_64 (D_h q_h) / 8: wave r < 4 rotates query row r, lane l holding
  // channels 2 l, 2 l + 1 (lanes 0..31 the hi half); the lane-exchange
  // stages stop below 32, the stage that would mix the halves
  if (wave < kDecRows) {
    const int r = wave;
    float x[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = 2 * lane + c;
      float v = 0.f;
      if (r < nrows) {
        const int64_t off = (row_base + r) * D + i;
        v = p.q_f16 ? (float)reinterpret_cast<const _Float16*>(p.q)[off]
                    : reinterpret_cast<const float*>(p.q)[off];
      }
      x[c] = ((kp->kflip[i >> 5] >> (i & 31)) & 1u) ? -v : v;
    }
    {
      const float a = x[0], bb = x[1];
      x[0] = a + bb;
      x[1] = a - bb;
    }
#pragma unroll
    for (int lb = 1; lb < kWave / 2; lb <<= 1) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float o = __shfl_xor(x[c], lb);
        x[c] = (lane & lb) ? (o - x[c]) : (x[c] + o);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) reinterpret_cast<float*>(s_qT)[4 * (2 * lane + c) + r] = x[c] * 0.125f;
  }
  __syncthreads();                                  // q_rot and the centroids
  float4* s_sqp = reinterpret_cast<float4*>(s_wn);
  if (sq_thread) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KLN / 4; ++j) {
      const int k = sh_half * HD + spart * KLN + 4 * j;
      a = f4fma(s_qT[k], srow[j].x, a);
      a = f4fma(s_qT[k + 1], srow[j].y, a);
      a = f4fma(s_qT[k + 2], srow[j].z, a);
      a = f4fma(s_qT[k + 3], srow[j].w, a);
    }
    s_sqp[spart * D + si] = a;
  }
  for (int t = tid; t < NFH * NEH; t += kT) {
    const int v = t % NEH, f = t / NEH;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int e = 0; e < KH::gk; ++e)
      a = f4fma(s_qT[f * KH::gk + e], s_kc[0][(v >> (e * CBKH)) & ((1 << CBKH) - 1)], a);
    s_lkh[t] = a;
  }
  for (int t = tid; t < NFL * NEL; t += kT) {
    const int v = t % NEL, f = t / NEL;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int e = 0; e < KL::gk; ++e)
      a = f4fma(s_qT[HD + f * KL::gk + e], s_kc[1][(v >> (e * CBKL)) & ((1 << CBKL) - 1)], a);
    s_lkl[t] = a;
  }
  for (int t = tid; t < Gm::NVEH; t += kT)
    s_lv[t] = make_float2(s_vc[0][t & ((1 << CBVH) - 1)], s_vc[0][t >> CBVH]);
  for (int t = tid; t < Gm::NVEL; t += kT)
    s_lv[Gm::NVEH + t] = make_float2(s_vc[1][t & ((1 << CBVL) - 1)], s_vc[1][t >> CBVL]);
  __syncthreads();                                  // Sq partials, LK, LV
  if (tid < D) {
    float4 a = s_sqp[tid];
#pragma unroll
    for (int q = 1; q < KP; ++q) a = f4add(a, s_sqp[q * D + tid]);
    s_sT[tid] = a;
  }
  __syncthreads();                                  // Sq
  // tot[h][r] = sum over half h of Sq[r][i]: wave r, one half after the other
  if (wave < kDecRows) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float t = wave_sum(reinterpret_cast<const float*>(s_sT)[4 * (h * HD + lane) + wave]);
      if (lane == 0) s_tot[h][wave] = t;
    }
  }
  for (int t = tid; t < NB * 32; t += kT) {
    const int pb = t >> 5, h = (t >> 4) & 1, n = t & 15;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((n >> e) & 1) a = f4add(a, s_sT[8 * pb + 4 * h + e]);
    s_nib[t] = a;
  }
  __syncthreads();                                  // nibble sums, tot
  for (int t = tid; t < NB * 256; t += kT) {
    const int pb = t >> 8, v = t & 255;
    s_lq[t] = f4add(s_nib[pb * 32 + (v & 15)], s_nib[pb * 32 + 16 + (v >> 4)]);
  }
  __syncthreads();
  const float4 toth = make_float4(s_tot[0][0], s_tot[0][1], s_tot[0][2], s_tot[0][3]);
  const float4 totl = make_float4(s_tot[1][0], s_tot[1][1], s_tot[1][2], s_tot[1][3]);

  // ---- scan ----
  float m_run[kDecRows], l_run[kDecRows];
  float acc[kDecRows][8];
#pragma unroll
  for (int r = 0; r < kDecRows; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }
  const float4* __restrict__ lkh = s_lkh;
  const float4* __restrict__ lkl = s_lkl;
  const float4* __restrict__ lq = s_lq;

  for (int64_t tile = first; tile < t1; tile += (int64_t)kW * kWave) {
    const SplitTile<CBKH, CBKL> R = cur;
    const int64_t next = tile + (int64_t)kW * kWave;
    if (next < t1) load_tile(next, cur);
    const int64_t tok = tile + lane;
    const bool valid = tok < t1;
    float4 mh[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    float4 ml[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
    for (int f = 0; f < NFH; ++f) {
      const uint32_t v = field_bits<Gm::WKH>(R.kh, f * KH::bits, KH::bits);
      mh[f & 1] = f4add(mh[f & 1], lkh[f * NEH + v]);
      // bound the table reads in flight (each holds 4 registers)
      if ((f & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < NFL; ++f) {
      const uint32_t v = field_bits<Gm::WKL>(R.kl, f * KL::bits, KL::bits);
      ml[f & 1] = f4add(ml[f & 1], lkl[f * NEL + v]);
      if ((f & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    float4 qh = make_float4(0.f, 0.f, 0.f, 0.f), ql = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int pb = 0; pb < NB; ++pb) {
      const uint32_t v = (R.sb[pb >> 2] >> (8 * (pb & 3))) & 255u;
      if (pb < NB / 2) qh = f4add(qh, lq[pb * 256 + v]);
      else ql = f4add(ql, lq[pb * 256 + v]);
      if ((pb & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    const float4 msh = f4add(mh[0], mh[1]), msl = f4add(ml[0], ml[1]);
    float s[kDecRows];
    s[0] = R.nkh * fmaf(R.gh, 2.f * qh.x - toth.x, msh.x) + R.nkl * fmaf(R.gl, 2.f * ql.x - totl.x, msl.x);
    s[1] = R.nkh * fmaf(R.gh, 2.f * qh.y - toth.y, msh.y) + R.nkl * fmaf(R.gl, 2.f * ql.y - totl.y, msl.y);
    s[2] = R.nkh * fmaf(R.gh, 2.f * qh.z - toth.z, msh.z) + R.nkl * fmaf(R.gl, 2.f * ql.z - totl.z, msl.z);
    s[3] = R.nkh * fmaf(R.gh, 2.f * qh.w - toth.w, msh.w) + R.nkl * fmaf(R.gl, 2.f * ql.w - totl.w, msl.w);
    if (p.scores_out != nullptr && valid) {
#pragma unroll
      for (int r = 0; r < kDecRows; ++r)
        if (r < nrows) p.scores_out[(row_base + r) * p.ctx + tok] = s[r];
    }
    // this tile's value codes, four tokens at a time: the next four load
    // while the current four accumulate (the split's two widths leave no
    // room to hold all sixteen through the scores)
    constexpr int VC = 4;
    const uint32_t trel = (uint32_t)(tile - t0) + (uint32_t)ts, tlast = (uint32_t)(t1 - 1 - t0);
    auto load_v = [&](int u0, uint32_t (&dst)[VC][2]) {
#pragma unroll
      for (int q = 0; q < VC; ++q) {
        uint32_t vt = trel + (uint32_t)((u0 + q) * TS);
        vt = vt <= tlast ? vt : 0u;
        const uint32_t* vr = vbase + vt * (vrow >> 2);
        dst[q][0] = vr[0];
        dst[q][1] = vstraddle ? vr[vw1 - vw0] : 0u;
      }
    };
    uint32_t vnext[VC][2];
    load_v(0, vnext);
    float pe[kDecRows];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
      const float sv = valid ? s[r] : -INFINITY;
      const float mt = wave_max(sv);
      const float mn = fmaxf(m_run[r], mt);
      const float alpha = __expf(m_run[r] - mn);
      m_run[r] = mn;
      const float e = valid ? __expf(sv - mn) : 0.f;
      l_run[r] = fmaf(l_run[r], alpha, e);
      pe[r] = e;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[r][k] *= alpha;
    }
    s_w[(wave * kWave + lane) * 2] =
        make_float4(pe[0] * R.nvh, pe[1] * R.nvh, pe[2] * R.nvh, pe[3] * R.nvh);
    s_w[(wave * kWave + lane) * 2 + 1] =
        make_float4(pe[0] * R.nvl, pe[1] * R.nvl, pe[2] * R.nvl, pe[3] * R.nvl);
    // LDS operations of one wave complete in order: no workgroup barrier
    __builtin_amdgcn_wave_barrier();
    // chunks of VC tokens, not unrolled: an unrolled loop over all sixteen
    // tokens spills (the table reads of every token get hoisted)
#pragma unroll 1
    for (int c = 0; c < TPL / VC; ++c) {
      uint32_t vc4[VC][2];
#pragma unroll
      for (int q = 0; q < VC; ++q) { vc4[q][0] = vnext[q][0]; vc4[q][1] = vnext[q][1]; }
      if (c + 1 < TPL / VC) load_v((c + 1) * VC, vnext);
#pragma unroll
      for (int q = 0; q < VC; ++q) {
        const int u = c * VC + q;
        const float4 w = s_w[(wave * kWave + u * TS + ts) * 2 + vh];
        const uint32_t bits = vstraddle ? __builtin_amdgcn_alignbit(vc4[q][1], vc4[q][0], vbit0 & 31)
                                        : (vc4[q][0] >> (vbit0 & 31));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t pv = (bits >> (2 * cbv * e)) & vmask;
          const float2 c2 = s_lv[lvoff + pv];
          acc[0][2 * e] = fmaf(w.x, c2.x, acc[0][2 * e]);
          acc[0][2 * e + 1] = fmaf(w.x, c2.y, acc[0][2 * e + 1]);
          acc[1][2 * e] = fmaf(w.y, c2.x, acc[1][2 * e]);
          acc[1][2 * e + 1] = fmaf(w.y, c2.y, acc[1][2 * e + 1]);
          acc[2][2 * e] = fmaf(w.z, c2.x, acc[2][2 * e]);
          acc[2][2 * e + 1] = fmaf(w.z, c2.y, acc[2][2 * e + 1]);
          acc[3][2 * e] = fmaf(w.w, c2.x, acc[3][2 * e]);
          acc[3][2 * e + 1] = fmaf(w.w, c2.y, acc[3][2 * e + 1]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the waves, write this range's (acc, max, sum) per row ----
#pragma unroll
  for (int r = 0; r < kDecRows; ++r) {
    l_run[r] = wave_sum(l_run[r]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma unroll
      for (int off = CG; off < kWave; off <<= 1) acc[r][k] += __shfl_xor(acc[r][k], off);
    }
  }
  __syncthreads();
  constexpr int REC = D + 2;
  float* mrg = reinterpret_cast<float*>(s_tab);
  if (ts == 0) {
#pragma unroll
    for (int r = 0; r < kDecRows; ++r)
#pragma unroll
      for (int k = 0; k < 8; ++k) mrg[(wave * kDecRows + r) * REC + 8 * cg + k] = acc[r][k];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
      mrg[(wave * kDecRows + r) * REC + D] = m_run[r];
      mrg[(wave * kDecRows + r) * REC + D + 1] = l_run[r];
    }
  }
  __syncthreads();
  const int64_t rec0 = ((int64_t)bgc * p.splits + split) * kDecRows;
  for (int t = tid; t < kDecRows * D; t += kT) {
    const int r = t / D, i = t % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, mrg[(w * kDecRows + r) * REC + D]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float mw = mrg[(w * kDecRows + r) * REC + D];
      const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
      a = fmaf(mrg[(w * kDecRows + r) * REC + i], f, a);
      L = fmaf(mrg[(w * kDecRows + r) * REC + D + 1], f, L);
    }
    float* rec = p.part + (rec0 + r) * REC;
    rec[i] = a;
    if (i == 0) {
      rec[D] = M;
      rec[D + 1] = L;
    }
  }
}

template <int CBKH, int CBKL, int CBVH, int CBVL>
static hipError_t run_decode_split(const DecodeSplitParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<CBKH, CBKL, CBVH, CBVL>), grid,
                     dim3(SplitGeom<CBKH, CBKL, CBVH, CBVL>::kThreads), 0, s, p);
  return hipGetLastError();
}

bool decode_split_supported(const tq_split_codec& kc, const tq_split_codec& vc) {
  const int kh = kc.hi.code_bits, kl = kc.lo.code_bits, vh = vc.hi.code_bits, vl = vc.lo.code_bits;
  const bool kok = (kh == 2 && kl == 1) || (kh == 3 && kl == 2);
  const bool vok = (vh == 3 && vl == 2) || (vh == 4 && vl == 3);
  return kok && vok;
}

hipError_t launch_decode_split(const tq_split_codec& kc, const tq_split_codec& vc, const void* q,
                               int q_dtype, int batch, int n_q, int hq, int hkv, const tq_packed* k,
                               const tq_packed* v, int64_t ctx, float scale, float* out,
                               float* scores_out, void* workspace, hipStream_t stream) {
  int nchunks, splits;
  int64_t split_len;
  plan_decode(batch, n_q, hq, hkv, ctx, nchunks, splits, split_len);
  const size_t groups = (size_t)batch * hkv * nchunks;
  DecodeSplitParams p = {};
  p.q = q;
  p.q_f16 = q_dtype == TQ_F16;
  for (int h = 0; h < 2; ++h) {
    const tq_codec& kh = h ? kc.lo : kc.hi;
    const tq_codec& vh = h ? vc.lo : vc.hi;
    p.kidx[h] = k[h].idx; p.kqjl[h] = k[h].qjl; p.knorm[h] = k[h].norm; p.krnorm[h] = k[h].rnorm;
    p.vidx[h] = v[h].idx; p.vnorm[h] = v[h].norm;
    p.S[h] = kh.S;
    for (int i = 0; i < 16; ++i) { p.kcent[h][i] = kh.centroids[i]; p.vcent[h][i] = vh.centroids[i]; }
    p.kflip[2 * h] = kh.flip[0];
    p.kflip[2 * h + 1] = kh.flip[1];
  }
  p.scores_out = scores_out;
  p.part = reinterpret_cast<float*>(workspace);
  p.ctx = ctx; p.batch = batch; p.hq = hq; p.hkv = hkv; p.n_q = n_q; p.G = hq / hkv;
  p.nchunks = nchunks; p.splits = splits; p.split_len = split_len;
  p.scale = scale > 0.f ? scale : (float)(1.0 / std::sqrt(128.0));
  p.qjl_scale = (float)(std::sqrt(M_PI / 2.0) / 64.0);
  const dim3 grid((unsigned)groups, (unsigned)splits);
  const int key = kc.hi.code_bits * 1000 + kc.lo.code_bits * 100 + vc.hi.code_bits * 10 + vc.lo.code_bits;
  hipError_t e;
  switch (key) {
    case 2132: e = run_decode_split<2, 1, 3, 2>(p, grid, stream); break;
    case 2143: e = run_decode_split<2, 1, 4, 3>(p, grid, stream); break;
    case 3232: e = run_decode_split<3, 2, 3, 2>(p, grid, stream); break;
    case 3243: e = run_decode_split<3, 2, 4, 3>(p, grid, stream); break;
    default: return hipErrorNotSupported;
  }
  if (e != hipSuccess) return e;
  MergeParams mp = {};
  mp.part = p.part;
  mp.out = out;
  mp.hq = hq; mp.hkv = hkv; mp.n_q = n_q; mp.G = hq / hkv; mp.nchunks = nchunks;
  mp.splits = splits;
  mp.wht_len = 64;
  mp.inv_sqrt_d = 0.125f;
  mp.vflip[0] = vc.hi.flip[0]; mp.vflip[1] = vc.hi.flip[1];
  mp.vflip[2] = vc.lo.flip[0]; mp.vflip[3] = vc.lo.flip[1];
  const unsigned rows = (unsigned)((int64_t)batch * hq * n_q);
  hipLaunchKernelGGL((merge_kernel<128>), dim3(rows), dim3(128), 0, stream, mp);
  return hipGetLastError();
}

}  // namespace tqk
