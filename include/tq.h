/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant KV-cache codec.
 *
 * The codec stores, per vector x of dimension d, its L2 norm nu = |x|, and
 * quantizes every coordinate of z = Pi (x / nu) with a scalar Lloyd-Max table
 * for the Beta coordinate density; Pi u = H_d (D * u) / sqrt(d) is a
 * randomized Walsh-Hadamard rotation (random sign flip D, then the Hadamard
 * matrix).  TurboQuant_prod (keys) spends b-1 bits on that table and one bit
 * per QJL row on the signs of S r, r = z - c[idx], S an m x d Gaussian
 * matrix, so that inner products can be estimated without bias; it also
 * stores gamma = |r|.  TurboQuant_mse (values) spends all b bits on the table.
 *
 * Sources (page titles and sections):
 *  - "FibQuant: Quantizzazione Vettoriale Universale per la Compressione della
 *    KV-Cache ad Accesso Casuale": "1. Enunciato del Problema" (fixed-rate
 *    codes at fixed addresses; normalize, rotate, quantize), "2.3 Codifica e
 *    Decodifica" (encoder and decoder steps), "5. Significato e Affermazioni"
 *    (fixed addresses let decompression fuse into attention kernels).
 *  - "Google presenta TurboQuant ..." (7minutos.es): "La mecánica geométrica
 *    de TurboQuant" (Beta coordinate law, cost C(f_X, b), codebooks solved
 *    once and stored), "Eliminación del sesgo interno del producto"
 *    (TurboQuant_prod, 1-bit QJL on the residual, unbiased estimator).
 *  - "Ablazione, Inferenza Statistica e Validazione per la Compressione della
 *    KV-Cache": "Configurazione Sperimentale" (randomized Walsh-Hadamard
 *    rotation, Beta Lloyd-Max codebook, QJL sketch on the key path only).
 *  - "TurboESM: ...": "2. Metodologia" part A (RoPE first, then the rotation)
 *    and part E (one fused pass: unpack, correct, attend with online softmax).
 *
 * Conventions for every entry point:
 *  - Pointers documented as "device" point to GPU memory; "host" to CPU
 *    memory.  The caller owns every buffer, the stream and the structs; the
 *    library keeps no pointer after a call returns and allocates nothing.
 *  - Calls that launch kernels enqueue them on `stream` and return at once;
 *    they never synchronize the host.  A fault inside a kernel surfaces at the
 *    caller's next synchronization, not as a status of the launching call.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    invalid call enqueues nothing and returns a negative status.
 *  - Vectors are rows of d elements, row-major, rows laid out
 *    [batch][head][token] (token fastest).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef TQ_STREAM_T_DEFINED
#define TQ_STREAM_T_DEFINED
typedef struct ihipStream_t* tq_stream_t; /* a hipStream_t; NULL = null stream */
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,   /* null or inconsistent argument */
  TQ_ERR_UNSUPPORTED = -2,   /* valid request this build has no kernel for */
  TQ_ERR_NOT_CONVERGED = -3, /* codebook iteration hit its limit */
  TQ_ERR_HIP = -4,           /* the HIP runtime reported a launch error */
  TQ_ERR_WORKSPACE = -5,     /* workspace null or smaller than required */
  TQ_ERR_TOO_LARGE = -6      /* request needs more than the fixed scratch of
                                tq_attend_decode_noalloc */
};

enum { TQ_MSE = 0, TQ_PROD = 1 };   /* codec mode */
enum { TQ_F16 = 0, TQ_F32 = 1 };    /* element type of input vectors */

#define TQ_MAX_LEVELS 16            /* 2^b' for b' <= 4 */
#define TQ_MAX_D 1536

/* Returns a static, human-readable name of a status code. */
const char* tq_status_string(int status);

/* ---- a0: codebook (host only) -----------------------------------------
 * Lloyd-Max scalar quantizer for the density of one coordinate of a uniform
 * point on S^{d-1}, f_d(x) ~ (1 - x^2)^((d-3)/2) on [-1, 1], at `bits`
 * (1..4) bits: minimises the MSE cost C(f_X, b) of "La mecánica geométrica de
 * TurboQuant", outer cells extending to -1 and +1.  Deterministic fp64.
 *   centroids  host, 2^bits doubles, ascending (output)
 *   thresholds host, 2^bits - 1 doubles, midpoints of neighbours (output)
 * Returns TQ_OK, TQ_ERR_INVALID_ARG (d < 3, bits outside 1..4, null output)
 * or TQ_ERR_NOT_CONVERGED.  Touches no GPU state; callable without a GPU. */
int tq_build_codebook(int d, int bits, double* centroids, double* thresholds);

/* ---- a1: one codec instance ---------------------------------------------
 * Plain host struct; kernels receive the table and the sign mask by value.
 * Fill it with tq_codec_init.  `code_bits` b' = bits - 1 for TQ_PROD and
 * bits for TQ_MSE. */
typedef struct tq_codec {
  int32_t d;          /* 64, 128 or 1536 on the GPU */
  int32_t mode;       /* TQ_MSE or TQ_PROD */
  int32_t bits;       /* total bits per coordinate b */
  int32_t code_bits;  /* scalar code width b' (1..4) */
  int32_t m;          /* QJL rows: d for TQ_PROD, 0 for TQ_MSE */
  int32_t reserved;
  float centroids[TQ_MAX_LEVELS];   /* first 2^b' used, fp32 of the fp64 table */
  float thresholds[TQ_MAX_LEVELS];  /* first 2^b' - 1 used */
  uint32_t flip[TQ_MAX_D / 32];     /* bit i%32 of word i/32 set <=> D_i = -1 */
  const float* S;     /* device, m x d row-major fp32, p_i = sum_k S[i][k] r_k;
                         NULL for TQ_MSE */
} tq_codec;

/* Builds the table for (d, b') with tq_build_codebook, rounds it to fp32 and
 * fills `codec`.  flip: host, ceil(d/32) words in the layout above.  S: the
 * caller's device matrix for TQ_PROD (m = d rows), ignored for TQ_MSE.
 * Host only.  Returns TQ_OK or TQ_ERR_INVALID_ARG / TQ_ERR_NOT_CONVERGED. */
int tq_codec_init(tq_codec* codec, int d, int mode, int bits,
                  const uint32_t* flip, const float* S);

/* ---- a7: packed planes ----------------------------------------------------
 * Fixed rate and fixed addresses: row j's codes start at byte j*(d*b'/8) of
 * `idx` and form one LSB-first bit stream (code i in stream bits
 * [i*b', (i+1)*b'), stream bit k = bit k%8 of byte k/8); its QJL bits start at
 * byte j*(m/8) of `qjl`, bit i = 1 iff (S r)_i >= 0, same bit order.  All
 * device pointers; idx and qjl 16-byte aligned. */
typedef struct tq_packed {
  uint8_t* idx;   /* n rows of d*b'/8 bytes */
  uint8_t* qjl;   /* n rows of m/8 bytes (TQ_PROD), else NULL */
  float* norm;    /* n floats: nu = |x| */
  float* rnorm;   /* n floats: gamma = |r| (TQ_PROD), else NULL */
} tq_packed;

/* RoPE before the rotation ("TurboESM", "2. Metodologia" part A): interleaved
 * pairs (2i, 2i+1) rotated by position * base^(-2i/d).  Row r of an encode
 * call sits at position r % seq_len; query a of an attend call at position
 * pos0 + a. */
typedef struct tq_rope {
  float base;       /* e.g. 10000 */
  int32_t pos0;     /* first query position (attend only) */
  int64_t seq_len;  /* tokens per sequence (encode only) */
} tq_rope;

/* ---- a2..a7: encode --------------------------------------------------------
 * Encodes n_rows rows of K with `kc` into `kout` and n_rows rows of V with
 * `vc` into `vout`; pass NULL for a side to skip it.  Per row:
 * (RoPE on K if `rope` is not NULL), nu = |x|, z = Pi x / nu, idx_i =
 * #{k : z_i >= t_k}, and for TQ_PROD r = z - c[idx], gamma = |r|, signs of
 * S r ("FibQuant" 2.3; "Google presenta TurboQuant" mechanics and prod
 * sections).  The zero vector encodes as z = 0 with nu = 0.  A vector with
 * an inf or NaN element (after RoPE, when applied) also encodes as z = 0 and
 * stores its non-finite norm: inf, or NaN when a NaN is present.
 *   k, v      device, n_rows x d elements of type `dtype`, 16-byte aligned
 *   kc, vc    host structs (kc TQ_PROD or TQ_MSE; vc either); d = 64, 128 or
 *             1536 (d = 1536: Pi uses H_12 (x) H_128, H_12 by Paley's
 *             construction at q = 11; qjl planes 16-byte aligned)
 *   kout/vout host structs of device planes sized for n_rows
 *   workspace device, >= tq_encode_kv_workspace(kc, vc, n_rows) bytes,
 *             256-byte aligned; may be NULL when that size is 0 (it is 0
 *             for d = 64 and 128 and for TQ_MSE).  Contents need no
 *             initialisation; calls sharing it must not overlap in time.
 * n_rows = 0 checks the codecs and returns TQ_OK without reading any
 * pointer (k, v, the planes and workspace may then be NULL).
 * Returns TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE or
 * TQ_ERR_HIP. */
size_t tq_encode_kv_workspace(const tq_codec* kc, const tq_codec* vc, int64_t n_rows);
int tq_encode_kv(const tq_codec* kc, const tq_codec* vc, const void* k,
                 const void* v, int dtype, int64_t n_rows, const tq_rope* rope,
                 const tq_packed* kout, const tq_packed* vout, void* workspace,
                 size_t workspace_bytes, tq_stream_t stream);

/* ---- decode: packed rows back to vectors ---------------------------------
 * The materializing decoder ("FibQuant", "2.3 Codifica e Decodifica": look
 * the centroids up, rotate back, rescale by the norm; "Google presenta
 * TurboQuant", unbiased prod section for the QJL term):
 *   TQ_MSE:  x_hat = nu * Pi^T c[idx]
 *   TQ_PROD: x_hat = nu * Pi^T (c[idx] + sqrt(pi/2)/m * gamma * S^T (2 sigma - 1))
 * with Pi^T w = D (H_d w) / sqrt(d).  It is the first pass of a two-pass
 * attention (decode, then plain attention on the vectors); tq_attend_decode
 * does not need it.
 *   c     host codec, d = 64 or 128 (other d: TQ_ERR_UNSUPPORTED)
 *   in    host struct of device planes holding n_rows rows
 *   out   device [n_rows][d] of out_dtype (TQ_F16, rounded toward zero, or
 *         TQ_F32), 16-byte aligned; written only
 * n_rows = 0 checks the codec and returns TQ_OK; `in` and `out` may then be
 * NULL.
 * Returns TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED or TQ_ERR_HIP. */
int tq_decode_kv(const tq_codec* c, const tq_packed* in, int64_t n_rows, void* out,
                 int out_dtype, tq_stream_t stream);

/* ---- outlier-channel split: rates between whole bits ----------------------
 * "Google presenta TurboQuant", "Desempeño teórico y empírico": for rates
 * between whole bits, outlier channels get more bits (e.g. 3) and the other
 * channels fewer (e.g. 2), for an effective 2.5 or 3.5 bits per channel.
 * A split codec is two codec instances over a channel partition: channels
 * [0, hi.d) of every row go through `hi`, channels [hi.d, hi.d + lo.d)
 * through `lo`, each with its own norm, sign flip, table, and (prod) S and
 * gamma.  The partition is positional.  A caller whose outlier channels sit
 * elsewhere applies one fixed channel permutation upstream (folded into the
 * projection weights that produce K, V and the queries), so that the outlier
 * channels come first; attention is unchanged by a permutation applied to
 * both q and k.  Supported: hi.d = lo.d = 64 (rows of 128 elements), for
 * (b_hi + b_lo) / 2 bits per channel plus the two norms: 3 + 2 -> 2.5,
 * 4 + 3 -> 3.5.  Inner products split the same way:
 * <q, x> = <q[0:64], x[0:64]> + <q[64:128], x[64:128]>. */
typedef struct tq_split_codec {
  tq_codec hi;   /* channels [0, hi.d) */
  tq_codec lo;   /* channels [hi.d, hi.d + lo.d) */
} tq_split_codec;

/* The channel order that puts a head's outlier channels first: the d_hi
 * channels of largest mean square over the calibration rows x (host,
 * n_rows x d fp32, row-major), ascending, then the other channels,
 * ascending; equal mean squares go to the lower channel.  order: host,
 * d int32 (output).  Returns TQ_OK, or TQ_ERR_INVALID_ARG (null pointer,
 * n_rows < 1, d_hi outside 0..d, or an inf / NaN in x).  Host only. */
int tq_outlier_order(const float* x, int64_t n_rows, int d, int d_hi, int32_t* order);

/* Encode rows of hi.d + lo.d elements, in place of two copies of the
 * halves: the `hi` channels of each row of k with kc->hi and the `lo`
 * channels with kc->lo, and likewise v with vc (either side may be null).
 *   k, v        device, n_rows x 128 of `dtype` (TQ_F16 or TQ_F32), 16-byte aligned
 *   kout, vout  arrays of two tq_packed: the hi half's planes, then the lo
 *               half's, each sized for its own codec as for tq_encode_kv
 * No RoPE and no workspace.  n_rows = 0 checks the codecs only (pointers may
 * be NULL).  Returns TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED (halves
 * other than 64 + 64) or TQ_ERR_HIP. */
int tq_encode_split(const tq_split_codec* kc, const tq_split_codec* vc, const void* k,
                    const void* v, int dtype, int64_t n_rows, const tq_packed* kout,
                    const tq_packed* vout, tq_stream_t stream);

/* Decode one tensor's two halves (in[0]: hi, in[1]: lo) into rows of
 * hi.d + lo.d elements of out_dtype (TQ_F16, rounded toward zero, or
 * TQ_F32) at `out` (device, 16-byte aligned), as tq_decode_kv does for
 * each half; n_rows = 0 checks the codec only. */
int tq_decode_split(const tq_split_codec* c, const tq_packed* in, int64_t n_rows, void* out,
                    int out_dtype, tq_stream_t stream);

/* ---- FibQuant k = 2: vector code on 2-coordinate blocks -------------------
 * "FibQuant", sections 2.1-2.3: the same normalise-rotate interface, but
 * each block (z_2j, z_2j+1) of the rotated unit vector is coded as the index
 * of its nearest codeword in one shared N-point code on the unit disk, at
 * b = log2(N) / 2 bits per coordinate (N = 2^1 .. 2^8: b = 0.5 .. 4, half-bit
 * steps).  Row j stores d/2 block codes of log2(N) bits in one LSB-first
 * stream at byte j * (d/2) * log2(N) / 8, and its norm. */
#define TQ_VQ_MAX_CODES 256

/* The N x 2 codebook for dimension d (host, fp64, deterministic): radii by
 * Bennett-Gersho companding of the block density (d-2)/(2 pi) (1-|y|^2)^((d-4)/2),
 * r_n^2 = 1 - (1 - (n + 1/2)/N)^(4/d); angles n times the golden angle
 * (planar Fibonacci spiral); then Lloyd iterations on a fixed polar
 * quadrature of the density, restarted at two spiral phases, the lower-MSE
 * code kept.
 *   codewords  host, 2 N doubles (x, y pairs), output
 * Returns TQ_OK or TQ_ERR_INVALID_ARG (d < 6, N not a power of two in
 * 2..256, null output).  Host only. */
int tq_build_vq_codebook(int d, int n_codes, double* codewords);

typedef struct tq_vq_codec {
  int32_t d;            /* 64 or 128 on the GPU */
  int32_t n_codes;      /* N */
  int32_t block_bits;   /* log2 N */
  int32_t reserved;
  float codewords[2 * TQ_VQ_MAX_CODES];  /* first N (x, y) pairs used, fp32 */
  uint32_t flip[TQ_MAX_D / 32];          /* as in tq_codec */
  const void* search;   /* device, TQ_VQ_SEARCH_BYTES, from tq_vq_search_build; NULL: full search */
} tq_vq_codec;

/* Builds the codebook with tq_build_vq_codebook, rounds it to fp32 and fills
 * `codec` (search = NULL); flip as for tq_codec_init.  Host only. */
int tq_vq_codec_init(tq_vq_codec* codec, int d, int n_codes, const uint32_t* flip);

/* The encoder's nearest-codeword search table.  Each block coordinate x is
 * companded, u = x / (|x| + a), and a TQ_VQ_GRID^2 grid is laid uniformly
 * over u in (-1, 1)^2: rectangular cells, narrow near 0 where the codewords
 * crowd, the outermost reaching the unit disk's edge.  For each cell it
 * lists, ascending, the codewords that can be nearest to some point of the
 * cell widened on every side (by 1e-5 plus 1e-6 of the companding slope),
 * within a score slack of 1e-5.  An empty list marks a cell for the full
 * search (a list longer than 48, or the longest lists when all of them
 * would overflow the TQ_VQ_ENTRIES pool).  The encoder tests a block only
 * against its cell's list, in ascending order with strict improvement,
 * which selects the same codeword as testing all N.  `a` is chosen per
 * codebook (from 2^(e/2 - 1) / sqrt(d), e = 0..12) to minimize the expected
 * number of tests on the block density.
 * Layout: float a, float G / 2, int32 G, int32 entries used; uint16
 * offsets[G^2 + 8] (cell k, row-major over (y cell, x cell), owns pool
 * entries [offsets[k], offsets[k + 1])); uint8 pool[TQ_VQ_ENTRIES] of
 * codeword indices.  tq_vq_search_build writes it for `c` into a host
 * buffer of at least TQ_VQ_SEARCH_BYTES; the caller copies it to device
 * memory (16-byte aligned) and sets c->search.  Returns TQ_OK or
 * TQ_ERR_INVALID_ARG.  Host only. */
#define TQ_VQ_GRID 64
#define TQ_VQ_ENTRIES 24576
#define TQ_VQ_SEARCH_BYTES (16 + 2 * (TQ_VQ_GRID * TQ_VQ_GRID + 8) + TQ_VQ_ENTRIES)
int tq_vq_search_build(const tq_vq_codec* c, void* table, size_t bytes);

/* Encode n_rows rows: nu = |x|, z = Pi x / nu, block code j = the nearest
 * codeword of (z_2j, z_2j+1) (ties to the lower index).  A zero row, or one
 * with a non-finite element, encodes as z = 0 (the latter keeps its
 * non-finite norm).
 *   x     device, n_rows x d of `dtype` (TQ_F16 or TQ_F32), 16-byte aligned
 *   idx   device, n_rows x (d/2) log2(N) / 8 bytes, 4-byte aligned (output)
 *   norm  device, n_rows floats (output)
 * d = 64 or 128 (other d: TQ_ERR_UNSUPPORTED).  n_rows = 0 checks the codec
 * only (pointers may be NULL).  Returns TQ_OK, TQ_ERR_INVALID_ARG,
 * TQ_ERR_UNSUPPORTED or TQ_ERR_HIP. */
int tq_encode_vq(const tq_vq_codec* c, const void* x, int dtype, int64_t n_rows,
                 uint8_t* idx, float* norm, tq_stream_t stream);

/* Decode: x_hat = nu * Pi^T (codewords of the row's blocks, concatenated),
 * written as n_rows x d of out_dtype (TQ_F16 rounded toward zero, or
 * TQ_F32) to `out` (device, 16-byte aligned); n_rows = 0 checks the codec
 * only. */
int tq_decode_vq(const tq_vq_codec* c, const uint8_t* idx, const float* norm, int64_t n_rows,
                 void* out, int out_dtype, tq_stream_t stream);

/* ---- a8..a11: attention from codes ----------------------------------------
 * For every batch b, query head h (KV head g = h / (hq / hkv)) and query a:
 *   s_j = scale * nu_j * ( <q', c_K[idx_j]> + sqrt(pi/2)/m * gamma_j *
 *                          <S q', 2 sigma_j - 1> ),   q' = Pi RoPE(q)
 *   o   = Pi_V^T ( sum_j softmax(s)_j * nu^V_j * c_V[idx^V_j] )
 * over all ctx tokens (no causal mask), computed in one pass over the codes
 * with an online softmax split over token ranges and merged by log-sum-exp
 * ("TurboESM" 2E; "Google presenta TurboQuant", unbiased estimator).
 *   kc  TQ_PROD codec of the keys; vc TQ_MSE codec of the values; d = 64 or
 *       128 (other d: TQ_ERR_UNSUPPORTED)
 *   q   device [batch][hq][n_q][d] of `q_dtype`
 *   k,v host structs of device planes, rows [batch][hkv][ctx]; ctx < 2^25
 *       (TQ_ERR_UNSUPPORTED beyond: 32-bit offsets inside a KV head)
 *   scale  0 selects 1/sqrt(d)
 *   out device [batch][hq][n_q][d] fp32
 *   scores_out  NULL, or device [batch][hq][n_q][ctx] fp32 receiving s_j
 *   workspace   device, >= tq_attend_decode_workspace(...) bytes, 16-byte
 *               aligned; it receives the per-token-range partial results
 *               (max, sum, weighted value sum per query row) that the merge
 *               reads back.  Every entry read is written first by the same
 *               call, so its contents need no initialisation.
 * Calls that share one workspace must not overlap in time. */
size_t tq_attend_decode_workspace(int batch, int n_q, int hq, int hkv,
                                  int64_t ctx, int d);
int tq_attend_decode(const tq_codec* kc, const tq_codec* vc, const void* q,
                     int q_dtype, int batch, int n_q, int hq, int hkv,
                     const tq_rope* q_rope, const tq_packed* k,
                     const tq_packed* v, int64_t ctx, float scale, float* out,
                     float* scores_out, void* workspace,
                     size_t workspace_bytes, tq_stream_t stream);

/* The same attention for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops or harnesses that forbid
 * allocation): arguments and results as tq_attend_decode, without the
 * workspace.  The kernels' scratch is a fixed device array inside the
 * library, TQ_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs
 * on holds until the process ends; its address is looked up the first time a
 * device calls in.  The call itself allocates nothing.
 * A request whose tq_attend_decode_workspace(...) exceeds
 * TQ_NOALLOC_SCRATCH_BYTES returns TQ_ERR_TOO_LARGE before anything is
 * enqueued.  All calls on one GPU share the array: calls that overlap in
 * time on one GPU (other streams, other host threads) race and must be
 * serialized by the caller.  Returns the statuses of tq_attend_decode, or
 * TQ_ERR_TOO_LARGE, or TQ_ERR_HIP when the scratch address cannot be
 * obtained. */
#define TQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int tq_attend_decode_noalloc(const tq_codec* kc, const tq_codec* vc, const void* q,
                             int q_dtype, int batch, int n_q, int hq, int hkv,
                             const tq_rope* q_rope, const tq_packed* k,
                             const tq_packed* v, int64_t ctx, float scale, float* out,
                             float* scores_out, tq_stream_t stream);

/* Attention from outlier-split codes: the keys and values of each token are
 * two d = 64 codecs over channels [0, 64) and [64, 128) (tq_encode_split), so
 *   s_j = scale * sum_h nu_hj ( <q'_h, c_Kh[idx_hj]> + sqrt(pi/2)/64 *
 *                               gamma_hj * <S_h q'_h, 2 sigma_hj - 1> ),
 *   q'_h = Pi_h q[h-th 64 channels],
 *   o[h-th 64 channels] = Pi_Vh^T ( sum_j softmax(s)_j * nu^V_hj * c_Vh[idx^V_hj] )
 * in one pass over the codes, like tq_attend_decode ("Google presenta
 * TurboQuant", "Desempeño teórico y empírico", for the rates between whole
 * bits; the estimator as in tq_attend_decode).
 *   kc  split codec of the keys (TQ_PROD halves), vc of the values (TQ_MSE
 *       halves); table widths (hi, lo) of (2, 1) or (3, 2) for the keys and
 *       (3, 2) or (4, 3) for the values (the 2.5- and 3.5-bit points);
 *       others: TQ_ERR_UNSUPPORTED
 *   q   device [batch][hq][n_q][128] of `q_dtype`, channels in the codecs'
 *       order (outlier channels first); no RoPE
 *   k,v arrays of two tq_packed (hi, lo), rows [batch][hkv][ctx]
 *   scale  0 selects 1/sqrt(128)
 *   out, scores_out, workspace: as tq_attend_decode, with the workspace size
 *       tq_attend_decode_workspace(batch, n_q, hq, hkv, ctx, 128)
 * (hq / hkv) * n_q <= 16 and ctx <= 2^26 (otherwise TQ_ERR_UNSUPPORTED).
 * Returns TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE or
 * TQ_ERR_HIP. */
int tq_attend_split(const tq_split_codec* kc, const tq_split_codec* vc, const void* q,
                    int q_dtype, int batch, int n_q, int hq, int hkv, const tq_packed* k,
                    const tq_packed* v, int64_t ctx, float scale, float* out,
                    float* scores_out, void* workspace, size_t workspace_bytes,
                    tq_stream_t stream);

/* ---- a12: inner-product scan (+ top-k) --------------------------------------
 * est(a, j) = nu_j ( <Pi q_a, c[idx_j]> + sqrt(pi/2)/m gamma_j
 *                    <S Pi q_a, 2 sigma_j - 1> )  (mse: first term only)
 * for n_q queries against n packed rows ("Google presenta TurboQuant",
 * "Velocidad y eficiencia de indexación").
 *   q        device [n_q][d] of `q_dtype`; d = 64, 128 or 1536 (at d = 1536
 *            a 1-bit table must be symmetric, c[0] = -c[1], as
 *            tq_codec_init builds it)
 *   out      NULL, or device [n_q][n] fp32
 *   top_k    0, or 1..64: per query the top_k largest estimates, descending,
 *            ties to the lower row index, into top_ids [n_q][top_k] (int64)
 *            and top_scores [n_q][top_k] (fp32), device
 *   workspace device, >= tq_inner_product_workspace(...) bytes (may be NULL
 *            when that is 0). */
size_t tq_inner_product_workspace(int64_t n_q, int64_t n, int d, int top_k);
int tq_inner_product(const tq_codec* c, const void* q, int q_dtype,
                     int64_t n_q, const tq_packed* x, int64_t n, float* out,
                     int top_k, int64_t* top_ids, float* top_scores,
                     void* workspace, size_t workspace_bytes,
                     tq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
