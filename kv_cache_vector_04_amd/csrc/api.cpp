// C-ABI entry points: argument validation on the host, then the launchers.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"
#include "tq.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool gpu_dim(int d) { return d == 64 || d == 128 || d == 1536; }

int check_codec(const tq_codec* c) {
  if (c == nullptr) return TQ_ERR_INVALID_ARG;
  if (c->mode != TQ_MSE && c->mode != TQ_PROD) return TQ_ERR_INVALID_ARG;
  if (c->code_bits < 1 || c->code_bits > 4) return TQ_ERR_INVALID_ARG;
  if (c->bits != c->code_bits + (c->mode == TQ_PROD ? 1 : 0)) return TQ_ERR_INVALID_ARG;
  if (c->mode == TQ_PROD && (c->m != c->d || c->S == nullptr || !aligned(c->S, 16)))
    return TQ_ERR_INVALID_ARG;
  if (c->mode == TQ_MSE && c->m != 0) return TQ_ERR_INVALID_ARG;
  if (!gpu_dim(c->d)) return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

int check_planes(const tq_codec* c, const tq_packed* p) {
  if (p == nullptr || p->idx == nullptr || p->norm == nullptr) return TQ_ERR_INVALID_ARG;
  const size_t row_bytes = (size_t)c->d * c->code_bits / 8;
  if (!aligned(p->idx, row_bytes % 16 == 0 ? 16 : 8) || !aligned(p->norm, 4))
    return TQ_ERR_INVALID_ARG;
  if (c->mode == TQ_PROD) {
    if (p->qjl == nullptr || p->rnorm == nullptr) return TQ_ERR_INVALID_ARG;
    if (!aligned(p->qjl, c->d == 1536 ? 16 : 8) || !aligned(p->rnorm, 4)) return TQ_ERR_INVALID_ARG;
  }
  return TQ_OK;
}

tqk::RopeHost rope_of(const tq_rope* r) {
  tqk::RopeHost h = {};
  if (r != nullptr) {
    h.on = true;
    h.base = r->base;
    h.pos0 = r->pos0;
    h.seq_len = r->seq_len;
  }
  return h;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

}  // namespace

namespace tqk {
int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}
}  // namespace tqk

namespace {

size_t encode_need(const tq_codec* kc, const tq_codec* vc, int64_t n_rows) {
  size_t need = 0;
  for (const tq_codec* c : {kc, vc}) {
    if (c == nullptr) continue;
    const size_t b = tqk::wide_encode_workspace_bytes(*c, n_rows);
    if (b > need) need = b;
  }
  return need;
}

}  // namespace

extern "C" size_t tq_encode_kv_workspace(const tq_codec* kc, const tq_codec* vc, int64_t n_rows) {
  if (n_rows <= 0) return 0;
  return encode_need(kc, vc, n_rows);
}

extern "C" int tq_encode_kv(const tq_codec* kc, const tq_codec* vc, const void* k,
                            const void* v, int dtype, int64_t n_rows, const tq_rope* rope,
                            const tq_packed* kout, const tq_packed* vout, void* workspace,
                            size_t workspace_bytes, tq_stream_t stream) {
  if (kc == nullptr && vc == nullptr) return TQ_ERR_INVALID_ARG;
  if (n_rows < 0) return TQ_ERR_INVALID_ARG;
  if (dtype != TQ_F16 && dtype != TQ_F32) return TQ_ERR_INVALID_ARG;
  if (rope != nullptr) {
    if (kc == nullptr || !(rope->base > 0.f) || rope->seq_len <= 0) return TQ_ERR_INVALID_ARG;
    // RoPE is fused for the d = 64 fp16 key path (the RoPE workload here)
    if (dtype != TQ_F16 || kc->d != 64) return TQ_ERR_UNSUPPORTED;
  }
  const tq_codec* cs[2] = {kc, vc};
  const void* xs[2] = {k, v};
  const tq_packed* outs[2] = {kout, vout};
  for (int s = 0; s < 2; ++s) {
    if (cs[s] == nullptr) continue;
    const int st = check_codec(cs[s]);
    if (st != TQ_OK) return st;
  }
  // zero rows: nothing to read or write, so no pointer needs to be valid
  if (n_rows == 0) return TQ_OK;
  for (int s = 0; s < 2; ++s) {
    if (cs[s] == nullptr) continue;
    const int st = check_planes(cs[s], outs[s]);
    if (st != TQ_OK) return st;
    if (xs[s] == nullptr || !aligned(xs[s], 16)) return TQ_ERR_INVALID_ARG;
  }
  const size_t need = encode_need(kc, vc, n_rows);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256)))
    return TQ_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (kc != nullptr && vc != nullptr && tqk::encode_kv_fusable(*kc, *vc, dtype, rope != nullptr))
    return hip_status(tqk::launch_encode_kv(*kc, *vc, k, v, n_rows, *kout, *vout, hs));
  for (int s = 0; s < 2; ++s) {
    if (cs[s] == nullptr) continue;
    const tqk::RopeHost rh = s == 0 ? rope_of(rope) : tqk::RopeHost{};
    const int st = hip_status(tqk::launch_encode(*cs[s], xs[s], dtype, n_rows, rh, *outs[s], workspace, hs));
    if (st != TQ_OK) return st;
  }
  return TQ_OK;
}

extern "C" int tq_decode_kv(const tq_codec* c, const tq_packed* in, int64_t n_rows, void* out,
                            int out_dtype, tq_stream_t stream) {
  int st = check_codec(c);
  if (st != TQ_OK) return st;
  if (c->d != 64 && c->d != 128) return TQ_ERR_UNSUPPORTED;
  if (n_rows < 0 || (out_dtype != TQ_F16 && out_dtype != TQ_F32)) return TQ_ERR_INVALID_ARG;
  // zero rows: nothing to read or write, so no pointer needs to be valid
  if (n_rows == 0) return TQ_OK;
  if ((st = check_planes(c, in)) != TQ_OK) return st;
  if (out == nullptr || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  return hip_status(tqk::launch_materialize(*c, *in, n_rows, out, out_dtype,
                                            reinterpret_cast<hipStream_t>(stream)));
}

namespace {

// both halves 64 wide: the split of a 128-channel row
int check_split_codec(const tq_split_codec* c) {
  int st = check_codec(&c->hi);
  if (st != TQ_OK) return st;
  if ((st = check_codec(&c->lo)) != TQ_OK) return st;
  return c->hi.d != 64 || c->lo.d != 64 ? TQ_ERR_UNSUPPORTED : TQ_OK;
}

int check_split(const tq_split_codec* c, const tq_packed* planes) {
  int st = check_split_codec(c);
  if (st != TQ_OK) return st;
  if (planes == nullptr) return TQ_ERR_INVALID_ARG;
  if ((st = check_planes(&c->hi, &planes[0])) != TQ_OK) return st;
  return check_planes(&c->lo, &planes[1]);
}

}  // namespace

extern "C" int tq_encode_split(const tq_split_codec* kc, const tq_split_codec* vc, const void* k,
                               const void* v, int dtype, int64_t n_rows, const tq_packed* kout,
                               const tq_packed* vout, tq_stream_t stream) {
  if (kc == nullptr && vc == nullptr) return TQ_ERR_INVALID_ARG;
  if (n_rows < 0 || (dtype != TQ_F16 && dtype != TQ_F32)) return TQ_ERR_INVALID_ARG;
  const tq_split_codec* cs[2] = {kc, vc};
  const void* xs[2] = {k, v};
  const tq_packed* outs[2] = {kout, vout};
  if (n_rows == 0) {
    // zero rows: the codecs must still be valid, no pointer is read
    for (int s = 0; s < 2; ++s) {
      if (cs[s] == nullptr) continue;
      const int st = check_split_codec(cs[s]);
      if (st != TQ_OK) return st;
    }
    return TQ_OK;
  }
  for (int s = 0; s < 2; ++s) {
    if (cs[s] == nullptr) continue;
    const int st = check_split(cs[s], outs[s]);
    if (st != TQ_OK) return st;
    if (xs[s] == nullptr || !aligned(xs[s], 16)) return TQ_ERR_INVALID_ARG;
  }
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const int64_t stride = 128;
  const size_t esize = dtype == TQ_F16 ? 2 : 4;
  for (int half = 0; half < 2; ++half) {
    const tq_codec* hc[2];
    const void* hx[2];
    for (int s = 0; s < 2; ++s) {
      hc[s] = cs[s] == nullptr ? nullptr : (half == 0 ? &cs[s]->hi : &cs[s]->lo);
      hx[s] = cs[s] == nullptr ? nullptr : static_cast<const char*>(xs[s]) + half * 64 * esize;
    }
    if (hc[0] != nullptr && hc[1] != nullptr && tqk::encode_kv_fusable(*hc[0], *hc[1], dtype, false)) {
      const int st = hip_status(tqk::launch_encode_kv(*hc[0], *hc[1], hx[0], hx[1], n_rows, kout[half],
                                                      vout[half], hs, stride));
      if (st != TQ_OK) return st;
      continue;
    }
    for (int s = 0; s < 2; ++s) {
      if (hc[s] == nullptr) continue;
      const int st = hip_status(tqk::launch_encode(*hc[s], hx[s], dtype, n_rows, tqk::RopeHost{},
                                                   outs[s][half], nullptr, hs, stride));
      if (st != TQ_OK) return st;
    }
  }
  return TQ_OK;
}

extern "C" int tq_decode_split(const tq_split_codec* c, const tq_packed* in, int64_t n_rows,
                               void* out, int out_dtype, tq_stream_t stream) {
  if (c == nullptr) return TQ_ERR_INVALID_ARG;
  int st = check_split_codec(c);
  if (st != TQ_OK) return st;
  if (n_rows < 0 || (out_dtype != TQ_F16 && out_dtype != TQ_F32)) return TQ_ERR_INVALID_ARG;
  // zero rows: nothing to read or write, so no pointer needs to be valid
  if (n_rows == 0) return TQ_OK;
  if ((st = check_split(c, in)) != TQ_OK) return st;
  if (out == nullptr || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const size_t esize = out_dtype == TQ_F16 ? 2 : 4;
  if ((st = hip_status(tqk::launch_materialize(c->hi, in[0], n_rows, out, out_dtype, hs, 128))) != TQ_OK)
    return st;
  return hip_status(tqk::launch_materialize(c->lo, in[1], n_rows, static_cast<char*>(out) + 64 * esize,
                                            out_dtype, hs, 128));
}

namespace {

int check_vq(const tq_vq_codec* c, int64_t n_rows) {
  if (c == nullptr || n_rows < 0) return TQ_ERR_INVALID_ARG;
  if (c->n_codes < 2 || c->n_codes > TQ_VQ_MAX_CODES || (c->n_codes & (c->n_codes - 1)) ||
      (1 << c->block_bits) != c->n_codes)
    return TQ_ERR_INVALID_ARG;
  if (c->d != 64 && c->d != 128) return TQ_ERR_UNSUPPORTED;
  if (c->search != nullptr && !aligned(c->search, 16)) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

}  // namespace

extern "C" int tq_encode_vq(const tq_vq_codec* c, const void* x, int dtype, int64_t n_rows,
                            uint8_t* idx, float* norm, tq_stream_t stream) {
  int st = check_vq(c, n_rows);
  if (st != TQ_OK) return st;
  if (dtype != TQ_F16 && dtype != TQ_F32) return TQ_ERR_INVALID_ARG;
  if (n_rows == 0) return TQ_OK;
  if (x == nullptr || idx == nullptr || norm == nullptr || !aligned(x, 16) || !aligned(idx, 4) ||
      !aligned(norm, 4))
    return TQ_ERR_INVALID_ARG;
  return hip_status(tqk::launch_encode_vq(*c, x, dtype, n_rows, idx, norm,
                                          reinterpret_cast<hipStream_t>(stream)));
}

extern "C" int tq_decode_vq(const tq_vq_codec* c, const uint8_t* idx, const float* norm,
                            int64_t n_rows, void* out, int out_dtype, tq_stream_t stream) {
  int st = check_vq(c, n_rows);
  if (st != TQ_OK) return st;
  if (out_dtype != TQ_F16 && out_dtype != TQ_F32) return TQ_ERR_INVALID_ARG;
  if (n_rows == 0) return TQ_OK;
  if (out == nullptr || idx == nullptr || norm == nullptr || !aligned(out, 16) || !aligned(idx, 4) ||
      !aligned(norm, 4))
    return TQ_ERR_INVALID_ARG;
  return hip_status(tqk::launch_decode_vq(*c, idx, norm, n_rows, out, out_dtype,
                                          reinterpret_cast<hipStream_t>(stream)));
}

extern "C" size_t tq_attend_decode_workspace(int batch, int n_q, int hq, int hkv,
                                             int64_t ctx, int d) {
  if (batch <= 0 || n_q <= 0 || hq <= 0 || hkv <= 0 || ctx <= 0 || d <= 0) return 0;
  return tqk::attend_workspace_bytes(batch, n_q, hq, hkv, ctx, d);
}

extern "C" int tq_attend_split(const tq_split_codec* kc, const tq_split_codec* vc, const void* q,
                               int q_dtype, int batch, int n_q, int hq, int hkv, const tq_packed* k,
                               const tq_packed* v, int64_t ctx, float scale, float* out,
                               float* scores_out, void* workspace, size_t workspace_bytes,
                               tq_stream_t stream) {
  if (kc == nullptr || vc == nullptr) return TQ_ERR_INVALID_ARG;
  int st = check_split(kc, k);
  if (st != TQ_OK) return st;
  if ((st = check_split(vc, v)) != TQ_OK) return st;
  if (kc->hi.mode != TQ_PROD || kc->lo.mode != TQ_PROD || vc->hi.mode != TQ_MSE || vc->lo.mode != TQ_MSE)
    return TQ_ERR_UNSUPPORTED;
  if (!tqk::decode_split_supported(*kc, *vc)) return TQ_ERR_UNSUPPORTED;
  if (q == nullptr || out == nullptr || !aligned(q, 16) || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F16 && q_dtype != TQ_F32) return TQ_ERR_INVALID_ARG;
  if (batch <= 0 || n_q <= 0 || hq <= 0 || hkv <= 0 || ctx <= 0) return TQ_ERR_INVALID_ARG;
  if (hq % hkv) return TQ_ERR_INVALID_ARG;
  if ((hq / hkv) * n_q > 16) return TQ_ERR_UNSUPPORTED;
  if (ctx > ((int64_t)1 << 26)) return TQ_ERR_UNSUPPORTED;      // 32-bit offsets in a token range
  if (!(scale >= 0.f)) return TQ_ERR_INVALID_ARG;
  for (int h = 0; h < 2; ++h)
    if (!aligned(k[h].qjl, 8) || !aligned(v[h].idx, 4)) return TQ_ERR_INVALID_ARG;
  const size_t need = tqk::attend_workspace_bytes(batch, n_q, hq, hkv, ctx, 128);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return TQ_ERR_WORKSPACE;
  return hip_status(tqk::launch_decode_split(*kc, *vc, q, q_dtype, batch, n_q, hq, hkv, k, v, ctx,
                                             scale, out, scores_out, workspace,
                                             reinterpret_cast<hipStream_t>(stream)));
}

extern "C" int tq_attend_decode(const tq_codec* kc, const tq_codec* vc, const void* q,
                                int q_dtype, int batch, int n_q, int hq, int hkv,
                                const tq_rope* q_rope, const tq_packed* k,
                                const tq_packed* v, int64_t ctx, float scale, float* out,
                                float* scores_out, void* workspace, size_t workspace_bytes,
                                tq_stream_t stream) {
  int st = check_codec(kc);
  if (st != TQ_OK) return st;
  if ((st = check_codec(vc)) != TQ_OK) return st;
  if (kc->mode != TQ_PROD || vc->mode != TQ_MSE) return TQ_ERR_UNSUPPORTED;
  if (kc->d != vc->d) return TQ_ERR_INVALID_ARG;
  if (kc->d != 64 && kc->d != 128) return TQ_ERR_UNSUPPORTED;   // attention kernels: d = 64, 128
  if (q == nullptr || out == nullptr || !aligned(q, 16) || !aligned(out, 16))
    return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F16 && q_dtype != TQ_F32) return TQ_ERR_INVALID_ARG;
  if (batch <= 0 || n_q <= 0 || hq <= 0 || hkv <= 0 || ctx <= 0) return TQ_ERR_INVALID_ARG;
  if (hq % hkv) return TQ_ERR_INVALID_ARG;
  if (hq / hkv > 16) return TQ_ERR_UNSUPPORTED;
  // the kernels address one (batch, KV head)'s rows (up to 64 bytes each)
  // with 32-bit byte offsets
  if (ctx >= ((int64_t)1 << 25)) return TQ_ERR_UNSUPPORTED;
  if (!(scale >= 0.f)) return TQ_ERR_INVALID_ARG;
  if (q_rope != nullptr && (!(q_rope->base > 0.f) || q_rope->pos0 < 0)) return TQ_ERR_INVALID_ARG;
  if ((st = check_planes(kc, k)) != TQ_OK) return st;
  if ((st = check_planes(vc, v)) != TQ_OK) return st;
  const size_t need = tqk::attend_workspace_bytes(batch, n_q, hq, hkv, ctx, kc->d);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return TQ_ERR_WORKSPACE;
  return hip_status(tqk::launch_attend(*kc, *vc, q, q_dtype, batch, n_q, hq, hkv,
                                       rope_of(q_rope), *k, *v, ctx, scale, out, scores_out,
                                       workspace, reinterpret_cast<hipStream_t>(stream)));
}

extern "C" size_t tq_inner_product_workspace(int64_t n_q, int64_t n, int d, int top_k) {
  if (n_q <= 0 || n <= 0 || d <= 0 || top_k < 0) return 0;
  return tqk::scan_workspace_bytes(n_q, n, d, top_k);
}

extern "C" int tq_inner_product(const tq_codec* c, const void* q, int q_dtype, int64_t n_q,
                                const tq_packed* x, int64_t n, float* out, int top_k,
                                int64_t* top_ids, float* top_scores, void* workspace,
                                size_t workspace_bytes, tq_stream_t stream) {
  int st = check_codec(c);
  if (st != TQ_OK) return st;
  if (q == nullptr || !aligned(q, 16)) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F16 && q_dtype != TQ_F32) return TQ_ERR_INVALID_ARG;
  if (n_q <= 0 || n <= 0) return TQ_ERR_INVALID_ARG;
  if (top_k < 0 || top_k > 64) return TQ_ERR_INVALID_ARG;
  if (top_k > 0 && (top_ids == nullptr || top_scores == nullptr)) return TQ_ERR_INVALID_ARG;
  if (top_k == 0 && out == nullptr) return TQ_ERR_INVALID_ARG;
  if (top_k > n) return TQ_ERR_INVALID_ARG;
  if ((st = check_planes(c, x)) != TQ_OK) return st;
  // d = 1536 with 1-bit codes scores with +-1 operands: the table must be symmetric
  if (c->d == 1536 && c->code_bits == 1 && !(c->centroids[0] == -c->centroids[1] && c->centroids[1] > 0.f))
    return TQ_ERR_UNSUPPORTED;
  const size_t need = tqk::scan_workspace_bytes(n_q, n, c->d, top_k);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 16)))
    return TQ_ERR_WORKSPACE;
  return hip_status(tqk::launch_scan(*c, q, q_dtype, n_q, *x, n, out, top_k, top_ids, top_scores,
                                     workspace, reinterpret_cast<hipStream_t>(stream)));
}
