// Launchers behind the C ABI (host side).  Arguments are validated by the
// entry points in api.cpp before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tqk {

struct RopeHost {
  bool on;
  float base;
  int32_t pos0;
  int64_t seq_len;
};

// Encode n_rows rows of one tensor with one codec.  Row j of the input
// starts at element j * x_stride (0: c.d; d = 64 and 128 only otherwise).
hipError_t launch_encode(const tq_codec& c, const void* x, int dtype,
                         int64_t n_rows, const RopeHost& rope,
                         const tq_packed& out, void* workspace, hipStream_t stream,
                         int64_t x_stride = 0);

// Keys (prod) and values (mse) of one call in a single launch, for fp16
// inputs without RoPE at d = 64 or 128 and the code widths encode_kv_fusable
// accepts; the results equal two launch_encode calls.
bool encode_kv_fusable(const tq_codec& kc, const tq_codec& vc, int dtype, bool rope);
hipError_t launch_encode_kv(const tq_codec& kc, const tq_codec& vc, const void* k, const void* v,
                            int64_t n_rows, const tq_packed& kout, const tq_packed& vout,
                            hipStream_t stream, int64_t x_stride = 0);

// FibQuant k = 2 block codes (vq.hip).
hipError_t launch_encode_vq(const tq_vq_codec& c, const void* x, int dtype, int64_t n_rows, uint8_t* idx,
                            float* norm, hipStream_t stream);
hipError_t launch_decode_vq(const tq_vq_codec& c, const uint8_t* idx, const float* norm, int64_t n_rows,
                            void* out, int out_dtype, hipStream_t stream);

// Packed rows back to vectors (materialize.hip): n_rows x d of out_dtype,
// row j at element j * out_stride of out (0: c.d).
hipError_t launch_materialize(const tq_codec& c, const tq_packed& in, int64_t n_rows, void* out,
                              int out_dtype, hipStream_t stream, int64_t out_stride = 0);

// Attention from outlier-split codes (decode.hip): keys prod and values mse,
// each two d = 64 halves; table widths (hi, lo) of (2, 1) or (3, 2) for keys
// and (3, 2) or (4, 3) for values; G n_q <= 16; the workspace of the d = 128
// decode path.
bool decode_split_supported(const tq_split_codec& kc, const tq_split_codec& vc);
hipError_t launch_decode_split(const tq_split_codec& kc, const tq_split_codec& vc, const void* q,
                               int q_dtype, int batch, int n_q, int hq, int hkv, const tq_packed* k,
                               const tq_packed* v, int64_t ctx, float scale, float* out,
                               float* scores_out, void* workspace, hipStream_t stream);

// d = 1536 (wide.hip).  The encode workspace holds S as fp16 hi / lo planes
// and the residual planes of one block of vectors (prod only); the scan
// workspace holds the S planes and the four query planes.
size_t wide_encode_workspace_bytes(const tq_codec& c, int64_t n_rows);
hipError_t launch_wide_encode(const tq_codec& c, const void* x, int dtype, int64_t n_rows,
                              const tq_packed& out, void* workspace, hipStream_t stream);
size_t wide_scan_workspace_bytes(int64_t n_q);
hipError_t launch_wide_scan(const tq_codec& c, const void* q, int q_dtype, int64_t n_q,
                            const tq_packed& x, int64_t n, float* scores, void* workspace,
                            hipStream_t stream);

size_t attend_workspace_bytes(int batch, int n_q, int hq, int hkv, int64_t ctx, int d);
hipError_t launch_attend(const tq_codec& kc, const tq_codec& vc, const void* q,
                         int q_dtype, int batch, int n_q, int hq, int hkv,
                         const RopeHost& rope, const tq_packed& k,
                         const tq_packed& v, int64_t ctx, float scale,
                         float* out, float* scores_out, void* workspace,
                         hipStream_t stream);

bool decode_path(int n_q, int hq, int hkv);
// many query rows per KV head at d = 64 (attend_mq.hip)
bool mq_path(int n_q, int hq, int hkv, int d);
size_t mq_workspace_bytes(int batch, int n_q, int hq);
hipError_t launch_attend_mq(const tq_codec& kc, const tq_codec& vc, const void* q, int q_dtype,
                            int batch, int n_q, int hq, int hkv, const RopeHost& rope,
                            const tq_packed& k, const tq_packed& v, int64_t ctx, float scale,
                            float* out, float* scores_out, void* workspace, hipStream_t stream);
size_t decode_workspace_bytes(int batch, int n_q, int hq, int hkv, int64_t ctx, int d);
// few-row decode at d = 128 on the matrix cores (decode_mfma.hip): writes the
// same per-range records as the decode kernel, for the same merge
bool decode_mfma_supported(const tq_codec& kc, const tq_codec& vc);
hipError_t launch_decode_mfma(const tq_codec& kc, const tq_codec& vc, const void* q, int q_dtype,
                              int n_q, int hq, int hkv, const RopeHost& rope, const tq_packed& k,
                              const tq_packed& v, int64_t ctx, float scale, float* scores_out,
                              float* part, int nchunks, int splits, int64_t split_len, dim3 grid,
                              hipStream_t stream);
hipError_t launch_decode(const tq_codec& kc, const tq_codec& vc, const void* q, int q_dtype,
                         int batch, int n_q, int hq, int hkv, const RopeHost& rope,
                         const tq_packed& k, const tq_packed& v, int64_t ctx, float scale,
                         float* out, float* scores_out, void* workspace, hipStream_t stream);

size_t scan_workspace_bytes(int64_t n_q, int64_t n, int d, int top_k);
hipError_t launch_scan(const tq_codec& c, const void* q, int q_dtype,
                       int64_t n_q, const tq_packed& x, int64_t n, float* out,
                       int top_k, int64_t* top_ids, float* top_scores,
                       void* workspace, hipStream_t stream);

int device_cu_count();

}  // namespace tqk
