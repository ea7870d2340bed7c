// Query preparation (q_rot = Pi RoPE(q), Sq = S q_rot) shared by attention
// and the inner-product scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.hpp"

namespace tqk {

struct QPrepParams {
  const void* q;
  int64_t n_rows;     // query rows to prepare
  int64_t n_q;        // queries per (batch, head): position of row r is pos0 + r % n_q
  int32_t pos0;
  uint32_t flip[48];
  const float* S;     // NULL: no Sq
  float* qrot;        // [n_rows][d]
  float* sq;          // [n_rows][d]
  float inv_sqrt_d;
  double theta[64];
};

hipError_t launch_qprep(const tq_codec& c, const void* q, int q_dtype, int64_t n_rows,
                        int64_t n_q, const RopeHost& rope, float* qrot, float* sq,
                        hipStream_t stream);

}  // namespace tqk
