// Attention from codes without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation): the same kernels as tq_attend_decode, with their
// partial-result scratch in a fixed file-scope device array.
//
// Each GPU holds its own copy of `scratch` for the life of the process.  Its
// device address is looked up once per device (the first call made with that
// device current) and kept; host code never passes the array's name, which
// on the host is only a stand-in for the symbol.  Calls that overlap in time
// on one GPU share the array and race; the kernels write every scratch entry
// they read back within the same call, so nothing needs clearing between
// calls.

#include <hip/hip_runtime.h>

#include <mutex>

#include "tq.h"

static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The current device's scratch address (looked up on its first use), or null.
void* device_scratch(int& status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    status = TQ_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    status = TQ_ERR_UNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      status = TQ_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  status = TQ_OK;
  return g_scratch[dev];
}

}  // namespace

extern "C" int tq_attend_decode_noalloc(const tq_codec* kc, const tq_codec* vc, const void* q,
                                        int q_dtype, int batch, int n_q, int hq, int hkv,
                                        const tq_rope* q_rope, const tq_packed* k,
                                        const tq_packed* v, int64_t ctx, float scale, float* out,
                                        float* scores_out, tq_stream_t stream) {
  int status = TQ_OK;
  void* ptr = device_scratch(status);
  if (ptr == nullptr) return status;
  if (kc != nullptr) {
    const size_t need = tq_attend_decode_workspace(batch, n_q, hq, hkv, ctx, kc->d);
    if (need > (size_t)TQ_NOALLOC_SCRATCH_BYTES) return TQ_ERR_TOO_LARGE;
  }
  return tq_attend_decode(kc, vc, q, q_dtype, batch, n_q, hq, hkv, q_rope, k, v, ctx, scale, out,
                          scores_out, ptr, (size_t)TQ_NOALLOC_SCRATCH_BYTES, stream);
}
