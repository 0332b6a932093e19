// The decode step without a caller-provided workspace: for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The split partials and balanced
// tile offsets that gqa_decode_step keeps in its workspace live here in one
// file-scope device array of GQA_STATIC_SCRATCH_BYTES per GPU, which every call
// on that GPU shares.  The call allocates nothing.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gqa_decode.h"
#include "gqa_decode_static.h"

// Each GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[GQA_STATIC_SCRATCH_BYTES];

namespace {

// The device address of `scratch` on each GPU, looked up once per device with
// that device current.  In host code the array's name is only a stand-in, so
// kernels and copies must always get this address, never `scratch` itself.
constexpr int kMaxDevices = 256;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

gqa_status_t scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GQA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GQA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GQA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return GQA_OK;
}

}  // namespace

extern "C" gqa_status_t gqa_decode_step_static(const gqa_decode_desc_t* desc, const void* q, void* k_cache,
                                               void* v_cache, const void* k_new, const void* v_new,
                                               const int32_t* lengths, void* out, void* stream) {
  try {
    size_t need = 0;
    gqa_status_t st = gqa_decode_workspace_size(desc, &need);
    if (st != GQA_OK) return st;
    if (need > GQA_STATIC_SCRATCH_BYTES) return GQA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if (need > 0 && desc->batch > 0 && (st = scratch_address(&ws)) != GQA_OK) return st;
    // The kernels need no cleared workspace (every partial they read was
    // written by the same call), so nothing is reset between calls.
    return gqa_decode_step(desc, q, k_cache, v_cache, k_new, v_new, lengths, out, ws,
                           ws != nullptr ? (size_t)GQA_STATIC_SCRATCH_BYTES : 0, stream);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}
