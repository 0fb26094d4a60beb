// noalloc.hip -- attn_bwd_noalloc: attn_bwd for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  attn_bwd's one
// scratch buffer, Delta (B*H*Sq floats, written in full by the Delta pre-pass before the gradient
// kernels read it), lives here in a file-scope device array instead of a caller workspace.
//
// The array's name is a host-side stand-in in host code, not a device address: the address is
// taken once per device with hipGetSymbolAddress (with that device current) and only that
// address is passed to kernels.  Each device holds its own copy until the process ends.  Every
// call on a device shares that device's copy, so calls that overlap on one device race.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "tha.h"
#include "tha_kernels.h"

namespace {

constexpr int64_t kScratchFloats = THA_NOALLOC_MAX_DELTA;  // 16 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // per-device address of `scratch`, set on the first call there

// Address of the current device's scratch array (nullptr on failure).
float* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return (float*)g_scratch[dev];
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, float* dq, float* dk, float* dv, int B, int Sq, int Sk, int H, int D,
                                int in_dt, unsigned mask_flags, long long q_pos0, long long k_pos0,
                                const int* kv_len, float scale, void* stream) {
  // Every argument check of attn_bwd first, then the capacity check; both before any HIP call.
  const int rc = tha::attn_bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, Sq, Sk, H, D, in_dt, mask_flags, q_pos0,
                                     k_pos0, kv_len, scale);
  if (rc != THA_OK) return rc;
  if ((int64_t)B * H * Sq > kScratchFloats) return THA_ERR_TOO_LARGE;
  float* delta = device_scratch();
  if (!delta) return THA_ERR_HIP;
  return tha::attn_bwd_launch(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Sq, Sk, H, D, in_dt, mask_flags, q_pos0,
                              k_pos0, kv_len, scale, stream);
}
