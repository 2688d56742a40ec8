// sep_attn_prefill_backward_noalloc: the prefill backward with its delta
// workspace taken from a fixed device array instead of caller memory, for
// callers that cannot allocate (code under HIP graph capture, serving loops
// that forbid allocation).
//
// The array lives in the library's code object, one copy per GPU, for the
// life of the process. Host code never passes the array's name to a kernel
// (in host code that name is a stand-in, not a device address): the device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and kept.
#include <mutex>

#include "internal.hpp"
#include "sepattn.h"

namespace {

// delta needs one float per query row: B * Hq * S <= SEP_NOALLOC_MAX_ROWS.
static __device__ __align__(256) float scratch[SEP_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call from that device).
int scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SEP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SEP_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return SEP_OK;
}

}  // namespace

extern "C" int sep_attn_prefill_backward_noalloc(const void* q, const void* k, const void* v, const void* out,
                                                 const void* dout, const float* lse, int dtype, int B, int Hq,
                                                 int Hkv, int S, int D, const uint8_t* is_sep, const int32_t* rank,
                                                 const int32_t* sep_pos, int a, int n, float scale, float* dq,
                                                 float* dk, float* dv, hipStream_t stream) {
  int st = sep::check_backward_args(q, k, v, out, dout, lse, dtype, B, Hq, Hkv, S, D, is_sep, rank, sep_pos, a, n,
                                    scale, dq, dk, dv);
  if (st != SEP_OK) return st;
  const int64_t heads = static_cast<int64_t>(B) * Hq;            // both factors are positive here
  if (heads > SEP_NOALLOC_MAX_ROWS || heads * S > SEP_NOALLOC_MAX_ROWS) return SEP_ERR_WORKSPACE;
  float* delta = nullptr;
  st = scratch_on_current_device(&delta);
  if (st != SEP_OK) return st;
  // delta is written in full by the backward's first kernel before any
  // kernel reads it, so nothing here needs clearing between calls
  const hipError_t e = sep::launch_prefill_backward(q, k, v, out, dout, lse, dtype, B, Hq, Hkv, S, D, is_sep, rank,
                                                    sep_pos, a, n, scale, delta, dq, dk, dv, stream);
  return e == hipSuccess ? SEP_OK : SEP_ERR_HIP;
}
