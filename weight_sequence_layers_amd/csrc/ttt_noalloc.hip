// The allocation-free sequence call (ttt_sequence_forward_noalloc): for callers that cannot
// allocate device memory -- code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc.  Every workspace buffer of the staged and resident paths is carved
// from one file-scope device array, `scratch`, instead of a state's arena; the fp32 fast
// weights live in the caller's buffer.  Nothing here or below calls hipMalloc or hipFree.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "ttt_internal.h"

namespace {

// The workspace.  Each GPU the library runs on holds its own copy until the process ends;
// every call on that GPU reuses it and finds the previous call's contents.
__device__ __align__(256) char scratch[TTT_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
char* g_scratch[MAX_DEVICES] = {};   // device address of `scratch`, per device

// The device address of `scratch` on the current device, looked up once per device with
// that device current.  In host code the array's name is only a host-side stand-in, so
// every kernel argument is derived from this address.
ttt_status scratch_address(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ttt::report(TTT_E_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return ttt::report(TTT_E_HIP, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[256];
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) failed: %s",
               hipGetErrorString(e));
      return ttt::report(TTT_E_HIP, msg);
    }
    g_scratch[dev] = static_cast<char*>(p);
  }
  *out = g_scratch[dev];
  return TTT_OK;
}

}  // namespace

extern "C" ttt_status ttt_sequence_forward_noalloc(const ttt_config* cfg, float* state,
                                                   const void* q, const void* k, const void* v,
                                                   const float* eta, void* out, int64_t seq_len,
                                                   void* stream) {
  // every host check (configuration, pointers, sizes, workspace limit) before any HIP call
  size_t need = 0;
  ttt_status st = ttt::sequence_in_workspace(cfg, state, q, k, v, eta, out, seq_len, nullptr,
                                             TTT_NOALLOC_SCRATCH_BYTES, &need, stream);
  if (st != TTT_OK) return st;
  char* ws = nullptr;
  if ((st = scratch_address(&ws)) != TTT_OK) return st;
  return ttt::sequence_in_workspace(cfg, state, q, k, v, eta, out, seq_len, ws,
                                    TTT_NOALLOC_SCRATCH_BYTES, &need, stream);
}
