// Attention backward for callers that cannot allocate device memory: code
// under hipGraph capture, tight serving loops, harnesses that forbid
// hipMalloc.  It runs the kernels of oases_attention_bwd, with their scratch
// (delta, then the dS matrices) in a file-scope device array instead of a
// workspace argument.
//
// The array lives in the library's code object: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory, so the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/oases_shard.h"
#include "kernels.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)48 << 20;  // 48 MiB per GPU
__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_scratch[MAX_DEVICES];  // device address of `scratch`, per device, once looked up

// Device address of `scratch` on the current device.
hipError_t scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int oases_attention_bwd_noalloc(int32_t nb, int32_t s, int32_t n_h, int32_t d, int32_t causal,
                                           const void *qkv, const void *o, const void *dout, const float *lse,
                                           void *dqkv, void *stream) {
  size_t need = 0;
  if (int r = oases::attention_bwd_validate(nb, s, n_h, d, causal, qkv, o, dout, lse, dqkv, &need)) return r;
  if (need == 0) return OASES_OK;
  if (need > SCRATCH_BYTES)
    return oases::call_fail(OASES_E_ARG, "oases_attention_bwd_noalloc: the problem needs " + std::to_string(need) +
                                             " bytes of scratch; the static scratch holds " +
                                             std::to_string(SCRATCH_BYTES) + " (use oases_attention_bwd)");
  void *p = nullptr;
  const hipError_t e = scratch_on_current_device(&p);
  if (e != hipSuccess)
    return oases::call_fail(OASES_E_HIP, std::string("oases_attention_bwd_noalloc: hipGetSymbolAddress: ") +
                                             hipGetErrorString(e));
  return oases::attention_bwd_call(nb, s, n_h, d, causal, qkv, o, dout, lse, dqkv, p, SCRATCH_BYTES,
                                   static_cast<hipStream_t>(stream));
}
