// nf4_lora_fwd_noalloc: the fused NF4 + LoRA forward without a caller workspace.
//
// For callers that cannot allocate device memory at the call (code under stream capture,
// tight serving loops, harnesses that forbid allocation): the split partials, the packed
// activation and the rank-r staging of nf4_lora_fwd live in one file-scope device array
// instead of a caller workspace.  Each GPU holds its own copy of the array from the first
// call on that device until the process ends.  The array's device address is looked up
// once per device with that device current (hipGetSymbolAddress) and only that address is
// handed to the kernels: in host code the array's name is a host-side stand-in, not a
// device address.
#include <mutex>

#include "../../include/msq.h"
#include "internal.hpp"

using namespace msq;

namespace {

constexpr size_t SCRATCH_BYTES = size_t(128) << 20;  // MSQ_NOALLOC_SCRATCH_BYTES
static_assert(SCRATCH_BYTES == MSQ_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// The device address of `scratch` on device `dev`, looked up once with `dev` current.
int scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= MAX_DEVICES)
    return set_error(MSQ_E_INVAL, "nf4_lora_fwd_noalloc: device %d outside [0, %d)", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_error(e, "nf4_lora_fwd_noalloc: hipGetDevice");
    if (cur != dev) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return hip_error(e, "nf4_lora_fwd_noalloc: hipSetDevice");
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_error(e, "nf4_lora_fwd_noalloc: hipGetSymbolAddress(scratch)");
    if (!p || (uintptr_t)p % 256)
      return set_error(MSQ_E_HIP, "nf4_lora_fwd_noalloc: scratch address %p is null or not 256-byte aligned", p);
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MSQ_OK;
}

}  // namespace

extern "C" {

int nf4_lora_fwd_noalloc(const void* x, int64_t t, int64_t k, int64_t n, const uint8_t* codes,
                         const float* absmax, const uint16_t* bias, const void* residual, const float* A,
                         const float* B, msq_lora_cfg cfg, msq_rng_key key, void* y, float* u_out,
                         msq_stream_t stream) {
  // host-only checks first: an invalid call or one too large for the array touches no HIP state
  const size_t need = nf4_lora_workspace_size(t, k, n, cfg.r);
  if (need > SCRATCH_BYTES)
    return set_error(MSQ_E_WORKSPACE,
                     "nf4_lora_fwd_noalloc: t=%lld k=%lld n=%lld r=%d needs %zu bytes of scratch, more than the "
                     "library's static %zu; use nf4_lora_fwd with a caller workspace",
                     (long long)t, (long long)k, (long long)n, cfg.r, need, SCRATCH_BYTES);
  if (need == 0)  // an invalid shape: nf4_lora_fwd reports it before it looks at the workspace
    return nf4_lora_fwd(x, t, k, n, codes, absmax, bias, residual, A, B, cfg, key, y, u_out, nullptr, 0, stream);
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_error(e, "nf4_lora_fwd_noalloc: device of the stream");
  void* ws = nullptr;
  const int rc = scratch_ptr(dev, &ws);
  if (rc) return rc;
  return nf4_lora_fwd(x, t, k, n, codes, absmax, bias, residual, A, B, cfg, key, y, u_out, ws, SCRATCH_BYTES,
                      stream);
}

}  // extern "C"
