// The step's optimizer update over the fp32 adapters: AdamW (decoupled weight decay), the
// reading the training-step paragraph of the "Poros" research post leaves open (it names
// one optimizer step after the backward, identical to a resident run's, and keeps only the
// adapters' optimizer state on the device).
//
// One launch updates up to ADAMW_MAX tensors; workgroup b owns elements
// [ADAMW_CHUNK * j, ADAMW_CHUNK * (j + 1)) of one tensor (j = b - that tensor's first
// workgroup) and reads p, g, m, v once, writing p, m, v once.  Each workgroup also writes
// the sum of g^2 over its elements, summed in a fixed order (per thread, then the wave
// by butterfly, then the four waves in order), so the step's gradient norm costs no
// second pass over the gradients and never depends on timing.
#include <string.h>

#include <algorithm>

#include "internal.hpp"

namespace msq {
namespace {

constexpr int ADAMW_MAX = 16;
constexpr int ADAMW_THREADS = 256;
constexpr int ADAMW_ITERS = 8;
constexpr int64_t ADAMW_CHUNK = (int64_t)ADAMW_THREADS * 4 * ADAMW_ITERS;  // 8192 elements

struct AdamwArgs {
  float* p[ADAMW_MAX];
  const float* g[ADAMW_MAX];
  float* m[ADAMW_MAX];
  float* v[ADAMW_MAX];
  int64_t n[ADAMW_MAX];
  int64_t blk0[ADAMW_MAX + 1];  // first workgroup of each tensor; blk0[nt] = workgroups
  int nt;
  float decay;   // 1 - lr * weight_decay
  float b1c;     // 1 - beta1: m moves this fraction of the way to g
  float b2, b2c; // beta2, 1 - beta2
  float bc2s;    // sqrt(1 - beta2^t)
  float eps;
  float step;    // lr / (1 - beta1^t)
};

// One element: p <- p (1 - lr wd);  m <- m + (1 - b1)(g - m);  v <- b2 v + (1 - b2) g^2;
// p <- p - (lr / (1 - b1^t)) * m / (sqrt(v) / sqrt(1 - b2^t) + eps).
__device__ __forceinline__ void adamw1(float& p, float g, float& m, float& v, const AdamwArgs& a, float& ss) {
  const float gg = g * g;
  ss += gg;
  p = p * a.decay;
  m = m + a.b1c * (g - m);
  v = v * a.b2 + a.b2c * gg;
  const float denom = sqrtf(v) / a.bc2s + a.eps;
  p = p - a.step * (m / denom);
}

__global__ __launch_bounds__(ADAMW_THREADS) void adamw_kernel(AdamwArgs a, float* gsq) {
  const int64_t b = blockIdx.x;
  int i = 0;
  while (i + 1 < a.nt && b >= a.blk0[i + 1]) ++i;  // uniform over the workgroup
  const int64_t n = a.n[i];
  const int64_t base = (b - a.blk0[i]) * ADAMW_CHUNK;
  float* P = a.p[i];
  const float* G = a.g[i];
  float* M = a.m[i];
  float* V = a.v[i];
  float ss = 0.0f;
#pragma unroll
  for (int it = 0; it < ADAMW_ITERS; ++it) {
    const int64_t e = base + ((int64_t)it * ADAMW_THREADS + threadIdx.x) * 4;
    if (e + 4 <= n) {
      float4 p = *reinterpret_cast<const float4*>(P + e);
      const float4 g = *reinterpret_cast<const float4*>(G + e);
      float4 m = *reinterpret_cast<const float4*>(M + e);
      float4 v = *reinterpret_cast<const float4*>(V + e);
      adamw1(p.x, g.x, m.x, v.x, a, ss);
      adamw1(p.y, g.y, m.y, v.y, a, ss);
      adamw1(p.z, g.z, m.z, v.z, a, ss);
      adamw1(p.w, g.w, m.w, v.w, a, ss);
      *reinterpret_cast<float4*>(P + e) = p;
      *reinterpret_cast<float4*>(M + e) = m;
      *reinterpret_cast<float4*>(V + e) = v;
    } else {
      for (int64_t k = e; k < n && k < e + 4; ++k) {
        float p = P[k], m = M[k], v = V[k];
        adamw1(p, G[k], m, v, a, ss);
        P[k] = p;
        M[k] = m;
        V[k] = v;
      }
    }
  }
  if (!gsq) return;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ float wsum[ADAMW_THREADS / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = wsum[0];
    for (int w = 1; w < ADAMW_THREADS / 64; ++w) t += wsum[w];
    gsq[b] = t;
  }
}

}  // namespace

int64_t adamw_workgroups(const int64_t* n, int nt) {
  int64_t w = 0;
  for (int i = 0; i < nt; ++i) w += (n[i] + ADAMW_CHUNK - 1) / ADAMW_CHUNK;
  return w;
}

// Algorithmic bytes: p, g, m, v read once, p, m, v written once (28 B per element).
hipError_t launch_adamw(float* const* p, const float* const* g, float* const* m, float* const* v,
                        const int64_t* n, int nt, const AdamwHyper& h, float* gsq, hipStream_t s) {
  for (int c0 = 0; c0 < nt; c0 += ADAMW_MAX) {
    AdamwArgs a;
    memset(&a, 0, sizeof(a));
    a.nt = std::min(ADAMW_MAX, nt - c0);
    int64_t blocks = 0, elems = 0;
    for (int i = 0; i < a.nt; ++i) {
      a.p[i] = p[c0 + i];
      a.g[i] = g[c0 + i];
      a.m[i] = m[c0 + i];
      a.v[i] = v[c0 + i];
      a.n[i] = n[c0 + i];
      a.blk0[i] = blocks;
      blocks += (a.n[i] + ADAMW_CHUNK - 1) / ADAMW_CHUNK;
      elems += a.n[i];
    }
    a.blk0[a.nt] = blocks;
    a.decay = h.decay;
    a.b1c = h.b1c;
    a.b2 = h.b2;
    a.b2c = h.b2c;
    a.bc2s = h.bc2s;
    a.eps = h.eps;
    a.step = h.step;
    if (blocks == 0) continue;
    char shape[32];
    snprintf(shape, sizeof(shape), "%lld", (long long)elems);
    const hipError_t e = timed_launch("adamw", shape, 0.0, 28.0 * elems, adamw_kernel, dim3((unsigned)blocks),
                                      dim3(ADAMW_THREADS), s, a, gsq);
    if (e != hipSuccess) return e;
    if (gsq) gsq += blocks;
  }
  return hipSuccess;
}

}  // namespace msq
