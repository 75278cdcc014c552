// Pointwise block glue of the Qwen2.5 decoder layer, fused under the pages' rule for
// kernels around the engine ("Poros" README, Roadmap, "The Poros kernel"): only
// pointwise chains whose fused form yields the same per-element values qualify -- the
// SwiGLU multiply, residual adds, rotary with precomputed tables, and here also the
// pointwise tail of RMSNorm (its mean stays an unfused reduction).
//
// Each kernel evaluates exactly the operations of the unfused chain it replaces, in the
// same order and with the same roundings.  Contraction into fused multiply-adds is off
// for this file: the unfused chain rounds every product it stores between kernels.  The
// one multiply-add the unfused chain does fuse -- 1 + g * (1 - s) inside the SiLU
// derivative kernel -- is written out as fmaf; exp is the device expf that the unfused
// element-wise kernels call.  The stack's tests check the equality bit for bit against
// the unfused PyTorch chain.
#include "internal.hpp"

#pragma clang fp contract(off)

namespace msq {
namespace {

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// a = silu(g) * u.  Thread i covers elements 4i .. 4i+3 (16-byte loads; the last thread
// takes the n % 4 tail one element at a time).
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const float* __restrict__ g, const float* __restrict__ u,
                                                         int64_t n, float* __restrict__ a) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  if (e + 4 <= n) {
    const float4 gv = *reinterpret_cast<const float4*>(g + e), uv = *reinterpret_cast<const float4*>(u + e);
    *reinterpret_cast<float4*>(a + e) =
        make_float4(silu(gv.x) * uv.x, silu(gv.y) * uv.y, silu(gv.z) * uv.z, silu(gv.w) * uv.w);
  } else {
    for (int64_t i = e; i < n; ++i) a[i] = silu(g[i]) * u[i];
  }
}

// The backward of a = silu(g) * u, as its two unfused steps compute it:
//   du = da * silu(g)                      (product rule, with the forward's silu(g))
//   t  = da * u                            (product rule)
//   dg = (t * s) * fma(g, 1 - s, 1),  s = 1 / (1 + exp(-g))   (SiLU derivative)
__device__ __forceinline__ void swiglu_grad(float da, float g, float u, float& dg, float& du) {
  du = da * silu(g);
  const float t = da * u;
  const float s = 1.0f / (1.0f + expf(-g));
  dg = (t * s) * __builtin_fmaf(g, 1.0f - s, 1.0f);
}

// dg may be g and du may be u (in place): g, u, dg and du are not declared non-aliasing,
// and each element's inputs are loaded before its outputs are stored.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ da, const float* g,
                                                         const float* u, int64_t n, float* dg, float* du) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  if (e + 4 <= n) {
    const float4 a = *reinterpret_cast<const float4*>(da + e), gv = *reinterpret_cast<const float4*>(g + e),
                 uv = *reinterpret_cast<const float4*>(u + e);
    float4 rg, ru;
    swiglu_grad(a.x, gv.x, uv.x, rg.x, ru.x);
    swiglu_grad(a.y, gv.y, uv.y, rg.y, ru.y);
    swiglu_grad(a.z, gv.z, uv.z, rg.z, ru.z);
    swiglu_grad(a.w, gv.w, uv.w, rg.w, ru.w);
    *reinterpret_cast<float4*>(dg + e) = rg;
    *reinterpret_cast<float4*>(du + e) = ru;
  } else {
    for (int64_t i = e; i < n; ++i) {
      const float a = da[i], gv = g[i], uv = u[i];
      float rg, ru;
      swiglu_grad(a, gv, uv, rg, ru);
      dg[i] = rg;
      du[i] = ru;
    }
  }
}

// Rotary embedding, rotate-half pairs (i, i + D/2), tables cos/sin [T][D]:
//   y1 = x1 * c1 + (-x2) * s1,   y2 = x2 * c2 + x1 * s2
// x, y are [T][H][D].  One thread per (t, h, i < D/2).
__global__ __launch_bounds__(256) void rope_fwd_kernel(const float* __restrict__ x, const float* __restrict__ cs,
                                                       const float* __restrict__ sn, int64_t T, int H, int D,
                                                       float* __restrict__ y) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * H * half) return;
  const int i = (int)(idx % half);
  const int64_t th = idx / half;  // t * H + h
  const int64_t t = th / H;
  const float* xr = x + th * D;
  const float* cr = cs + t * D;
  const float* sr = sn + t * D;
  const float x1 = xr[i], x2 = xr[i + half];
  y[th * D + i] = x1 * cr[i] + (-x2) * sr[i];
  y[th * D + i + half] = x2 * cr[i + half] + x1 * sr[i + half];
}

// Its backward: each input element collects the direct term and the rotated term,
//   dx1 = dy1 * c1 + dy2 * s2,   dx2 = dy2 * c2 + (-(dy1 * s1))
__global__ __launch_bounds__(256) void rope_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ cs,
                                                       const float* __restrict__ sn, int64_t T, int H, int D,
                                                       float* __restrict__ dx) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * H * half) return;
  const int i = (int)(idx % half);
  const int64_t th = idx / half;
  const int64_t t = th / H;
  const float* gr = dy + th * D;
  const float* cr = cs + t * D;
  const float* sr = sn + t * D;
  const float g1 = gr[i], g2 = gr[i + half];
  dx[th * D + i] = g1 * cr[i] + g2 * sr[i + half];
  dx[th * D + i + half] = g2 * cr[i + half] + (-(g1 * sr[i]));
}

// RMSNorm's pointwise tail, with r[t] = rsqrt(mean_c h[t][c]^2 + eps) formed outside (a
// reduction, left unfused):  y = (h * r) * w.  Its backward, as the two unfused products'
// gradients compute it: g = dy * w, dh = g * r, hdot = g * h (hdot is summed over c by the
// caller into dr).  Rows of d elements, d % 4 == 0; thread i covers elements 4i .. 4i+3.
__global__ __launch_bounds__(256) void rmsnorm_apply_fwd_kernel(const float* __restrict__ h,
                                                                const float* __restrict__ r,
                                                                const float* __restrict__ w, int64_t n, int64_t d,
                                                                float* __restrict__ y) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  const float rt = r[e / d];
  const float4 hv = *reinterpret_cast<const float4*>(h + e);
  const float4 wv = *reinterpret_cast<const float4*>(w + e % d);
  *reinterpret_cast<float4*>(y + e) =
      make_float4((hv.x * rt) * wv.x, (hv.y * rt) * wv.y, (hv.z * rt) * wv.z, (hv.w * rt) * wv.w);
}

__global__ __launch_bounds__(256) void rmsnorm_apply_bwd_kernel(const float* __restrict__ dy,
                                                                const float* __restrict__ h,
                                                                const float* __restrict__ r,
                                                                const float* __restrict__ w, int64_t n, int64_t d,
                                                                float* __restrict__ dh, float* __restrict__ hdot) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  const float rt = r[e / d];
  const float4 gv = *reinterpret_cast<const float4*>(dy + e);
  const float4 hv = *reinterpret_cast<const float4*>(h + e);
  const float4 wv = *reinterpret_cast<const float4*>(w + e % d);
  const float4 g = make_float4(gv.x * wv.x, gv.y * wv.y, gv.z * wv.z, gv.w * wv.w);
  *reinterpret_cast<float4*>(dh + e) = make_float4(g.x * rt, g.y * rt, g.z * rt, g.w * rt);
  *reinterpret_cast<float4*>(hdot + e) = make_float4(g.x * hv.x, g.y * hv.y, g.z * hv.z, g.w * hv.w);
}

}  // namespace

// Algorithmic bytes: each fp32 operand read once and each result written once.
hipError_t launch_swiglu_fwd(const float* g, const float* u, int64_t n, float* a, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  char shape[32];
  snprintf(shape, sizeof(shape), "%lld", (long long)n);
  return timed_launch("swiglu_fwd", shape, 0.0, 12.0 * n, swiglu_fwd_kernel,
                      dim3((unsigned)(((n + 3) / 4 + 255) / 256)), dim3(256), s, g, u, n, a);
}

hipError_t launch_swiglu_bwd(const float* da, const float* g, const float* u, int64_t n, float* dg, float* du,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  char shape[32];
  snprintf(shape, sizeof(shape), "%lld", (long long)n);
  return timed_launch("swiglu_bwd", shape, 0.0, 20.0 * n, swiglu_bwd_kernel,
                      dim3((unsigned)(((n + 3) / 4 + 255) / 256)), dim3(256), s, da, g, u, n, dg, du);
}

hipError_t launch_rope(bool backward, const float* x, const float* cs, const float* sn, int64_t T, int H, int D,
                       float* y, hipStream_t s) {
  const int64_t n = T * H * (D / 2);
  if (n == 0) return hipSuccess;
  char shape[32];
  snprintf(shape, sizeof(shape), "%lldx%dx%d", (long long)T, H, D);
  const double bytes = 8.0 * T * H * D + 8.0 * T * D;
  const dim3 grid((unsigned)((n + 255) / 256));
  return backward ? timed_launch("rope_bwd", shape, 0.0, bytes, rope_bwd_kernel, grid, dim3(256), s, x, cs, sn, T, H,
                                 D, y)
                  : timed_launch("rope_fwd", shape, 0.0, bytes, rope_fwd_kernel, grid, dim3(256), s, x, cs, sn, T, H,
                                 D, y);
}

hipError_t launch_rmsnorm_apply(bool backward, const float* dy, const float* h, const float* r, const float* w,
                                int64_t T, int64_t D, float* out, float* hdot, hipStream_t s) {
  const int64_t n = T * D;
  if (n == 0) return hipSuccess;
  char shape[32];
  snprintf(shape, sizeof(shape), "%lldx%lld", (long long)T, (long long)D);
  const dim3 grid((unsigned)((n / 4 + 255) / 256));
  if (backward)
    return timed_launch("rmsnorm_apply_bwd", shape, 0.0, 16.0 * n + 4.0 * (T + D), rmsnorm_apply_bwd_kernel, grid,
                        dim3(256), s, dy, h, r, w, n, D, out, hdot);
  return timed_launch("rmsnorm_apply_fwd", shape, 0.0, 8.0 * n + 4.0 * (T + D), rmsnorm_apply_fwd_kernel, grid,
                      dim3(256), s, h, r, w, n, D, out);
}

}  // namespace msq
