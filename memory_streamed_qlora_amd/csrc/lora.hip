// LoRA-side kernels of the fused NF4 + LoRA linear.
//
// The rank-r products of the adapter are skinny (r = 16 against K, N in the
// thousands) and bound by HBM/L2 traffic, not by MFMA:
//   rowdot          u = drop(x) A^T  (forward, recompute)  and  du = s dy B  (backward)
//   colgrad(+reduce) dA = du^T drop(x)  and  dB = s dy^T u, reduced over tokens in
//                   fixed-size chunks and then summed in chunk order
//   epilogues       sum the split-reduction partials of the base GEMM in split order
//                   and add bias and the LoRA term (forward) or the masked LoRA input
//                   gradient (backward), then round once to bf16 (or store fp32).
// Activations may be bf16 or fp32; with fp32 the rank-r products use the fp32
// values and only the MFMA operand of the base product is rounded to bf16.
// Every reduction has a fixed shape-determined order and no atomics, so results are
// bitwise reproducible.  Dropout masks are regenerated from the Philox key wherever
// they are needed; the same key gives the same mask in the forward, the recompute and
// the backward (the pages' RNG replay requirement, "Poros" research post).
#include "internal.hpp"

namespace msq {
namespace {

constexpr int RD_THREADS = 256;

// Activation element types: bf16 bit patterns (uint16_t) or fp32.
// Eight consecutive elements at p (16-byte aligned for bf16, 32 for fp32) -> floats.
__device__ __forceinline__ void load8(const uint16_t* p, float f[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}
__device__ __forceinline__ void load8(const float* p, float f[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float f[4]) {
  const uint2 raw = *reinterpret_cast<const uint2*>(p);
  f[0] = bf16_to_f32(raw.x & 0xffffu);
  f[1] = bf16_to_f32(raw.x >> 16);
  f[2] = bf16_to_f32(raw.y & 0xffffu);
  f[3] = bf16_to_f32(raw.y >> 16);
}
__device__ __forceinline__ void load4(const float* p, float f[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
}
// Four output values at p: one rounding to bf16, or stored as fp32.
__device__ __forceinline__ void store4(uint16_t* p, const float a[4]) {
  *reinterpret_cast<uint2*>(p) =
      make_uint2(bf16_rne(a[0]) | (bf16_rne(a[1]) << 16), bf16_rne(a[2]) | (bf16_rne(a[3]) << 16));
}
__device__ __forceinline__ void store4(float* p, const float a[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(a[0], a[1], a[2], a[3]);
}

// out[t][j] = scale * sum_c h[t][c] * mat(j, c); one workgroup per row t.
template <int RT, int MAT_KIND, typename TIN>
__global__ __launch_bounds__(RD_THREADS) void lora_rowdot(const TIN* __restrict__ in, int64_t C,
                                                          const float* __restrict__ mat, int r,
                                                          float scale, Dropout d,
                                                          float* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  float acc[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) acc[j] = 0.0f;
  const TIN* row = in + t * C;
  for (int64_t c = 8 * (int64_t)tid; c < C; c += 8 * RD_THREADS) {
    float h[8];
    load8(row + c, h);
    if (d.threshold != 0u) {
      const uint64_t e0 = (uint64_t)t * (uint64_t)C + (uint64_t)c;
      const uint32_t keep = keep4(d, e0) | (keep4(d, e0 + 4) << 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = ((keep >> q) & 1u) ? h[q] * d.sigma : 0.0f;
    }
    if (MAT_KIND == 0) {  // mat [r][C]
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        if (j < r) {
          const float4 m0 = *reinterpret_cast<const float4*>(mat + (int64_t)j * C + c);
          const float4 m1 = *reinterpret_cast<const float4*>(mat + (int64_t)j * C + c + 4);
          float s = acc[j];
          s = fmaf(h[0], m0.x, s);
          s = fmaf(h[1], m0.y, s);
          s = fmaf(h[2], m0.z, s);
          s = fmaf(h[3], m0.w, s);
          s = fmaf(h[4], m1.x, s);
          s = fmaf(h[5], m1.y, s);
          s = fmaf(h[6], m1.z, s);
          s = fmaf(h[7], m1.w, s);
          acc[j] = s;
        }
      }
    } else {  // mat [C][r]
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float* mr = mat + (c + q) * (int64_t)r;
#pragma unroll
        for (int j = 0; j < RT; ++j)
          if (j < r) acc[j] = fmaf(h[q], mr[j], acc[j]);
      }
    }
  }
  // wave reduction (butterfly, fixed order), then across the 4 waves in order
  __shared__ float red[RD_THREADS / 64][RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    float v = acc[j];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    acc[j] = v;
  }
  if ((tid & 63) == 0) {
#pragma unroll
    for (int j = 0; j < RT; ++j) red[tid >> 6][j] = acc[j];
  }
  __syncthreads();
  if (tid < r) {
    float v = red[0][tid];
#pragma unroll
    for (int w = 1; w < RD_THREADS / 64; ++w) v += red[w][tid];
    out[t * r + tid] = scale * v;
  }
}

// part[ch][j][c] = sum_{t in chunk} coef[t][j] * h[t][c], for j in [j0, j0+16)
// grid (ceil(C/256), nch, ceil(r/16)), 64 threads, 4 columns per thread.
constexpr int CG_THREADS = 64;
constexpr int CG_J = 16;

template <typename TIN>
__global__ __launch_bounds__(CG_THREADS) void lora_colgrad(const TIN* __restrict__ in, int64_t T,
                                                           int64_t C, const float* __restrict__ coef,
                                                           int r, Dropout d, int tchunk,
                                                           float* __restrict__ part) {
  const int64_t c = ((int64_t)blockIdx.x * CG_THREADS + threadIdx.x) * 4;
  const int ch = blockIdx.y;
  const int j0 = blockIdx.z * CG_J;
  const int64_t t0 = (int64_t)ch * tchunk;
  const int64_t t1 = min(T, t0 + tchunk);
  __shared__ float sc[COLGRAD_TCHUNK][CG_J];
  for (int i = threadIdx.x; i < COLGRAD_TCHUNK * CG_J; i += CG_THREADS) {
    const int tt = i / CG_J, jj = i % CG_J;
    const int64_t t = t0 + tt;
    sc[tt][jj] = (t < t1 && j0 + jj < r) ? coef[t * r + j0 + jj] : 0.0f;
  }
  __syncthreads();
  if (c >= C) return;
  float acc[CG_J][4];
#pragma unroll
  for (int j = 0; j < CG_J; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[j][q] = 0.0f;
  for (int64_t t = t0; t < t1; ++t) {
    float h[4];
    load4(in + t * C + c, h);
    if (d.threshold != 0u) {
      const uint32_t keep = keep4(d, (uint64_t)t * (uint64_t)C + (uint64_t)c);
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = ((keep >> q) & 1u) ? h[q] * d.sigma : 0.0f;
    }
    const int tt = (int)(t - t0);
#pragma unroll
    for (int j = 0; j < CG_J; ++j) {
      const float cj = sc[tt][j];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[j][q] = fmaf(cj, h[q], acc[j][q]);
    }
  }
#pragma unroll
  for (int j = 0; j < CG_J; ++j) {
    if (j0 + j < r) {
      float4 v = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
      *reinterpret_cast<float4*>(part + ((int64_t)ch * r + j0 + j) * C + c) = v;
    }
  }
}

__global__ __launch_bounds__(256) void lora_colgrad_reduce(const float* __restrict__ part, int nch,
                                                           int r, int64_t C, float scale,
                                                           float* __restrict__ out, int64_t sj,
                                                           int64_t sc, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over r*C, c fastest
  if (i >= (int64_t)r * C) return;
  const int64_t j = i / C, c = i % C;
  float s = 0.0f;
  for (int ch = 0; ch < nch; ++ch) s += part[((int64_t)ch * r + j) * C + c];
  s *= scale;
  float* o = out + j * sj + c * sc;
  *o = accumulate ? (*o + s) : s;
}

// y[t][n..n+3] = out(sum_s P + bias + lscale * u[t] . B[n])
template <typename TOUT>
__global__ __launch_bounds__(256) void lora_fwd_epilogue(const float* __restrict__ part, int splits,
                                                         int64_t T, int64_t N,
                                                         const uint16_t* __restrict__ bias,
                                                         const float* __restrict__ u,
                                                         const float* __restrict__ B, int r,
                                                         float lscale, TOUT* __restrict__ y) {
  const int64_t t = blockIdx.y;
  const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (n >= N) return;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(part + ((int64_t)s * T + t) * N + n);
    a[0] += p.x;
    a[1] += p.y;
    a[2] += p.z;
    a[3] += p.w;
  }
  if (bias) {
    const uint2 b = *reinterpret_cast<const uint2*>(bias + n);
    a[0] += bf16_to_f32(b.x & 0xffffu);
    a[1] += bf16_to_f32(b.x >> 16);
    a[2] += bf16_to_f32(b.y & 0xffffu);
    a[3] += bf16_to_f32(b.y >> 16);
  }
  if (r > 0) {
    const float* ur = u + t * r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* br = B + (n + q) * (int64_t)r;
      float l = 0.0f;
      for (int j = 0; j < r; ++j) l = fmaf(ur[j], br[j], l);
      a[q] += lscale * l;
    }
  }
  store4(y + t * N + n, a);
}

// dx[t][k..k+3] = out([dx_old +] (sum_s P + sigma*keep*(du[t] . A[:,k])))
template <typename TOUT>
__global__ __launch_bounds__(256) void lora_bwd_epilogue(const float* __restrict__ part, int splits,
                                                         int64_t T, int64_t K,
                                                         const float* __restrict__ du,
                                                         const float* __restrict__ A, int r,
                                                         Dropout d, TOUT* __restrict__ dx,
                                                         int accumulate) {
  const int64_t t = blockIdx.y;
  const int64_t k = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (k >= K) return;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(part + ((int64_t)s * T + t) * K + k);
    a[0] += p.x;
    a[1] += p.y;
    a[2] += p.z;
    a[3] += p.w;
  }
  if (r > 0) {
    float l[4] = {0.f, 0.f, 0.f, 0.f};
    const float* dur = du + t * r;
    for (int j = 0; j < r; ++j) {
      const float4 av = *reinterpret_cast<const float4*>(A + (int64_t)j * K + k);
      const float dj = dur[j];
      l[0] = fmaf(dj, av.x, l[0]);
      l[1] = fmaf(dj, av.y, l[1]);
      l[2] = fmaf(dj, av.z, l[2]);
      l[3] = fmaf(dj, av.w, l[3]);
    }
    const uint32_t keep = keep4(d, (uint64_t)t * (uint64_t)K + (uint64_t)k);
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] += ((keep >> q) & 1u) ? d.sigma * l[q] : 0.0f;
  }
  TOUT* o = dx + t * K + k;
  if (accumulate) {
    float old[4];
    load4(o, old);
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = old[q] + a[q];
  }
  store4(o, a);
}

// Round fp32 activations to bf16 (RNE) for the MFMA operand; 8 per thread.
__global__ __launch_bounds__(256) void cvt_f32_bf16(const float* __restrict__ in, int64_t n8,
                                                    uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float f[8];
  load8(in + 8 * i, f);
  *reinterpret_cast<uint4*>(out + 8 * i) =
      make_uint4(bf16_rne(f[0]) | (bf16_rne(f[1]) << 16), bf16_rne(f[2]) | (bf16_rne(f[3]) << 16),
                 bf16_rne(f[4]) | (bf16_rne(f[5]) << 16), bf16_rne(f[6]) | (bf16_rne(f[7]) << 16));
}

template <int MAT_KIND, typename TIN>
hipError_t rowdot_dispatch(const TIN* in, int64_t T, int64_t C, const float* mat, int r, float scale,
                           const Dropout& d, float* out, hipStream_t s) {
  const dim3 grid((unsigned)T), block(RD_THREADS);
  if (r <= 16)
    hipLaunchKernelGGL((lora_rowdot<16, MAT_KIND, TIN>), grid, block, 0, s, in, C, mat, r, scale, d, out);
  else if (r <= 32)
    hipLaunchKernelGGL((lora_rowdot<32, MAT_KIND, TIN>), grid, block, 0, s, in, C, mat, r, scale, d, out);
  else
    hipLaunchKernelGGL((lora_rowdot<64, MAT_KIND, TIN>), grid, block, 0, s, in, C, mat, r, scale, d, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rowdot(const void* in, bool in_f32, int64_t T, int64_t C, const float* mat,
                         int mat_kind, int r, float scale, const Dropout& d, float* out, hipStream_t s) {
  if (T == 0 || r == 0) return hipSuccess;
  if (in_f32)
    return mat_kind == 0 ? rowdot_dispatch<0>((const float*)in, T, C, mat, r, scale, d, out, s)
                         : rowdot_dispatch<1>((const float*)in, T, C, mat, r, scale, d, out, s);
  return mat_kind == 0 ? rowdot_dispatch<0>((const uint16_t*)in, T, C, mat, r, scale, d, out, s)
                       : rowdot_dispatch<1>((const uint16_t*)in, T, C, mat, r, scale, d, out, s);
}

hipError_t launch_colgrad(const void* in, bool in_f32, int64_t T, int64_t C, const float* coef, int r,
                          const Dropout& d, int nch, float* part, hipStream_t s) {
  if (T == 0 || r == 0) return hipSuccess;
  const dim3 grid((unsigned)((C / 4 + CG_THREADS - 1) / CG_THREADS), (unsigned)nch,
                  (unsigned)((r + CG_J - 1) / CG_J));
  if (in_f32)
    hipLaunchKernelGGL(lora_colgrad<float>, grid, dim3(CG_THREADS), 0, s, (const float*)in, T, C, coef,
                       r, d, COLGRAD_TCHUNK, part);
  else
    hipLaunchKernelGGL(lora_colgrad<uint16_t>, grid, dim3(CG_THREADS), 0, s, (const uint16_t*)in, T, C,
                       coef, r, d, COLGRAD_TCHUNK, part);
  return hipGetLastError();
}

hipError_t launch_colgrad_reduce(const float* part, int nch, int r, int64_t C, float scale,
                                 float* out, int64_t sj, int64_t sc, int accumulate, hipStream_t s) {
  const int64_t n = (int64_t)r * C;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(lora_colgrad_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                     nch, r, C, scale, out, sj, sc, accumulate);
  return hipGetLastError();
}

hipError_t launch_fwd_epilogue(const float* part, int splits, int64_t T, int64_t N,
                               const uint16_t* bias, const float* u, const float* B, int r,
                               float lscale, void* y, bool out_f32, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((N / 4 + 255) / 256), (unsigned)T);
  if (out_f32)
    hipLaunchKernelGGL(lora_fwd_epilogue<float>, grid, dim3(256), 0, s, part, splits, T, N, bias, u, B,
                       r, lscale, (float*)y);
  else
    hipLaunchKernelGGL(lora_fwd_epilogue<uint16_t>, grid, dim3(256), 0, s, part, splits, T, N, bias, u,
                       B, r, lscale, (uint16_t*)y);
  return hipGetLastError();
}

hipError_t launch_bwd_epilogue(const float* part, int splits, int64_t T, int64_t K,
                               const float* du, const float* A, int r, const Dropout& d,
                               void* dx, bool out_f32, int accumulate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((K / 4 + 255) / 256), (unsigned)T);
  if (out_f32)
    hipLaunchKernelGGL(lora_bwd_epilogue<float>, grid, dim3(256), 0, s, part, splits, T, K, du, A, r,
                       d, (float*)dx, accumulate);
  else
    hipLaunchKernelGGL(lora_bwd_epilogue<uint16_t>, grid, dim3(256), 0, s, part, splits, T, K, du, A,
                       r, d, (uint16_t*)dx, accumulate);
  return hipGetLastError();
}

hipError_t launch_cvt_bf16(const float* in, int64_t n, uint16_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(cvt_f32_bf16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, in, n8, out);
  return hipGetLastError();
}

}  // namespace msq
