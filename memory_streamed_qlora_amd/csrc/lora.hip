// LoRA-side kernels of the fused NF4 + LoRA linear.
//
// The rank-r products of the adapter are skinny (r = 16 against K, N in the
// thousands) and bound by HBM/L2 traffic, not by MFMA:
//   skinny(+reduce)  u = drop(x) A^T  (forward, recompute)  and  du = s dy B  (backward),
//                   tiled over 16 tokens x 512 columns, chunk partials summed in order
//   colgrad(+reduce) dA = du^T drop(x)  and  dB = s dy^T u, reduced over tokens in
//                   fixed-size chunks and then summed in chunk order
//   split_reduce    sums split-reduction partials of the base GEMM in split order and
//                   adds the bias (forward) or the old dx (accumulating backward), then
//                   rounds once to bf16 (or stores fp32); the LoRA term itself is folded
//                   into the GEMM's output tiles.
// Activations may be bf16 or fp32; with fp32 the rank-r products use the fp32
// values and only the MFMA operand of the base product is rounded to bf16.
// Every reduction has a fixed shape-determined order and no atomics, so results are
// bitwise reproducible.  Dropout masks are regenerated from the Philox key wherever
// they are needed; the same key gives the same mask in the forward, the recompute and
// the backward (the pages' RNG replay requirement, "Poros" research post).
#include "internal.hpp"

namespace msq {
namespace {


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

// Skinny product out[t][j] = scale * sum_c h[t][c] * M(c, j) for r <= 64 ranks.
// Workgroup: 16 tokens x SKINNY_CHUNK columns x 16 ranks (grid z over rank groups);
// the input tile (dropout applied while staging) and the matrix chunk are staged in
// LDS, each thread owns one (token, rank) pair and reduces over the chunk; the chunk
// partials go to part[chunk][t][j] and skinny_reduce sums them in chunk order.
constexpr int SK_T = 16, SK_J = 16, SK_LD = SKINNY_CHUNK + 4;

template <typename TIN, int MAT_KIND>
__global__ __launch_bounds__(256) void lora_skinny(const TIN* __restrict__ in, int64_t T, int64_t C,
                                                   const float* __restrict__ mat, int r, Dropout d,
                                                   float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float xs[SK_T * SK_LD];
  __shared__ __attribute__((aligned(16))) float ms[SK_J * SK_LD];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * SK_T;
  const int64_t c0 = (int64_t)blockIdx.y * SKINNY_CHUNK;
  const int j0 = blockIdx.z * SK_J;
  // input tile [16][CHUNK], 4 consecutive columns per load
  for (int idx = tid; idx < SK_T * SKINNY_CHUNK / 4; idx += 256) {
    const int row = idx / (SKINNY_CHUNK / 4), c4 = idx % (SKINNY_CHUNK / 4);
    const int64_t t = t0 + row, c = c0 + 4 * c4;
    float h[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < T && c < C) {
      load4(in + t * C + c, h);
      if (d.threshold != 0u) {
        const uint32_t keep = keep4(d, (uint64_t)t * (uint64_t)C + (uint64_t)c);
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = ((keep >> q) & 1u) ? h[q] * d.sigma : 0.0f;
      }
    }
    *reinterpret_cast<float4*>(&xs[row * SK_LD + 4 * c4]) = make_float4(h[0], h[1], h[2], h[3]);
  }
  // matrix chunk, stored [rank][column]
  if (MAT_KIND == 0) {  // mat [r][C]
    for (int idx = tid; idx < SK_J * SKINNY_CHUNK / 4; idx += 256) {
      const int j = idx / (SKINNY_CHUNK / 4), c4 = idx % (SKINNY_CHUNK / 4);
      const int64_t c = c0 + 4 * c4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + j < r && c < C) v = *reinterpret_cast<const float4*>(mat + (int64_t)(j0 + j) * C + c);
      *reinterpret_cast<float4*>(&ms[j * SK_LD + 4 * c4]) = v;
    }
  } else {  // mat [C][r]
    for (int idx = tid; idx < SK_J * SKINNY_CHUNK; idx += 256) {
      const int c = idx / SK_J, j = idx % SK_J;
      float v = 0.0f;
      if (j0 + j < r && c0 + c < C) v = mat[(c0 + c) * (int64_t)r + j0 + j];
      ms[j * SK_LD + c] = v;
    }
  }
  __syncthreads();
  const int row = tid / SK_J, j = tid % SK_J;
  const float* xr = &xs[row * SK_LD];
  const float* mr = &ms[j * SK_LD];
  float acc = 0.0f;
#pragma unroll 8
  for (int c = 0; c < SKINNY_CHUNK; c += 4) {
    const float4 a = *reinterpret_cast<const float4*>(xr + c);
    const float4 b = *reinterpret_cast<const float4*>(mr + c);
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
  }
  const int64_t t = t0 + row;
  if (t < T && j0 + j < r) part[((int64_t)blockIdx.y * T + t) * r + j0 + j] = acc;
}

__global__ __launch_bounds__(256) void lora_skinny_reduce(const float* __restrict__ part, int nck,
                                                          int64_t n, float scale,
                                                          float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int c = 0; c < nck; ++c) s += part[(int64_t)c * n + i];
  out[i] = scale * s;
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

// out[t][n..n+3] = sum_s P[s][t][n..n+3] (+ bias[n..n+3]) (+ old out), one rounding.
template <typename TOUT>
__global__ __launch_bounds__(256) void split_reduce(const float* __restrict__ part, int splits,
                                                    int64_t T, int64_t N,
                                                    const uint16_t* __restrict__ bias,
                                                    TOUT* __restrict__ out, int accumulate) {
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i4 * 4 >= T * N) return;
  const int64_t o = i4 * 4;
  const int64_t n = o % N;
  const int64_t plane = T * N;
  float a[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(part + s * plane + o);
    a[0] += p.x;
    a[1] += p.y;
    a[2] += p.z;
    a[3] += p.w;
  }
  if (bias) {
    float b[4];
    load4(bias + n, b);
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] += b[q];
  }
  if (accumulate) {
    float old[4];
    load4(out + o, old);
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = old[q] + a[q];
  }
  store4(out + o, a);
}

// Round fp32 activations to bf16 (RNE) for the MFMA operand; 8 per thread.
// Activation operand of the fused GEMM in MFMA-fragment order (see launch_pack_frag).
// One workgroup packs one block of 32 rows x 64 reduction columns: thread t reads
// 8 consecutive elements (row t >> 3, chunk t & 7) with coalesced loads and stores them
// as lane (row + 32 * (chunk >> 2)) of sub-step (chunk & 3).
template <typename TIN>
__global__ __launch_bounds__(256) void pack_frag(const TIN* __restrict__ in, int64_t M, int64_t R, int steps,
                                                 uint16_t* __restrict__ out) {
  const int grp = blockIdx.y, step = blockIdx.x;
  const int t = threadIdx.x, row = t >> 3, chunk = t & 7;
  const int64_t m = (int64_t)grp * 32 + row;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (m < M) {
    float f[8];
    load8(in + m * R + (int64_t)step * 64 + chunk * 8, f);
    v = make_uint4(bf16_rne(f[0]) | (bf16_rne(f[1]) << 16), bf16_rne(f[2]) | (bf16_rne(f[3]) << 16),
                   bf16_rne(f[4]) | (bf16_rne(f[5]) << 16), bf16_rne(f[6]) | (bf16_rne(f[7]) << 16));
  }
  const int lane = row + 32 * (chunk >> 2), c = chunk & 3;
  *reinterpret_cast<uint4*>(out + (((int64_t)grp * steps + step) * 4 + c) * 512 + lane * 8) = v;
}

template <typename TIN, int MAT_KIND>
hipError_t skinny_dispatch(const TIN* in, int64_t T, int64_t C, const float* mat, int r,
                           const Dropout& d, float* part, hipStream_t s) {
  const dim3 grid((unsigned)((T + SK_T - 1) / SK_T), (unsigned)((C + SKINNY_CHUNK - 1) / SKINNY_CHUNK),
                  (unsigned)((r + SK_J - 1) / SK_J));
  hipLaunchKernelGGL((lora_skinny<TIN, MAT_KIND>), grid, dim3(256), 0, s, in, T, C, mat, r, d, part);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(const void* in, bool in_f32, int64_t T, int64_t C, const float* mat,
                         int mat_kind, int r, float scale, const Dropout& d, float* part, float* out,
                         hipStream_t s) {
  if (T == 0 || r == 0) return hipSuccess;
  hipError_t e;
  if (in_f32)
    e = mat_kind == 0 ? skinny_dispatch<float, 0>((const float*)in, T, C, mat, r, d, part, s)
                      : skinny_dispatch<float, 1>((const float*)in, T, C, mat, r, d, part, s);
  else
    e = mat_kind == 0 ? skinny_dispatch<uint16_t, 0>((const uint16_t*)in, T, C, mat, r, d, part, s)
                      : skinny_dispatch<uint16_t, 1>((const uint16_t*)in, T, C, mat, r, d, part, s);
  if (e != hipSuccess) return e;
  const int nck = (int)((C + SKINNY_CHUNK - 1) / SKINNY_CHUNK);
  const int64_t n = T * r;
  hipLaunchKernelGGL(lora_skinny_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, nck,
                     n, scale, out);
  return hipGetLastError();
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

hipError_t launch_split_reduce(const float* part, int splits, int64_t T, int64_t N,
                               const uint16_t* bias, void* out, bool out_f32, int accumulate,
                               hipStream_t s) {
  const int64_t n4 = T * N / 4;
  if (n4 == 0) return hipSuccess;
  const dim3 grid((unsigned)((n4 + 255) / 256));
  if (out_f32)
    hipLaunchKernelGGL(split_reduce<float>, grid, dim3(256), 0, s, part, splits, T, N, bias, (float*)out,
                       accumulate);
  else
    hipLaunchKernelGGL(split_reduce<uint16_t>, grid, dim3(256), 0, s, part, splits, T, N, bias,
                       (uint16_t*)out, accumulate);
  return hipGetLastError();
}

hipError_t launch_pack_frag(const void* in, bool in_f32, int64_t M, int64_t R, uint16_t* out, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int steps = (int)(R / 64);
  const dim3 grid((unsigned)steps, (unsigned)((M + 31) / 32));
  if (in_f32)
    hipLaunchKernelGGL(pack_frag<float>, grid, dim3(256), 0, s, (const float*)in, M, R, steps, out);
  else
    hipLaunchKernelGGL(pack_frag<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)in, M, R, steps, out);
  return hipGetLastError();
}

}  // namespace msq
