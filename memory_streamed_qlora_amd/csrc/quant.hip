// NF4 quantize / dequantize kernels.
//
// Quantization is a load-time step (the pages' loader quantizes each tensor as it
// is staged: "Poros" research post, the streamed NF4 loader paragraph), so it favours
// exactness over speed: each 64-element block's decisions are exact double-precision
// comparisons w > absmax * m_i against the codebook midpoints.
#include "internal.hpp"

namespace msq {
namespace {

constexpr int QTHREADS = 256;

__global__ __launch_bounds__(QTHREADS) void nf4_quantize_kernel(const uint16_t* __restrict__ w,
                                                                int64_t nblocks,
                                                                uint8_t* __restrict__ codes,
                                                                float* __restrict__ absmax,
                                                                Nf4Mid mid) {
  const int64_t b = (int64_t)blockIdx.x * QTHREADS + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(w + b * 64);
  uint32_t v[32];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 q = src[i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
  // absmax over |w|: bf16 magnitudes order like their bit patterns
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    amax_bits = max(amax_bits, v[i] & 0x7fffu);
    amax_bits = max(amax_bits, (v[i] >> 16) & 0x7fffu);
  }
  const float a = bf16_to_f32(amax_bits);
  uint32_t out[8];
  if (amax_bits == 0u) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = 0x77777777u;
  } else {
    double thr[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) thr[i] = (double)a * mid.m[i];  // exact: 24 x 29 bits
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // element 8i+e
        const uint32_t bits = (e & 1) ? (v[4 * i + e / 2] >> 16) : (v[4 * i + e / 2] & 0xffffu);
        const double x = (double)bf16_to_f32(bits);
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < 15; ++j) c += (x > thr[j]) ? 1u : 0u;
        // byte (e/2) of the dword: element 2p in the high nibble, 2p+1 in the low
        const int byte = e >> 1;
        const int shift = 8 * byte + ((e & 1) ? 0 : 4);
        word |= c << shift;
      }
      out[i] = word;
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  absmax[b] = a;
}

__global__ __launch_bounds__(QTHREADS) void nf4_dequantize_kernel(const uint8_t* __restrict__ codes,
                                                                  const float* __restrict__ absmax,
                                                                  int64_t nchunks,
                                                                  uint16_t* __restrict__ w,
                                                                  Nf4Lut lut) {
  const int64_t c = (int64_t)blockIdx.x * QTHREADS + threadIdx.x;  // chunk of 32 elements
  if (c >= nchunks) return;
  const uint4 q = *reinterpret_cast<const uint4*>(codes + c * 16);
  const Nf4Planes P = nf4_planes(lut, absmax[c >> 1]);
  uint32_t out[16];
  nf4_dequant32(P, q, out);
  uint4* dst = reinterpret_cast<uint4*>(w + c * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
}

}  // namespace

hipError_t launch_quantize(const uint16_t* w, int64_t nblocks, uint8_t* codes, float* absmax,
                           hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks + QTHREADS - 1) / QTHREADS;
  hipLaunchKernelGGL(nf4_quantize_kernel, dim3((unsigned)grid), dim3(QTHREADS), 0, s, w, nblocks,
                     codes, absmax, nf4_mid());
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const float* absmax, int64_t nchunks32,
                             uint16_t* w, hipStream_t s) {
  if (nchunks32 == 0) return hipSuccess;
  const int64_t grid = (nchunks32 + QTHREADS - 1) / QTHREADS;
  hipLaunchKernelGGL(nf4_dequantize_kernel, dim3((unsigned)grid), dim3(QTHREADS), 0, s, codes,
                     absmax, nchunks32, w, nf4_lut());
  return hipGetLastError();
}

}  // namespace msq
