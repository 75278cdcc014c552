// Device-side building blocks shared by the HIP kernels of libmsq (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16 NF4 levels, passed by value in kernel arguments (they land in SGPRs).
struct Nf4Lut {
  float v[16];
};

// Exact quantization thresholds m_i = (L_i + L_{i+1}) / 2 in double.
struct Nf4Mid {
  double m[15];
};

// Dropout description of one projection's LoRA input (see msq_rng_key in msq.h).
struct Dropout {
  uint32_t k0, k1;        // Philox key: seed lo32, hi32
  uint32_t c1, c2, c3;    // counter words 1..3: (layer << 4) | proj, step, micro
  uint32_t threshold;     // keep iff word >= threshold; 0 disables dropout entirely
  float sigma;            // fp32(1 / fp32(1 - p))
};

// fp32 -> bf16 bits, round to nearest even on the 16 dropped bits.  Exact for every
// finite input, subnormals included; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64 multiplies,
// Weyl key schedule between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Keep bits (bit q set = element e0+q kept) of the 4 elements e0..e0+3, e0 % 4 == 0.
__device__ __forceinline__ uint32_t keep4(const Dropout& d, uint64_t e0) {
  if (d.threshold == 0u) return 0xfu;
  const uint4 w = philox4x32_10(make_uint4((uint32_t)(e0 >> 2), d.c1, d.c2, d.c3), d.k0, d.k1);
  return (uint32_t)(w.x >= d.threshold) | ((uint32_t)(w.y >= d.threshold) << 1) |
         ((uint32_t)(w.z >= d.threshold) << 2) | ((uint32_t)(w.w >= d.threshold) << 3);
}

// ---------------------------------------------------------------------------
// NF4 dequantization through a per-block 16-entry bf16 table.
// For one 64-element block with scale a, the table holds bf16_rne(L[c] * a) for the
// 16 codes, split into low-byte and high-byte planes of four dwords each, so that
// one v_perm_b32 looks up four codes at once (selector bytes 0..7 address an
// 8-byte table held in two registers).
struct Nf4Planes {
  uint32_t lo[4], hi[4];
};

// Two floats -> packed bf16 pair (RNE), element a in the low half: one
// v_cvt_pk_bf16_f32 on gfx950 (the vector conversion keeps the pair together).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ Nf4Planes nf4_planes(const Nf4Lut& lut, float a) {
  uint32_t pk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = pack_bf16x2(lut.v[2 * i] * a, lut.v[2 * i + 1] * a);
  Nf4Planes P;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // pk[2i] holds codes 4i, 4i+1; pk[2i+1] holds 4i+2, 4i+3 (bytes lo, hi, lo, hi)
    P.lo[i] = __builtin_amdgcn_perm(pk[2 * i + 1], pk[2 * i], 0x06040200u);
    P.hi[i] = __builtin_amdgcn_perm(pk[2 * i + 1], pk[2 * i], 0x07050301u);
  }
  return P;
}

// sel: four selector bytes whose low nibbles are codes 0..15 (high nibbles are
// ignored).  Returns the four bf16 values as two dwords (element 0 in the low half
// of .x).  Each plane is looked up in both 8-entry halves of the table; a third
// v_perm then takes byte i from the upper half when bit 3 of code i is set.
__device__ __forceinline__ uint2 nf4_lookup4(const Nf4Planes& P, uint32_t sel) {
  const uint32_t s7 = sel & 0x07070707u;
  const uint32_t pick = ((sel >> 1) & 0x04040404u) | 0x03020100u;  // byte i: i, or 4+i if code >= 8
  const uint32_t lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(P.lo[3], P.lo[2], s7),
                                            __builtin_amdgcn_perm(P.lo[1], P.lo[0], s7), pick);
  const uint32_t hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(P.hi[3], P.hi[2], s7),
                                            __builtin_amdgcn_perm(P.hi[1], P.hi[0], s7), pick);
  return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

// Eight codes of one packed dword (bytes b0..b3, even element in the high nibble)
// -> eight bf16 values in four dwords.  u = w >> 4 carries the high nibbles in its
// byte-wise low nibbles, so two v_perm interleave [b0.hi, b0.lo, b1.hi, b1.lo] etc.
__device__ __forceinline__ void nf4_dequant8(const Nf4Planes& P, uint32_t w, uint32_t out[4]) {
  const uint32_t u = w >> 4;
  const uint2 r0 = nf4_lookup4(P, __builtin_amdgcn_perm(w, u, 0x05010400u));
  const uint2 r1 = nf4_lookup4(P, __builtin_amdgcn_perm(w, u, 0x07030602u));
  out[0] = r0.x;
  out[1] = r0.y;
  out[2] = r1.x;
  out[3] = r1.y;
}

// 32 codes (16 packed bytes) of one block -> 32 bf16 values in 16 dwords.
__device__ __forceinline__ void nf4_dequant32(const Nf4Planes& P, uint4 c, uint32_t out[16]) {
  nf4_dequant8(P, c.x, out + 0);
  nf4_dequant8(P, c.y, out + 4);
  nf4_dequant8(P, c.z, out + 8);
  nf4_dequant8(P, c.w, out + 12);
}

}  // namespace msq
