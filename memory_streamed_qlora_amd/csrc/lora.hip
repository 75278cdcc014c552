// LoRA-side kernels of the fused NF4 + LoRA linear.
//
// The rank-r products of the adapter are skinny (r = 16 against K, N in the
// thousands) and bound by HBM/L2 traffic, not by MFMA:
//   pack_lora(+reduce) one coalesced pass over an activation that writes its bf16 copy
//                   in MFMA-fragment order for the base GEMM and forms the rank-r product
//                   u = drop(x) A^T (forward, recompute) or du = s dy B (backward) in
//                   LORA_CHUNK-column partials, summed in chunk order
//   colgrad(+reduce) dA = du^T drop(x)  and  dB = s dy^T u, reduced over tokens in
//                   fixed-size chunks and then summed in chunk order
//   split_reduce    sums split-reduction partials of the base GEMM in split order,
//                   adds the bias (forward), then adds that to a residual (forward) or
//                   to the old dx (accumulating backward), and rounds once to bf16 (or
//                   stores fp32); the LoRA term itself is folded into the GEMM's output
//                   tiles.
// Activations may be bf16 or fp32.  The rank-r products keep fp32 accuracy: in the
// packing pass they run on the MFMA with each fp32 operand split into bf16 hi and lo
// parts, in the column gradients as fp32 FMAs; only the base product's MFMA operand is
// rounded to bf16.
// Every reduction has a fixed shape-determined order and no atomics, so results are
// bitwise reproducible.  Dropout masks are regenerated from the Philox key wherever
// they are needed; the same key gives the same mask in the forward, the recompute and
// the backward (the pages' RNG replay requirement, "Poros" research post).
#include <string.h>

#include <algorithm>

#include "internal.hpp"
#include "split_bf16.hpp"

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
// The values a store4 to an output of p's type would hold (the pointer only selects it).
__device__ __forceinline__ void round4(const uint16_t*, float a[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) a[q] = bf16_to_f32(bf16_rne(a[q]));
}
__device__ __forceinline__ void round4(const float*, float[4]) {}

// Packing pass over up to GEMM_MAX_SEGS activations [T][C_i] (bf16 or fp32) in one launch,
// fused with the rank-r products that read them (each its own adapter and dropout mask).
// Grid x runs over the LORA_CHUNK-column chunks of the inputs in turn (input i owns x in
// [blk0_i, blk0_i + nck_i)), y over 32-row token groups, z over (product of the input,
// rank group of 16).  One workgroup covers 32 rows x LORA_CHUNK columns (4 k-steps of 64)
// of one input, one product and its ranks j0..j0+15.  Wave w takes the 16 rows from
// 16 (w & 1) and the k-steps 2 (w >> 1), 2 (w >> 1) + 1; its lane (r16, kg) loads the 8
// columns 32 kb + 8 kg .. of row r16 in both 32-column halves kb of each k-step
// (coalesced), and
//   - writes them as bf16 in MFMA-fragment order (z == 0 only, if `packed`): lane
//     (row + 32 kb) of sub-step kg, k-step pstep0_i + step of its group;
//   - multiplies them, masked by the projection's dropout (the rank-r copy only), with
//     the adapter chunk staged in LDS rank-major: they are the A operand of a 16 x 16 x 32
//     bf16 MFMA whose B operand is 8 consecutive columns of one rank row, each fp32
//     operand split into bf16 hi and lo parts (hi*hi + hi*lo + lo*hi);
// then the two waves of a row block add their fp32 results in k order and scale the sum
// by the dropout's 1 / (1 - p), and the chunk partial goes to the projection's
// part[chunk][t][j]; lora_skinny_reduce sums the chunks in order.
constexpr int PK_STEPS = LORA_CHUNK / 64;

struct PackSeg {
  const void* in;
  int64_t C;
  int steps, blk0, pstep0, prod0, nprod;
};
struct PackProj {
  const float* mat;
  float* part;
  Dropout d;
};
struct PackArgs {
  int64_t T;
  int r, rgroups, nseg;
  uint16_t* packed;
  int pstride;
  PackSeg s[GEMM_MAX_SEGS];
  PackProj p[GEMM_MAX_SEGS];
};

template <typename TIN, int MAT_KIND>
__global__ __launch_bounds__(256) void pack_lora(PackArgs a) {
  __shared__ __attribute__((aligned(16))) float ms[16][LORA_CHUNK + 4];
  const int64_t T = a.T;
  const int r = a.r;
  // input, product and rank group of this workgroup (uniform); argument fields are picked
  // at constant indices
  const int bx = blockIdx.x;
  const int si = (a.nseg > 2 && bx >= a.s[2].blk0) ? 2 : (a.nseg > 1 && bx >= a.s[1].blk0) ? 1 : 0;
  PackSeg sg = a.s[0];
  if (si == 1) sg = a.s[1];
  if (si == 2) sg = a.s[2];
  const int zp = (int)blockIdx.z / a.rgroups, rg = (int)blockIdx.z % a.rgroups;
  if (r > 0 && zp >= sg.nprod) return;
  const int pi = sg.prod0 + zp;
  const float* __restrict__ mat = pi == 0 ? a.p[0].mat : pi == 1 ? a.p[1].mat : a.p[2].mat;
  float* __restrict__ part = pi == 0 ? a.p[0].part : pi == 1 ? a.p[1].part : a.p[2].part;
  Dropout d = a.p[0].d;
  if (pi == 1) d = a.p[1].d;
  if (pi == 2) d = a.p[2].d;
  const TIN* __restrict__ in = (const TIN*)sg.in;
  const int64_t C = sg.C;
  const int steps = sg.steps;
  uint16_t* __restrict__ packed = zp == 0 ? a.packed : nullptr;
  const int pstride = a.pstride, pstep0 = sg.pstep0;
  // Lane (r16, kg) of wave w: row 16 (w & 1) + r16 of the group, k-steps 2 (w >> 1) and
  // 2 (w >> 1) + 1 of the chunk, in each the columns 32 kb + 8 kg .. + 7 of both halves kb:
  // exactly the A operand of a 16 x 16 x 32 MFMA (row r16, k-group kg), and a 16-byte piece
  // of the packed fragment (lane row + 32 kb, sub-step kg).
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4, rb = wave & 1, kh = wave >> 1;
  const int grp = blockIdx.y, chunk = bx - sg.blk0, s0 = chunk * PK_STEPS;
  const int nst = min(PK_STEPS, steps - s0);
  const int j0 = rg * 16;
  const int row = 16 * rb + r16;
  const int64_t m = (int64_t)grp * 32 + row, mc = min(m, T - 1);
  const bool mrow = m < T;
  const int64_t c0 = (int64_t)s0 * 64;
  // this lane's activation loads first, so that their latency overlaps the staging of the
  // adapter chunk below (k-steps past the chunk and rows past T re-read valid ones; their
  // values are replaced by zeros)
  float fx[2][2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      load8(in + mc * C + (int64_t)(s0 + min(2 * kh + b, nst - 1)) * 64 + 32 * kb + 8 * kg, fx[b][kb]);
  if (r > 0) {
    // the chunk of the adapter, staged rank-major: every load issued before any LDS store
    const int ncol = nst * 64;
    if (MAT_KIND == 0) {  // mat [r][C]: 4 float4 per thread
      constexpr int NV = 16 * LORA_CHUNK / 4 / 256;
      float4 v[NV];
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int idx = tid + 256 * q, j = idx / (LORA_CHUNK / 4), c4 = 4 * (idx % (LORA_CHUNK / 4));
        v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j0 + j < r && c4 < ncol) v[q] = *reinterpret_cast<const float4*>(mat + (int64_t)(j0 + j) * C + c0 + c4);
      }
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int idx = tid + 256 * q, j = idx / (LORA_CHUNK / 4), c4 = 4 * (idx % (LORA_CHUNK / 4));
        *reinterpret_cast<float4*>(&ms[j][c4]) = v[q];
      }
    } else {  // mat [C][r]: 16 values per thread
      constexpr int NV = 16 * LORA_CHUNK / 256;
      float v[NV];
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int idx = tid + 256 * q, c = idx / 16, j = idx % 16;
        v[q] = (j0 + j < r && c < ncol) ? mat[(c0 + c) * (int64_t)r + j0 + j] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < NV; ++q) {
        const int idx = tid + 256 * q, c = idx / 16, j = idx % 16;
        ms[j][c] = v[q];
      }
    }
    __syncthreads();
  }
  // the product over this wave's 128 columns: per 32-column block one MFMA per pair of
  // bf16 parts (x hi and lo, the adapter's hi and lo; x lo is zero for bf16 inputs and
  // skipped), accumulated in fp32
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int sl = 2 * kh + b;  // k-step within the chunk (uniform per wave)
    const bool sok = sl < nst;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (sok && mrow) ? fx[b][kb][e] : 0.0f;
      if (packed && sok) {
        const uint4 v = make_uint4(bf16_rne(f[0]) | (bf16_rne(f[1]) << 16), bf16_rne(f[2]) | (bf16_rne(f[3]) << 16),
                                   bf16_rne(f[4]) | (bf16_rne(f[5]) << 16), bf16_rne(f[6]) | (bf16_rne(f[7]) << 16));
        *reinterpret_cast<uint4*>(packed + (((int64_t)grp * pstride + pstep0 + s0 + sl) * 4 + kg) * 512 +
                                  (row + 32 * kb) * 8) = v;
      }
      if (r > 0 && sok) {  // uniform
        const int cl = sl * 64 + 32 * kb + 8 * kg;
        if (d.threshold != 0u && mrow) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t keep = keep4(d, (uint64_t)m * (uint64_t)C + (uint64_t)(c0 + cl + 4 * h));
#pragma unroll
            for (int q = 0; q < 4; ++q) f[4 * h + q] = ((keep >> q) & 1u) ? f[4 * h + q] : 0.0f;
          }
        }
        const float4 a0 = *reinterpret_cast<const float4*>(&ms[r16][cl]);
        const float4 a1 = *reinterpret_cast<const float4*>(&ms[r16][cl + 4]);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        bf16x8_t xh, xl, ah, al;
        split8_bf16(f, xh, xl);
        split8_bf16(av, ah, al);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, ah, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, al, acc, 0, 0, 0);
        if (sizeof(TIN) == 4) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, ah, acc, 0, 0, 0);
      }
    }
  }
  if (r == 0) return;
  // the two waves of a row block (k-step pairs 0 and 1) summed in that order; the dropout
  // scale applied once to the sum.  Lane (r16, kg) holds rank r16 of rows 4 kg .. 4 kg + 3.
  __shared__ f32x4_t red[2][64];
  if (kh == 1) red[rb][lane] = acc;
  __syncthreads();
  if (kh == 1) return;
  const f32x4_t o = red[rb][lane];
  const float sc = d.threshold != 0u ? d.sigma : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t mi = (int64_t)grp * 32 + 16 * rb + 4 * kg + i;
    const float v = (acc[i] + o[i]) * sc;
    if (mi < T && j0 + r16 < r) part[((int64_t)chunk * T + mi) * r + j0 + r16] = v;
  }
}

// out[i] = scale * sum_c part[c][i] for i < n, for up to GEMM_MAX_SEGS products (grid y).
// A workgroup owns 64 outputs; its four waves sum four contiguous ranges of chunks in order
// (loads issued ahead of the adds) and the four range sums are added in range order, so
// the result is fixed.
struct ReduceTask {
  const float* part;
  float* out;
  float scale;
  int nck;
};
struct ReduceArgs {
  ReduceTask t[GEMM_MAX_SEGS];
  int64_t n;
};

__global__ __launch_bounds__(256) void lora_skinny_reduce(ReduceArgs ra) {
  __shared__ float red[4][64];
  const int ti = blockIdx.y;
  const float* __restrict__ part = ti == 0 ? ra.t[0].part : ti == 1 ? ra.t[1].part : ra.t[2].part;
  float* __restrict__ out = ti == 0 ? ra.t[0].out : ti == 1 ? ra.t[1].out : ra.t[2].out;
  const float scale = ti == 0 ? ra.t[0].scale : ti == 1 ? ra.t[1].scale : ra.t[2].scale;
  const int nck = ti == 0 ? ra.t[0].nck : ti == 1 ? ra.t[1].nck : ra.t[2].nck;
  const int64_t n = ra.n;
  const int g = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int q = (nck + 3) / 4, c0 = g * q, c1 = min(nck, c0 + q);
  float s = 0.0f;
  if (i < n) {
    int c = c0;
    for (; c + 4 <= c1; c += 4) {
      const float a0 = part[(int64_t)c * n + i], a1 = part[(int64_t)(c + 1) * n + i];
      const float a2 = part[(int64_t)(c + 2) * n + i], a3 = part[(int64_t)(c + 3) * n + i];
      s += a0;
      s += a1;
      s += a2;
      s += a3;
    }
    for (; c < c1; ++c) s += part[(int64_t)c * n + i];
  }
  red[g][threadIdx.x & 63] = s;
  __syncthreads();
  if (g == 0 && i < n) out[i] = scale * (((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x]);
}

// Column gradients of the LoRA factors, several in one launch:
//   task i: out_i[j][c] (or out_i[c][j]) = [out_i +] scale_i * sum_t coef_i[t][j] * h_i[t][c],
//   h_i = drop_i(in_i), j < r, c < C_i
// (dA = du^T drop(x) with out [r][K]; dB = s dy^T u with out [N][r]).  A workgroup owns
// 16 columns (narrow) or 64 (wide) of one task and 16 ranks over all T tokens, so nothing
// is written twice and no second pass sums partials.  The product is a 16 x 16 x 32 bf16
// MFMA per (16-column block, 32-token block): A = the coefficients transposed (ranks x
// tokens, staged in LDS CG_TB tokens at a time), B = the inputs (tokens x columns, each
// wave staging its own 32-token tile in LDS after a coalesced load, the next tile's loads
// in flight meanwhile), fp32 operands split into bf16 hi and lo parts (hi*hi + lo*hi +
// hi*lo; an input's lo part is zero for bf16 inputs and skipped).  Token block b goes to
// wave b mod 4, and the four waves' sums are added in wave order: both widths run every
// output's products and sums in the same order, so a task's result does not depend on the
// width or on the other tasks of the launch.  The dropout mask zeroes inputs where they
// are staged; its 1 / (1 - p) is applied with the task's scale.
constexpr int CG_J = 16;
constexpr int CG_TB = 512;  // tokens whose coefficients are staged in LDS at a time
constexpr int CG_KB = 32;   // tokens of one MFMA k-block
constexpr int CG_CTP = CG_TB + 4;  // LDS pitch of a transposed coefficient row (floats)

// Workgroup width of a launch: 64 columns when its tasks give enough 64-column workgroups
// to fill the chip, else 16.
inline bool colgrad_wide(int64_t ctot) { return ctot / 64 >= 512; }

struct CgTaskDev {
  const void* in;
  const float* coef;
  float* out;
  int64_t C;
  float scale;
  int out_cr;
  int block0;  // first workgroup of the task (blockIdx.x)
  Dropout d;
};
struct CgArgs {
  CgTaskDev t[COLGRAD_MAX_TASKS];
  int ntask;
  int64_t T;
  int r;
  int accumulate;
};

// The input tile of one k-block as loaded: 32 tokens x COLS columns in 16-byte pieces.
template <typename TIN, int COLS>
struct CgTile {
  static constexpr int EP = 16 / (int)sizeof(TIN);  // elements per piece
  static constexpr int LPR = COLS / EP;              // lanes per token row
  static constexpr int RPI = 64 / LPR;               // token rows per 64-lane load
  static constexpr int NP = CG_KB / RPI;             // pieces per lane
  static constexpr int PITCH = COLS + 2;             // fp32 LDS pitch (8-byte aligned rows)
};

// VEC: r % 4 == 0 and every task's coefficient rows 16-byte aligned (float4 staging loads);
// WIDE: 64 columns per workgroup.  Template parameters, so that every load in the token
// loop is unconditional and the compiler counts them exactly.
template <typename TIN, bool VEC, bool WIDE>
__global__ __launch_bounds__(256) void lora_colgrad(CgArgs a) {
  constexpr int COLS = WIDE ? 64 : 16, NCB = COLS / 16;
  using TL = CgTile<TIN, COLS>;
  __shared__ __attribute__((aligned(16))) float ct[CG_J * CG_CTP];  // [rank][token]
  // per wave: its input tile [token][column] in the loop; after it, the partial sums
  __shared__ __attribute__((aligned(16))) float wt[4 * CG_KB * TL::PITCH > 4 * NCB * 4 * 64 ? 4 * CG_KB * TL::PITCH
                                                                                           : 4 * NCB * 4 * 64];
  // this workgroup's task (uniform): the last one whose first block is at or before it,
  // its fields picked at constant indices
  CgTaskDev tk = a.t[0];
#pragma unroll
  for (int i = 1; i < COLGRAD_MAX_TASKS; ++i)
    if (i < a.ntask && (int)blockIdx.x >= a.t[i].block0) tk = a.t[i];
  const TIN* in = (const TIN*)tk.in;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int64_t cbase = (int64_t)((int)blockIdx.x - tk.block0) * COLS;
  const int j0 = blockIdx.y * CG_J;
  const int r = a.r;
  const int64_t T = a.T, C = tk.C;
  const bool drop = tk.d.threshold != 0u;
  float* tile = wt + wave * CG_KB * TL::PITCH;
  // this lane's pieces: token row p * RPI + lane / LPR of the k-block, columns
  // (lane % LPR) * EP .. + EP - 1 of the workgroup's
  const int prow = lane / TL::LPR, pcol = (lane % TL::LPR) * TL::EP;

  f32x4_t acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 qa[TL::NP], qb[TL::NP];
  // k-block kb of the staging block at tb0 (past the tokens: the last token again)
  auto load = [&](u32x4 (&q)[TL::NP], int64_t tb0, int kb) {
#pragma unroll
    for (int p = 0; p < TL::NP; ++p) {
      const int64_t t = min(tb0 + (int64_t)kb * CG_KB + p * TL::RPI + prow, T - 1);
      q[p] = *reinterpret_cast<const u32x4*>(in + t * C + cbase + pcol);
    }
  };
  // the pieces into the wave's tile as fp32: zero past T, masked by the dropout
  auto stage = [&](const u32x4 (&q)[TL::NP], int64_t tb0, int kb) {
#pragma unroll
    for (int p = 0; p < TL::NP; ++p) {
      const int row = p * TL::RPI + prow;
      const int64_t t = tb0 + (int64_t)kb * CG_KB + row;
      float v[TL::EP];
      if (sizeof(TIN) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(q[p][e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = bf16_to_f32(q[p][e] & 0xffffu);
          v[2 * e + 1] = bf16_to_f32(q[p][e] >> 16);
        }
      }
      uint32_t keep = t < T ? 0xffffffffu : 0u;
      if (drop && t < T) {
        uint32_t kb = 0;
#pragma unroll
        for (int g = 0; g < TL::EP / 4; ++g)
          kb |= keep4(tk.d, (uint64_t)t * (uint64_t)C + (uint64_t)(cbase + pcol + 4 * g)) << (4 * g);
        keep = kb;
      }
#pragma unroll
      for (int e = 0; e < TL::EP; e += 2) {
        const f32x2_t w = {((keep >> e) & 1u) ? v[e] : 0.0f, ((keep >> (e + 1)) & 1u) ? v[e + 1] : 0.0f};
        *reinterpret_cast<f32x2_t*>(&tile[row * TL::PITCH + pcol + e]) = w;
      }
    }
  };
  // the k-block's products: A = coefficients of ranks r16, tokens 8 kg .. (hi, lo), B =
  // column 16 cb + r16 of the tile, the same tokens
  auto multiply = [&](int kb) {
    const float4 c0 = *reinterpret_cast<const float4*>(&ct[r16 * CG_CTP + kb * CG_KB + 8 * kg]);
    const float4 c1 = *reinterpret_cast<const float4*>(&ct[r16 * CG_CTP + kb * CG_KB + 8 * kg + 4]);
    const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    bf16x8_t ch, cl;
    split8_bf16(cv, ch, cl);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float hv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = tile[(8 * kg + e) * TL::PITCH + 16 * cb + r16];
      bf16x8_t hh, hl;
      split8_bf16(hv, hh, hl);
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch, hh, acc[cb], 0, 0, 0);
      acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cl, hh, acc[cb], 0, 0, 0);
      if (sizeof(TIN) == 4) acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch, hl, acc[cb], 0, 0, 0);
    }
  };

  for (int64_t tb0 = 0; tb0 < T; tb0 += CG_TB) {
    const int nt = (int)min((int64_t)CG_TB, T - tb0);
    const int nkb = (nt + CG_KB - 1) / CG_KB;
    // the wave's first tile in flight while the coefficients are staged
    load(qa, tb0, min(wave, nkb - 1));
    __syncthreads();  // the previous block's coefficients are no longer read
    // coefficients [token][rank] -> ct[rank][token], zero past the block or past r; every
    // load issued before any store
    if (VEC) {
      constexpr int STG = CG_TB * (CG_J / 4) / 256;
      f32x4_t cv[STG];
#pragma unroll
      for (int k = 0; k < STG; ++k) {
        const int idx = tid + 256 * k, t = min(idx >> 2, nt - 1), q4 = 4 * (idx & 3);
        cv[k] = *reinterpret_cast<const f32x4_t*>(tk.coef + (tb0 + t) * r + min(j0 + q4, r - 4));
      }
#pragma unroll
      for (int k = 0; k < STG; ++k) {
        const int idx = tid + 256 * k, t = idx >> 2, q4 = 4 * (idx & 3);
        const bool ok = t < nt && j0 + q4 < r;
#pragma unroll
        for (int e = 0; e < 4; ++e) ct[(q4 + e) * CG_CTP + t] = ok ? cv[k][e] : 0.0f;
      }
    } else {
      for (int idx = tid; idx < CG_TB * CG_J; idx += 256) {
        const int t = idx / CG_J, j = idx % CG_J;
        ct[j * CG_CTP + t] = (t < nt && j0 + j < r) ? tk.coef[(tb0 + t) * r + j0 + j] : 0.0f;
      }
    }
    __syncthreads();
    // the wave's k-blocks wave, wave + 4, ...: two tiles in turn, the next one's loads
    // issued before this one is staged and multiplied (one exit, on a wave-uniform count;
    // every loaded tile is staged, a tile past the block re-reads valid tokens and is not
    // multiplied)
    for (int kb = wave; kb < nkb; kb += 8) {
      load(qb, tb0, min(kb + 4, nkb - 1));
      stage(qa, tb0, kb);
      __builtin_amdgcn_wave_barrier();
      multiply(kb);
      __builtin_amdgcn_wave_barrier();
      load(qa, tb0, min(kb + 8, nkb - 1));
      stage(qb, tb0, kb + 4);
      __builtin_amdgcn_wave_barrier();
      if (kb + 4 < nkb) multiply(kb + 4);
      __builtin_amdgcn_wave_barrier();
    }
  }
  // the four waves' sums in wave order; lane l of a wave holds ranks 4 (l >> 4) + i of
  // column l & 15 of each block
  __syncthreads();  // every wave is done with its tile, which the partials overwrite
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) wt[((wave * NCB + cb) * 4 + i) * 64 + lane] = acc[cb][i];
  __syncthreads();
  const float sc = tk.scale * (drop ? tk.d.sigma : 1.0f);
#pragma unroll
  for (int k = 0; k < NCB; ++k) {
    const int o = tid + 256 * k;
    // [r][C] output: consecutive threads take consecutive columns; [C][r]: consecutive ranks
    const int j = tk.out_cr ? (o & (CG_J - 1)) : (o / COLS);
    const int cc = tk.out_cr ? (o / CG_J) : (o & (COLS - 1));
    const int cb = cc >> 4, l = 16 * (j >> 2) + (cc & 15), i = j & 3;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) v += wt[((w * NCB + cb) * 4 + i) * 64 + l];
    v *= sc;
    const int64_t col = cbase + cc;
    if (j0 + j >= r || col >= C) continue;
    float* po = tk.out_cr ? tk.out + col * r + j0 + j : tk.out + (int64_t)(j0 + j) * C + col;
    *po = a.accumulate ? *po + v : v;
  }
}

// out[t][n..n+3] = sum_s P[s][t][n..n+3] (+ bias[n..n+3]) (+ old out), one rounding.
template <typename TOUT>
__global__ __launch_bounds__(256) void split_reduce(const float* __restrict__ part, int splits,
                                                    int64_t T, int64_t N,
                                                    const uint16_t* __restrict__ bias,
                                                    const TOUT* addend, int round_first,
                                                    TOUT* out) {  // addend may alias out
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
  if (addend) {
    float old[4];
    load4(addend + o, old);
    if (round_first) round4(out, a);
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = old[q] + a[q];
  }
  store4(out + o, a);
}

template <typename TIN, int MAT_KIND>
hipError_t pack_dispatch(const PackArgs& a, dim3 grid, double bytes, const char* name, const char* shape,
                         hipStream_t s) {
  return timed_launch(name, shape, 0.0, bytes, pack_lora<TIN, MAT_KIND>, grid, dim3(256), s, a);
}

}  // namespace

hipError_t launch_pack(const PackInput* ins, int nin, bool in_f32, int64_t T, int mat_kind, int r,
                       LoraProduct* prods, uint16_t* packed, int pack_steps, hipStream_t s) {
  if (nin < 1 || nin > GEMM_MAX_SEGS || r < 0 || T < 0) return hipErrorInvalidValue;
  PackArgs a;
  memset(&a, 0, sizeof(a));
  a.T = T;
  a.r = r;
  a.rgroups = r > 0 ? (r + 15) / 16 : 1;
  a.nseg = nin;
  a.packed = packed;
  int steps_total = 0, nprod = 0, zmax = 1;
  for (int i = 0; i < nin; ++i) {
    if (ins[i].C < 64 || ins[i].C % 64 || (r > 0 && ins[i].nprod < 1)) return hipErrorInvalidValue;
    steps_total += (int)(ins[i].C / 64);
    if (r > 0) {
      nprod += ins[i].nprod;
      zmax = std::max(zmax, ins[i].nprod);
    }
  }
  if (nprod > GEMM_MAX_SEGS) return hipErrorInvalidValue;
  a.pstride = pack_steps == 0 ? steps_total : pack_steps;
  int blocks = 0, prod0 = 0;
  double bytes = 0.0;
  int64_t ctot = 0;
  for (int i = 0; i < nin; ++i) {
    PackSeg& g = a.s[i];
    g.in = ins[i].in;
    g.C = ins[i].C;
    g.steps = (int)(g.C / 64);
    g.blk0 = blocks;
    g.pstep0 = ins[i].pstep0;
    g.prod0 = prod0;
    g.nprod = r > 0 ? ins[i].nprod : 0;
    if (g.pstep0 < 0 || g.pstep0 + g.steps > a.pstride) return hipErrorInvalidValue;
    const int nck = (int)((g.C + LORA_CHUNK - 1) / LORA_CHUNK);
    for (int q = 0; q < g.nprod; ++q) prods[prod0 + q].nck = nck;
    blocks += nck;
    prod0 += g.nprod;
    ctot += g.C;
    // the input once, its packed copy, each product's adapter and chunk partials
    bytes += (double)T * g.C * (in_f32 ? 4 : 2) + (packed ? (double)frag_rows(T) * g.C * 2 : 0.0) +
             g.nprod * ((double)r * g.C * 4 + (double)nck * T * r * 4);
  }
  if (T == 0 || (r == 0 && !packed)) return hipSuccess;
  for (int i = 0; i < nprod; ++i) {
    a.p[i].mat = prods[i].mat;
    a.p[i].part = prods[i].part;
    a.p[i].d = prods[i].drop;
  }
  const dim3 grid((unsigned)blocks, (unsigned)((T + 31) / 32), (unsigned)(zmax * a.rgroups));
  const char* name = packed ? "pack_lora" : "lora_product";
  char shape[48];
  snprintf(shape, sizeof(shape), "%lldx%lld r%d p%d i%d", (long long)T, (long long)ctot, r, nprod, nin);
  if (in_f32)
    return mat_kind == 0 ? pack_dispatch<float, 0>(a, grid, bytes, name, shape, s)
                         : pack_dispatch<float, 1>(a, grid, bytes, name, shape, s);
  return mat_kind == 0 ? pack_dispatch<uint16_t, 0>(a, grid, bytes, name, shape, s)
                       : pack_dispatch<uint16_t, 1>(a, grid, bytes, name, shape, s);
}

hipError_t launch_product_reduce(const LoraProduct* prods, int nprod, int64_t T, int r, hipStream_t s) {
  if (T == 0 || r == 0 || nprod == 0) return hipSuccess;
  if (nprod < 0 || nprod > GEMM_MAX_SEGS) return hipErrorInvalidValue;
  ReduceArgs ra;
  memset(&ra, 0, sizeof(ra));
  ra.n = T * r;
  double bytes = 0.0;
  int nck_max = 0;
  for (int i = 0; i < nprod; ++i) {
    ra.t[i] = {prods[i].part, prods[i].out, prods[i].scale, prods[i].nck};
    bytes += (double)(prods[i].nck + 1) * ra.n * 4;
    nck_max = std::max(nck_max, prods[i].nck);
  }
  char shape[40];
  snprintf(shape, sizeof(shape), "%lldx%d c%d p%d", (long long)T, r, nck_max, nprod);
  return timed_launch("lora_product_reduce", shape, 0.0, bytes, lora_skinny_reduce,
                      dim3((unsigned)((ra.n + 63) / 64), (unsigned)nprod), dim3(256), s, ra);
}

hipError_t launch_pack_lora(const void* in, bool in_f32, int64_t T, int64_t C, const float* mat, int mat_kind,
                            int r, float scale, const Dropout& d, uint16_t* packed, float* part, float* out,
                            hipStream_t s, int pack_steps, int pack_step0) {
  LoraProduct pr{mat, d, scale, part, out, 0};
  const PackInput pi{in, C, pack_step0, r > 0 ? 1 : 0};
  hipError_t e = launch_pack(&pi, 1, in_f32, T, mat_kind, r, &pr, packed, pack_steps, s);
  if (e == hipSuccess) e = launch_product_reduce(&pr, r > 0 ? 1 : 0, T, r, s);
  return e;
}

hipError_t launch_colgrad(const ColgradTask* tasks, int ntask, bool in_f32, int64_t T, int r, int accumulate,
                          hipStream_t s) {
  if (ntask < 1 || ntask > COLGRAD_MAX_TASKS || r < 1 || T < 0) return hipErrorInvalidValue;
  CgArgs a;
  memset(&a, 0, sizeof(a));
  a.ntask = ntask;
  a.T = T;
  a.r = r;
  a.accumulate = accumulate;
  double bytes = 0.0;
  int64_t ctot = 0;
  bool vec = r % 4 == 0;
  for (int i = 0; i < ntask; ++i) {
    const ColgradTask& q = tasks[i];
    if (q.C < 64 || q.C % 64) return hipErrorInvalidValue;  // whole 64-column groups
    if (reinterpret_cast<uintptr_t>(q.coef) & 15) vec = false;
    ctot += q.C;
  }
  const bool wide = colgrad_wide(ctot);
  const int cols = wide ? 64 : 16;
  int blocks = 0;
  for (int i = 0; i < ntask; ++i) {
    const ColgradTask& q = tasks[i];
    CgTaskDev& d = a.t[i];
    d.in = q.in;
    d.coef = q.coef;
    d.out = q.out;
    d.C = q.C;
    d.scale = q.scale;
    d.out_cr = q.out_cr;
    d.d = q.drop;
    d.block0 = blocks;
    blocks += (int)(q.C / cols);
    bytes += (double)T * q.C * (in_f32 ? 4 : 2) + (double)T * r * 4 + (double)r * q.C * 4 * (accumulate ? 2 : 1);
  }
  const dim3 grid((unsigned)blocks, (unsigned)((r + CG_J - 1) / CG_J));
  char shape[40];
  snprintf(shape, sizeof(shape), "%lldx%lld r%d n%d", (long long)T, (long long)ctot, r, ntask);
#define MSQ_CG(TIN, VEC, WIDE) \
  timed_launch("lora_colgrad", shape, 0.0, bytes, lora_colgrad<TIN, VEC, WIDE>, grid, dim3(256), s, a)
  if (in_f32) {
    if (vec) return wide ? MSQ_CG(float, true, true) : MSQ_CG(float, true, false);
    return wide ? MSQ_CG(float, false, true) : MSQ_CG(float, false, false);
  }
  if (vec) return wide ? MSQ_CG(uint16_t, true, true) : MSQ_CG(uint16_t, true, false);
  return wide ? MSQ_CG(uint16_t, false, true) : MSQ_CG(uint16_t, false, false);
#undef MSQ_CG
}

hipError_t launch_split_reduce(const float* part, int splits, int64_t T, int64_t N,
                               const uint16_t* bias, const void* addend, bool round_first, void* out,
                               bool out_f32, hipStream_t s) {
  const int64_t n4 = T * N / 4;
  if (n4 == 0) return hipSuccess;
  const dim3 grid((unsigned)((n4 + 255) / 256));
  const double ob = out_f32 ? 4.0 : 2.0;
  const double bytes = (double)splits * T * N * 4 + (double)T * N * ob * (addend ? 2 : 1) + (bias ? 2.0 * N : 0.0);
  char shape[32];
  snprintf(shape, sizeof(shape), "%lldx%lld s%d", (long long)T, (long long)N, splits);
  if (out_f32)
    return timed_launch("split_reduce", shape, 0.0, bytes, split_reduce<float>, grid, dim3(256), s, part, splits, T,
                        N, bias, (const float*)addend, (int)round_first, (float*)out);
  return timed_launch("split_reduce", shape, 0.0, bytes, split_reduce<uint16_t>, grid, dim3(256), s, part, splits,
                      T, N, bias, (const uint16_t*)addend, (int)round_first, (uint16_t*)out);
}

}  // namespace msq
