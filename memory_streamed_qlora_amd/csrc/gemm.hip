// Fused NF4-dequant + bf16 MFMA GEMMs of the frozen base.
//
// Forward:  P[s][t][n] = sum_{k in split s} x[t][k]  * W[n][k]    ("NT")
// Backward: P[s][t][k] = sum_{n in split s} dy[t][n] * W[n][k]    ("NN", dx of the base)
// W is never materialised: each workgroup reads NF4 codes and per-64 absmax straight
// from HBM (coalesced 16-byte loads), builds the block's 16-entry bf16 table
// bf16_rne(L[c] * absmax), looks codes up four at a time with v_perm, and writes the
// bf16 tile into LDS in the layout the MFMA operand reads want; the contraction
// runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The pages' base is
// frozen (never differentiated: "Poros" research post, training-step paragraph),
// so there is no dW kernel.
//
// Tile: BM=128 rows of t x BN=128 output columns x BK=64 reduction, 256 threads =
// 4 waves in a 2x2 grid, each wave owns a 64x64 sub-tile = 2x2 MFMA 32x32 blocks.
// The reduction can be split over gridDim.z; partial tiles go to a workspace and a
// separate epilogue sums them in split order, so results never depend on timing.
#include "internal.hpp"

namespace msq {
namespace {

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int PAD = 8;              // bf16 elements of row padding in LDS
constexpr int LDW = BK + PAD;       // LDS row pitch in bf16 elements (144 bytes)
constexpr int THREADS = 256;

struct GemmArgs {
  const uint16_t* act;   // [M][R]
  const uint8_t* codes;  // [N][K/2]
  const float* absmax;   // [N][K/64]
  float* part;           // [S][M][Nc]
  int64_t M, N, K;       // W is [N][K]
  int64_t R, Nc;         // reduction length and output columns
  int steps, steps_per_split;
  Nf4Lut lut;
};

template <int MODE>
__device__ __forceinline__ void gemm_body(const GemmArgs& g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int split = blockIdx.z;
  const int s_begin = split * g.steps_per_split;
  const int s_end = min(g.steps, s_begin + g.steps_per_split);

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int64_t kw_half = g.K / 2, kw_blk = g.K / 64;

  for (int step = s_begin; step < s_end; ++step) {
    const int64_t r0 = (int64_t)step * BK;
    // ---- activations tile [BM][BK] -> sA ---------------------------------------
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + THREADS * c;
      const int row = idx >> 3, c8 = idx & 7;
      const int64_t gm = m0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (gm < g.M) v = *reinterpret_cast<const uint4*>(g.act + gm * g.R + r0 + c8 * 8);
      *reinterpret_cast<uint4*>(&sA[row * LDW + c8 * 8]) = v;
    }
    // ---- dequantized weight tile -> sB[out col][reduction] -------------------------
    if (MODE == 0) {
      // rows n0..n0+127 of W, columns r0..r0+63 (exactly one absmax block per row)
      const int row = tid >> 1, half = tid & 1;
      const int64_t gn = n0 + row;
      uint32_t out[16];
      if (gn < g.Nc) {
        const uint4 q = *reinterpret_cast<const uint4*>(g.codes + gn * kw_half + r0 / 2 + half * 16);
        const Nf4Planes P = nf4_planes(g.lut, g.absmax[gn * kw_blk + r0 / 64]);
        nf4_dequant32(P, q, out);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = 0u;
      }
      uint4* dst = reinterpret_cast<uint4*>(&sB[row * LDW + half * 32]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    } else {
      // rows r0..r0+63 of W (reduction), columns n0..n0+127 (output), stored transposed
      const int row = tid >> 2, q4 = tid & 3;
      const int64_t kc = n0 + 32 * q4;
      uint32_t out[16];
      if (kc < g.Nc) {
        const uint4 q = *reinterpret_cast<const uint4*>(g.codes + (r0 + row) * kw_half + kc / 2);
        const Nf4Planes P = nf4_planes(g.lut, g.absmax[(r0 + row) * kw_blk + kc / 64]);
        nf4_dequant32(P, q, out);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) out[i] = 0u;
      }
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t v = (j & 1) ? (out[j >> 1] >> 16) : (out[j >> 1] & 0xffffu);
        sB[(32 * q4 + j) * LDW + row] = (uint16_t)v;
      }
    }
    __syncthreads();
    // ---- MFMA over the tile --------------------------------------------------------
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kof = ks * 16 + 8 * (lane >> 5);
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[(wm * 64 + i * 32 + (lane & 31)) * LDW + kof]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sB[(wn * 64 + j * 32 + (lane & 31)) * LDW + kof]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  // ---- partial tile -> workspace ------------------------------------------------------
  float* P = g.part + (int64_t)split * g.M * g.Nc;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < g.M && n < g.Nc) P[m * g.Nc + n] = acc[i][j][v];
      }
    }
}

__global__ __launch_bounds__(THREADS) void nf4_fwd_gemm(GemmArgs g) { gemm_body<0>(g); }
__global__ __launch_bounds__(THREADS) void nf4_bwd_gemm(GemmArgs g) { gemm_body<1>(g); }

}  // namespace

GemmPlan gemm_plan(int64_t m, int64_t nc, int64_t red) {
  GemmPlan p;
  p.steps = (int)(red / BK);
  const int64_t tiles = ((m + BM - 1) / BM) * ((nc + BN - 1) / BN);
  int s = 1;
  while (tiles * s < 512 && (int64_t)p.steps >= 8 * s) s *= 2;
  p.splits = s;
  p.steps_per_split = (p.steps + s - 1) / s;
  return p;
}

hipError_t launch_gemm(int mode, const uint16_t* act, const uint8_t* codes, const float* absmax,
                       int64_t M, int64_t N, int64_t K, const GemmPlan& plan, float* part,
                       hipStream_t s) {
  GemmArgs g;
  g.act = act;
  g.codes = codes;
  g.absmax = absmax;
  g.part = part;
  g.M = M;
  g.N = N;
  g.K = K;
  g.R = mode == 0 ? K : N;
  g.Nc = mode == 0 ? N : K;
  g.steps = plan.steps;
  g.steps_per_split = plan.steps_per_split;
  g.lut = nf4_lut();
  const dim3 grid((unsigned)((g.Nc + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)plan.splits);
  const double flops = 2.0 * (double)M * (double)N * (double)K;
  int rec;
  if (mode == 0) {
    rec = timing_begin("nf4_fwd_gemm", flops, s);
    hipLaunchKernelGGL(nf4_fwd_gemm, grid, dim3(THREADS), 0, s, g);
  } else {
    rec = timing_begin("nf4_bwd_gemm", flops, s);
    hipLaunchKernelGGL(nf4_bwd_gemm, grid, dim3(THREADS), 0, s, g);
  }
  const hipError_t e = hipGetLastError();
  timing_end(rec, s);
  return e;
}

}  // namespace msq
