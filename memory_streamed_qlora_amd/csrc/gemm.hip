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
// The rank-r LoRA term of the same output tile is one more MFMA k-step per 16 ranks
// (operands split into bf16 hi/lo pairs for ~fp32 accuracy); in the backward it goes
// to a second accumulator so the dropout keep-mask can be applied per element.
// Unsplit launches write the final output (bias or the old dx added, rounded once);
// the reduction can instead be split over gridDim.z, in which case split 0 carries
// the LoRA term and fp32 partial tiles go to a workspace summed in split order by a
// separate kernel, so results never depend on timing.
#include "internal.hpp"

namespace msq {
namespace {

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int PAD = 8;              // bf16 elements of row padding in LDS
constexpr int LDW = BK + PAD;       // LDS row pitch in bf16 elements (144 bytes)
constexpr int THREADS = 256;

struct GemmArgs {
  const uint16_t* act;   // [M][R] bf16
  const uint8_t* codes;  // [N][K/2]
  const float* absmax;   // [N][K/64]
  int64_t M, N, K;       // W is [N][K]
  int64_t R, Nc;         // reduction length and output columns
  int steps, steps_per_split, splits;
  Nf4Lut lut;
  // LoRA term, added once (by split 0):
  //   forward  lscale * lu[m][:] . lw[n][:]          lu = u [M][r], lw = B [N][r]
  //   backward keep(m,k) * sigma * lu[m][:] . lw[:][k]  lu = du [M][r], lw = A [r][K]
  const float* lu;
  const float* lw;
  int r;
  float lscale;
  Dropout drop;
  // output: splits == 1 -> y / dx directly (bf16 or fp32, + bias / + old dx);
  //         splits  > 1 -> fp32 partials [splits][M][Nc]
  const uint16_t* bias;
  void* out;
  int out_f32, accumulate;
};

// fp32 -> (hi, lo) bf16 pair with hi + lo = v to ~2^-16 relative; products of the
// pairs are exact in fp32, so hi*hi + hi*lo + lo*hi carries ~fp32 accuracy on MFMA.
__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne(v);
  lo = bf16_rne(v - bf16_to_f32(hi));
}

// Launch order -> output tile.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup g runs on XCD g % 8), each with its own L2.  Tiles are listed m-fastest
// (the M-tiles of one weight tile are neighbours) and handed to the XCDs in 8
// contiguous ranges, so the workgroups that read the same NF4 tile share an L2.
__device__ __forceinline__ void tile_of(int64_t& n0, int64_t& m0, int& split) {
  const int64_t Mt = gridDim.y, Nt = gridDim.x;
  const int64_t Q = Mt * Nt * gridDim.z;
  const int64_t g = (int64_t)blockIdx.x + (int64_t)gridDim.x * ((int64_t)blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
  const int64_t x = g % 8, j = g / 8, q = Q / 8, rem = Q % 8;
  const int64_t t = x * q + (x < rem ? x : rem) + j;
  const int64_t m = t % Mt, rest = t / Mt;
  n0 = (rest % Nt) * BN;
  split = (int)(rest / Nt);
  m0 = m * BM;
}

template <int MODE, bool DROP>
__device__ __forceinline__ void gemm_body(const GemmArgs& g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int64_t n0, m0;
  int split;
  tile_of(n0, m0, split);
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

  // Per-thread share of one k-step's global data, prefetched one step ahead.
  uint4 ra[4];   // activations: 4 x 8 bf16
  uint4 rq;      // 32 NF4 codes of one (row, 64-block)
  float rs;      // that block's absmax
  // fixed per-thread coordinates
  const int w_row = MODE == 0 ? (tid >> 1) : (tid >> 2);      // fwd: W row in tile; bwd: reduction row
  const int w_sub = MODE == 0 ? (tid & 1) : (tid & 3);        // fwd: 32-code half; bwd: 32-col quarter
  const int64_t w_col = MODE == 0 ? (n0 + w_row) : (n0 + 32 * w_sub);  // fwd: W row; bwd: W column
  const bool w_ok = w_col < g.Nc;

  auto gload = [&](int step) {
    const int64_t r0 = (int64_t)step * BK;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + THREADS * c;
      const int row = idx >> 3, c8 = idx & 7;
      const int64_t gm = m0 + row;
      ra[c] = gm < g.M ? *reinterpret_cast<const uint4*>(g.act + gm * g.R + r0 + c8 * 8)
                       : make_uint4(0u, 0u, 0u, 0u);
    }
    if (w_ok) {
      if (MODE == 0) {
        rq = *reinterpret_cast<const uint4*>(g.codes + w_col * kw_half + r0 / 2 + w_sub * 16);
        rs = g.absmax[w_col * kw_blk + r0 / 64];
      } else {
        rq = *reinterpret_cast<const uint4*>(g.codes + (r0 + w_row) * kw_half + w_col / 2);
        rs = g.absmax[(r0 + w_row) * kw_blk + w_col / 64];
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int idx = tid + THREADS * c;
      const int row = idx >> 3, c8 = idx & 7;
      *reinterpret_cast<uint4*>(&sA[buf][row * LDW + c8 * 8]) = ra[c];
    }
    uint32_t out[16];
    if (w_ok) {
      const Nf4Planes P = nf4_planes(g.lut, rs);
      nf4_dequant32(P, rq, out);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = 0u;
    }
    if (MODE == 0) {
      uint4* dst = reinterpret_cast<uint4*>(&sB[buf][w_row * LDW + w_sub * 32]);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_uint4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t v = (j & 1) ? (out[j >> 1] >> 16) : (out[j >> 1] & 0xffffu);
        sB[buf][(32 * w_sub + j) * LDW + w_row] = (uint16_t)v;
      }
    }
  };

  if (s_begin < s_end) gload(s_begin);
  for (int step = s_begin; step < s_end; ++step) {
    const int buf = (step - s_begin) & 1;
    lstore(buf);
    __syncthreads();
    if (step + 1 < s_end) gload(step + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kof = ks * 16 + 8 * (lane >> 5);
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][(wm * 64 + i * 32 + (lane & 31)) * LDW + kof]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][(wn * 64 + j * 32 + (lane & 31)) * LDW + kof]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();

  // ---- LoRA term: one extra MFMA k-step per 16 ranks, operands split hi/lo ---------------
  f32x16_t acc2[2][2];
  if (DROP) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc2[i][j][v] = 0.0f;
  }
  if (split == 0 && g.r > 0) {
    for (int rc = 0; rc < g.r; rc += 16) {
      {
        const int row = tid >> 1, jh = (tid & 1) * 8;
        const int64_t gm = m0 + row;
        const int64_t gc = n0 + row;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = rc + jh + jj;
          float a = 0.0f, b = 0.0f;
          if (j < g.r) {
            if (gm < g.M) a = g.lscale * g.lu[gm * g.r + j];
            if (gc < g.Nc) b = (MODE == 0) ? g.lw[gc * g.r + j] : g.lw[(int64_t)j * g.K + gc];
          }
          uint32_t hi, lo;
          split_bf16(a, hi, lo);
          sA[0][row * LDW + jh + jj] = (uint16_t)hi;
          sA[0][row * LDW + 16 + jh + jj] = (uint16_t)lo;
          split_bf16(b, hi, lo);
          sB[0][row * LDW + jh + jj] = (uint16_t)hi;
          sB[0][row * LDW + 16 + jh + jj] = (uint16_t)lo;
        }
      }
      __syncthreads();
      const int kof = 8 * (lane >> 5);
      bf16x8_t ah[2], al[2], bh[2], bl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int rw = (wm * 64 + i * 32 + (lane & 31)) * LDW;
        ah[i] = *reinterpret_cast<const bf16x8_t*>(&sA[0][rw + kof]);
        al[i] = *reinterpret_cast<const bf16x8_t*>(&sA[0][rw + 16 + kof]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rw = (wn * 64 + j * 32 + (lane & 31)) * LDW;
        bh[j] = *reinterpret_cast<const bf16x8_t*>(&sB[0][rw + kof]);
        bl[j] = *reinterpret_cast<const bf16x8_t*>(&sB[0][rw + 16 + kof]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          f32x16_t t = DROP ? acc2[i][j] : acc[i][j];
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], t, 0, 0, 0);
          t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], t, 0, 0, 0);
          if (DROP)
            acc2[i][j] = t;
          else
            acc[i][j] = t;
        }
      __syncthreads();
    }
    if (DROP) {  // masked LoRA input gradient: acc += keep * sigma * acc2
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (m < g.M && n < g.Nc) {
              const uint64_t e = (uint64_t)m * (uint64_t)g.Nc + (uint64_t)n;
              const uint32_t keep = (keep4(g.drop, e & ~(uint64_t)3) >> (e & 3)) & 1u;
              if (keep) acc[i][j][v] += g.drop.sigma * acc2[i][j][v];
            }
          }
        }
    }
  }

  // ---- output ---------------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.Nc) continue;
      const float bn = (MODE == 0 && g.splits == 1 && g.bias) ? bf16_to_f32(g.bias[n]) : 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m >= g.M) continue;
        float val = acc[i][j][v];
        if (g.splits > 1) {
          reinterpret_cast<float*>(g.out)[((int64_t)split * g.M + m) * g.Nc + n] = val;
          continue;
        }
        const int64_t o = m * g.Nc + n;
        if (MODE == 0) val += bn;
        if (g.out_f32) {
          float* po = reinterpret_cast<float*>(g.out);
          po[o] = (MODE == 1 && g.accumulate) ? po[o] + val : val;
        } else {
          uint16_t* po = reinterpret_cast<uint16_t*>(g.out);
          if (MODE == 1 && g.accumulate) val = bf16_to_f32(po[o]) + val;
          po[o] = (uint16_t)bf16_rne(val);
        }
      }
    }
}

__global__ __launch_bounds__(THREADS) void nf4_fwd_gemm(GemmArgs g) { gemm_body<0, false>(g); }
__global__ __launch_bounds__(THREADS) void nf4_bwd_gemm(GemmArgs g) { gemm_body<1, false>(g); }
__global__ __launch_bounds__(THREADS) void nf4_bwd_gemm_dropout(GemmArgs g) { gemm_body<1, true>(g); }

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

hipError_t launch_gemm(const GemmLaunch& L, hipStream_t s) {
  GemmArgs g;
  g.act = L.act;
  g.codes = L.codes;
  g.absmax = L.absmax;
  g.M = L.M;
  g.N = L.N;
  g.K = L.K;
  g.R = L.mode == 0 ? L.K : L.N;
  g.Nc = L.mode == 0 ? L.N : L.K;
  g.steps = L.plan.steps;
  g.steps_per_split = L.plan.steps_per_split;
  g.splits = L.plan.splits;
  g.lut = nf4_lut();
  g.lu = L.lu;
  g.lw = L.lw;
  g.r = L.r;
  g.lscale = L.lscale;
  g.drop = L.drop;
  g.bias = L.bias;
  g.out = L.out;
  g.out_f32 = L.out_f32;
  g.accumulate = L.accumulate;
  const dim3 grid((unsigned)((g.Nc + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM), (unsigned)g.splits);
  const double flops = 2.0 * (double)g.M * (double)g.N * (double)g.K;
  int rec;
  if (L.mode == 0) {
    rec = timing_begin("nf4_fwd_gemm", flops, s);
    hipLaunchKernelGGL(nf4_fwd_gemm, grid, dim3(THREADS), 0, s, g);
  } else if (L.r > 0 && L.drop.threshold != 0u) {
    rec = timing_begin("nf4_bwd_gemm", flops, s);
    hipLaunchKernelGGL(nf4_bwd_gemm_dropout, grid, dim3(THREADS), 0, s, g);
  } else {
    rec = timing_begin("nf4_bwd_gemm", flops, s);
    hipLaunchKernelGGL(nf4_bwd_gemm, grid, dim3(THREADS), 0, s, g);
  }
  const hipError_t e = hipGetLastError();
  timing_end(rec, s);
  return e;
}

}  // namespace msq
