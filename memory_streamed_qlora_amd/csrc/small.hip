// Small-tile path of the fused NF4 (or bf16) + LoRA linear, for shapes at which the tiled
// path's launches are latency-bound.  The tiled path runs a forward as a packing pass, a
// product reduction, a 512 x 128-tile GEMM with a split reduction and its partial sums
// (four or five launches, each with its own fixed pipeline; the single 896 x 896 linear
// at 512 tokens gets 7 column tiles).  Here the forward is one launch and the backward
// two (the input gradient together with du, then the column gradients of A and B), and
// nothing crosses a workgroup except through the outputs.
//
// small_fwd: a workgroup of four waves owns a 64 (tokens) x 64 (outputs) tile of y over
// all of K.  Wave w takes the k-steps s = w, w + 4, ... of 64 columns: an in-workgroup
// split of the reduction, so the waves never wait for each other inside the loop.  Per
// k-step a lane loads, straight into registers in the v_mfma_f32_32x32x16_bf16 operand
// layout, 32 consecutive x values of each of its two rows (lane half hk takes columns
// 32 hk .. 32 hk + 31 of the step, sub-step c the 8 from 8 c) and 32 NF4 codes of each of
// its two W rows (dequantized through the block's 16-entry table, as in the tiled path),
// and multiplies the wave's 2 x 2 blocks of 32 x 32.  The same x registers, masked by the
// dropout keep bits, feed the wave's share of u = drop(x) A^T: A (fp32) split into bf16
// hi + lo, x bf16 exactly (or split too when x is fp32).  After the loop the four
// partial tiles go through LDS and are summed in wave order; wave w then owns output
// block (w & 1, w >> 1): y += (alpha / r) u B^T (u and B split hi/lo), + bias, rounding,
// + residual.  u is written by the workgroups of output tile 0.
//
// small_bwd: the same decomposition over dx (64 tokens x 64 input columns), reducing over
// the n rows of W.  W^T is formed per wave in LDS (each lane dequantizes two W rows of the
// k-step and writes them as (row, row + 1) bf16 pairs down the tile's 64 columns); B^T
// likewise, for du = s dy B, accumulated beside dx from the same dy registers.  After the
// wave-order sum, dx += keep * sigma * (du A) on the owning wave, then the old dx when
// accumulating (one rounding of the fp32 sum).  du goes to a buffer for the column
// gradients (lora_colgrad, the tiled path's kernel), written by input tile 0.
//
// The sums run in a fixed order that depends only on the shape, so results are bitwise
// reproducible; they differ in rounding order from the tiled path's.
#include <string.h>

#include <algorithm>

#include "internal.hpp"

namespace msq {
namespace {

constexpr int SM_T = 64;       // tokens per workgroup
constexpr int SM_C = 64;       // output (forward) or input (backward) columns per workgroup
constexpr int SM_WAVES = 4;
constexpr int SM_BLK = 16 * 64;  // one 32 x 32 fp32 block in register order: [v][lane]

// Eight fp32 values -> bf16 hi and lo operands (hi = rne(v), lo = rne(v - hi)).
__device__ __forceinline__ void sm_split8(const float (&v)[8], bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    l[i] = pack_bf16x2(v[2 * i] - bf16_to_f32(h[i] & 0xffffu), v[2 * i + 1] - bf16_to_f32(h[i] >> 16));
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

// Zero the bf16 elements of a packed 8-element operand whose keep bit (bit e) is clear.
__device__ __forceinline__ uint4 sm_mask8(uint4 q, uint32_t keep) {
  uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = (((keep >> (2 * i)) & 1u) ? 0x0000ffffu : 0u) | (((keep >> (2 * i + 1)) & 1u) ? 0xffff0000u : 0u);
    w[i] &= m;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The register row (of a 32 x 32 MFMA result block) that lane half hk holds in register v.
__device__ __forceinline__ int sm_row(int v, int hk) { return 8 * (v >> 2) + 4 * hk + (v & 3); }

struct SmallFwdArgs {
  const void* x;          // [T][K] bf16 or fp32
  const uint8_t* codes;   // NF4 base [N][K/2], absmax [N][K/64]; or
  const float* absmax;
  const uint16_t* wbf;    // bf16 base [N][K]
  const uint16_t* bias;   // [N] or null
  const void* residual;   // [T][N] in y's type or null
  const float* A;         // [r][K]
  const float* B;         // [N][r]
  void* y;                // [T][N] bf16 or fp32 (unused with u_only)
  float* u;               // [T][r] or null
  int64_t T, K, N;
  int r;
  float lscale;
  int out_f32, u_only;
  Dropout d;
  Nf4Lut lut;
};

// MAIN: y is formed (false: u alone); LORA: r > 0.  Both are template parameters so that
// every load of a k-step is unconditional and the compiler counts them exactly (a load
// under a runtime branch makes it wait for all of them, the prefetched step included).
template <bool XF32, bool BF16W, bool MAIN, bool LORA>
__global__ __launch_bounds__(256) void small_fwd(SmallFwdArgs a) {
  // the waves' partial tiles: [wave][block: y (i, j) as i + 2 j, then u row block 4 + i][v][lane]
  __shared__ __attribute__((aligned(16))) float red[SM_WAVES * 6 * SM_BLK];
  __shared__ __attribute__((aligned(16))) float ust[SM_WAVES][32 * 33];  // a wave's u block, [row][rank]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hk = lane >> 5, r32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * SM_C, m0 = (int64_t)blockIdx.y * SM_T;
  const int64_t T = a.T, K = a.K, N = a.N;
  const int steps = (int)(K / 64), r = a.r;
  constexpr bool main = MAIN, lora = LORA;
  const Dropout d = a.d;
  // the lane's two token rows (clamped: rows past T only feed results that are dropped)
  // and its two W rows; its rank in the u product
  const int64_t mr0 = min(m0 + r32, T - 1), mr1 = min(m0 + 32 + r32, T - 1);
  const int64_t wn0 = n0 + r32, wn1 = n0 + 32 + r32;
  const int rk = min(r32, max(r - 1, 0));
  const bool rk_ok = r32 < r;

  f32x16_t acc[2][2], ua[2];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc[0][0][v] = acc[0][1][v] = acc[1][0][v] = acc[1][1][v] = 0.0f;
    ua[0][v] = ua[1][v] = 0.0f;
  }

  // the B factor of this wave's output block (its LoRA term after the loop), loaded now
  const int oi = wave & 1, oj = wave >> 1;  // this wave's output block
  const int64_t nc = n0 + 32 * oj + r32;    // this lane's output column
  float bpre[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 16 * h + 8 * hk + e;
      bpre[h][e] = (main && j < r) ? a.B[nc * r + j] : 0.0f;
    }

  // One k-step's loads, straight into the MFMA operand layout: x (the lane's 32 columns of
  // each of its two rows), the W rows' codes and scales (or bf16 values), A's row of the
  // lane's rank.  The next k-step of the wave is loaded before this one is multiplied.
  constexpr int XQ = XF32 ? 8 : 4;  // 16-byte pieces of a lane's 32 x values per row
  constexpr int WQ = BF16W ? 4 : 1;
  struct Stage {
    uint4 xq[2][XQ];
    uint4 wq[2][WQ];
    float ws[2];
    float4 aq[8];
  };
  auto load = [&](Stage& st, int s) {
    const int64_t kc = (int64_t)s * 64 + 32 * hk;  // first column of this lane's 32
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      if (XF32) {
        st.xq[0][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.x) + mr0 * K + kc)[q];
        st.xq[1][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.x) + mr1 * K + kc)[q];
      } else {
        st.xq[0][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.x) + mr0 * K + kc)[q];
        st.xq[1][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.x) + mr1 * K + kc)[q];
      }
    }
    if (main) {
#pragma unroll
      for (int q = 0; q < WQ; ++q) {
        if (BF16W) {
          st.wq[0][q] = reinterpret_cast<const uint4*>(a.wbf + wn0 * K + kc)[q];
          st.wq[1][q] = reinterpret_cast<const uint4*>(a.wbf + wn1 * K + kc)[q];
        } else {
          st.wq[0][q] = *reinterpret_cast<const uint4*>(a.codes + wn0 * (K / 2) + kc / 2);
          st.wq[1][q] = *reinterpret_cast<const uint4*>(a.codes + wn1 * (K / 2) + kc / 2);
        }
      }
      if (!BF16W) {
        st.ws[0] = a.absmax[wn0 * (K / 64) + s];
        st.ws[1] = a.absmax[wn1 * (K / 64) + s];
      }
    }
    if (lora) {
#pragma unroll
      for (int q = 0; q < 8; ++q) st.aq[q] = reinterpret_cast<const float4*>(a.A + (int64_t)rk * K + kc)[q];
    }
  };
  auto compute = [&](const Stage& st, int s) {
    const int64_t kc = (int64_t)s * 64 + 32 * hk;
    // W operands of the two column blocks, sub-steps 0..3
    uint32_t wb[2][16];
    if (main) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (BF16W) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            wb[j][4 * q] = st.wq[j][q].x;
            wb[j][4 * q + 1] = st.wq[j][q].y;
            wb[j][4 * q + 2] = st.wq[j][q].z;
            wb[j][4 * q + 3] = st.wq[j][q].w;
          }
        } else {
          const Nf4Planes P = nf4_planes(a.lut, st.ws[j]);
          nf4_dequant32(P, st.wq[j][0], wb[j]);
        }
      }
    }
    // dropout keep bits of the lane's 32 values of each row (bit e: column kc + e)
    uint32_t keep[2] = {0xffffffffu, 0xffffffffu};
    if (lora && d.threshold != 0u) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint64_t e0 = (uint64_t)(i ? mr1 : mr0) * (uint64_t)K + (uint64_t)kc;
        uint32_t kb = 0;
#pragma unroll
        for (int g = 0; g < 8; ++g) kb |= keep4(d, e0 + 4 * g) << (4 * g);
        keep[i] = kb;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t ax[2], axl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (XF32) {
          const uint4 p0 = st.xq[i][2 * c], p1 = st.xq[i][2 * c + 1];
          const uint32_t w8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
          float xv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = __uint_as_float(w8[e]);
          sm_split8(xv, ax[i], axl[i]);
        } else {
          ax[i] = __builtin_bit_cast(bf16x8_t, st.xq[i][c]);
        }
      }
      if (main) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const bf16x8_t b =
              __builtin_bit_cast(bf16x8_t, make_uint4(wb[j][4 * c], wb[j][4 * c + 1], wb[j][4 * c + 2], wb[j][4 * c + 3]));
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[i], b, acc[i][j], 0, 0, 0);
        }
      }
      if (lora) {
        const float av[8] = {st.aq[2 * c].x, st.aq[2 * c].y, st.aq[2 * c].z, st.aq[2 * c].w,
                             st.aq[2 * c + 1].x, st.aq[2 * c + 1].y, st.aq[2 * c + 1].z, st.aq[2 * c + 1].w};
        float avz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) avz[e] = rk_ok ? av[e] : 0.0f;
        bf16x8_t ah, al;
        sm_split8(avz, ah, al);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          bf16x8_t xm = ax[i], xml = axl[i];
          if (d.threshold != 0u) {  // uniform: no masking work without dropout
            const uint32_t kb = (keep[i] >> (8 * c)) & 0xffu;
            xm = __builtin_bit_cast(bf16x8_t, sm_mask8(__builtin_bit_cast(uint4, ax[i]), kb));
            if (XF32) xml = __builtin_bit_cast(bf16x8_t, sm_mask8(__builtin_bit_cast(uint4, axl[i]), kb));
          }
          ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xm, ah, ua[i], 0, 0, 0);
          ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xm, al, ua[i], 0, 0, 0);
          if (XF32) ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xml, ah, ua[i], 0, 0, 0);
        }
      }
    }
  };
  {
    Stage s0, s1;
    int s = wave;
    if (s < steps) load(s0, s);
    while (s < steps) {
      // the next step's loads (past the end: the last step again, loaded and not used)
      const int s1i = s + SM_WAVES;
      load(s1, min(s1i, steps - 1));
      compute(s0, s);
      if (s1i >= steps) break;
      const int s2i = s1i + SM_WAVES;
      load(s0, min(s2i, steps - 1));
      compute(s1, s1i);
      s = s2i;
    }
  }

  // ---- the waves' partials, summed in wave order ------------------------------------
  float* mine = red + wave * 6 * SM_BLK;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    mine[(0 * 16 + v) * 64 + lane] = acc[0][0][v];
    mine[(1 * 16 + v) * 64 + lane] = acc[1][0][v];
    mine[(2 * 16 + v) * 64 + lane] = acc[0][1][v];
    mine[(3 * 16 + v) * 64 + lane] = acc[1][1][v];
    mine[(4 * 16 + v) * 64 + lane] = ua[0][v];
    mine[(5 * 16 + v) * 64 + lane] = ua[1][v];
  }
  __syncthreads();
  auto wsum = [&](int blk, int v) {
    const int o = (blk * 16 + v) * 64 + lane;
    return ((red[o] + red[6 * SM_BLK + o]) + red[12 * SM_BLK + o]) + red[18 * SM_BLK + o];
  };
  f32x16_t y, uf;
  const float usig = d.threshold != 0u ? d.sigma : 1.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    y[v] = wsum(oi + 2 * oj, v);
    uf[v] = lora ? usig * wsum(4 + oi, v) : 0.0f;
  }
  const int64_t rb = m0 + 32 * oi;  // first token row of the block
  if (lora && a.u && blockIdx.x == 0 && oj == 0 && rk_ok) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = rb + sm_row(v, hk);
      if (m < T) a.u[m * r + r32] = uf[v];
    }
  }
  if (!main) return;

  // ---- LoRA term: y += (alpha / r) u B^T, u through LDS into the operand layout -------
  if (lora) {
    float* us = &ust[wave][0];
#pragma unroll
    for (int v = 0; v < 16; ++v) us[sm_row(v, hk) * 33 + r32] = a.lscale * uf[v];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (16 * h >= r) break;
      float uv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * h + 8 * hk + e;
        uv[e] = j < r ? us[r32 * 33 + j] : 0.0f;
      }
      bf16x8_t uh, ul, bh, bl;
      sm_split8(uv, uh, ul);
      sm_split8(bpre[h], bh, bl);
      y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uh, bh, y, 0, 0, 0);
      y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uh, bl, y, 0, 0, 0);
      y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ul, bh, y, 0, 0, 0);
    }
  }

  // ---- output: + bias, rounding, + residual (y rounded first, as a separate add) -------
  const float bn = a.bias ? bf16_to_f32(a.bias[nc]) : 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t m = rb + sm_row(v, hk);
    if (m >= T) continue;
    float val = y[v] + bn;
    if (a.out_f32) {
      float* po = reinterpret_cast<float*>(a.y) + m * N + nc;
      if (a.residual) val = reinterpret_cast<const float*>(a.residual)[m * N + nc] + val;
      *po = val;
    } else {
      uint16_t* po = reinterpret_cast<uint16_t*>(a.y) + m * N + nc;
      if (a.residual) {
        val = bf16_to_f32(bf16_rne(val));
        val = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.residual)[m * N + nc]) + val;
      }
      *po = (uint16_t)bf16_rne(val);
    }
  }
}

struct SmallBwdArgs {
  const void* dy;         // [T][N] bf16 or fp32
  const uint8_t* codes;   // NF4 base [N][K/2], absmax [N][K/64]; or
  const float* absmax;
  const uint16_t* wbf;    // bf16 base [N][K]
  const float* A;         // [r][K]
  const float* B;         // [N][r]
  void* dx;               // [T][K] bf16 or fp32
  float* du;              // [T][r]: s dy B, written by input tile 0 (null: not written)
  int64_t T, K, N;
  int r;
  float lscale;
  int out_f32, accumulate;
  Dropout d;              // the forward's LoRA input mask (replayed)
  Nf4Lut lut;
};

// LDS of small_bwd: in the loop each wave has a W^T tile (64 input columns x 32 bf16 pairs
// of W rows, pitch 36 dwords) and a B^T tile (32 ranks x 64 W rows fp32, pitch 68); after
// it, the waves' partial blocks (6 per wave) and a u-side staging block per wave.
constexpr int SB_WT = 64 * 36;      // dwords per wave
constexpr int SB_BT = 32 * 68;      // floats per wave
constexpr int SB_LOOP = SM_WAVES * (SB_WT + SB_BT);
constexpr int SB_END = SM_WAVES * 6 * SM_BLK + SM_WAVES * 32 * 33;
constexpr int SB_WORDS = SB_LOOP > SB_END ? SB_LOOP : SB_END;

// LORA: r > 0 (then r % 4 == 0: B's rows are loaded as float4).  A template parameter for
// the reason given at small_fwd.
template <bool XF32, bool BF16W, bool LORA>
__global__ __launch_bounds__(256) void small_bwd(SmallBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[SB_WORDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hk = lane >> 5, r32 = lane & 31;
  const int64_t k0 = (int64_t)blockIdx.x * SM_C, m0 = (int64_t)blockIdx.y * SM_T;
  const int64_t T = a.T, K = a.K, N = a.N;
  const int steps = (int)(N / 64), r = a.r;
  constexpr bool lora = LORA;
  const int64_t mr0 = min(m0 + r32, T - 1), mr1 = min(m0 + 32 + r32, T - 1);
  uint32_t* wt = lds + wave * (SB_WT + SB_BT);
  float* bt = reinterpret_cast<float*>(wt + SB_WT);
  // the W rows this lane dequantizes: 2 (lane & 31) and the next, columns k0 + 32 hk ..
  const int pr = 2 * r32;

  f32x16_t acc[2][2], ua[2];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    acc[0][0][v] = acc[0][1][v] = acc[1][0][v] = acc[1][1][v] = 0.0f;
    ua[0][v] = ua[1][v] = 0.0f;
  }
  // A's column of this wave's output block (its LoRA term after the loop), loaded now
  const int oi = wave & 1, oj = wave >> 1;
  const int64_t kc = k0 + 32 * oj + r32;  // this lane's dx column
  float apre[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 16 * h + 8 * hk + e;
      apre[h][e] = j < r ? a.A[(int64_t)j * K + kc] : 0.0f;
    }

  // One reduction step's loads: dy (the lane's 32 reduction columns of each of its two
  // rows), two W rows over the lane's 32 input columns, B's row (64 per step, one per lane).
  // The next step of the wave is loaded before this one is transposed and multiplied.
  constexpr int XQ = XF32 ? 8 : 4;
  constexpr int WQ = BF16W ? 8 : 1;
  const int rq = max(r / 4, 1);  // float4 pieces of a B row
  struct Stage {
    uint4 xq[2][XQ];
    uint4 wq[2][WQ];
    float ws[2];
    float bq[32];
  };
  auto load = [&](Stage& st, int s) {
    const int64_t nr = (int64_t)s * 64 + 32 * hk;  // first reduction row of this lane's 32
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      if (XF32) {
        st.xq[0][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.dy) + mr0 * N + nr)[q];
        st.xq[1][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(a.dy) + mr1 * N + nr)[q];
      } else {
        st.xq[0][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.dy) + mr0 * N + nr)[q];
        st.xq[1][q] = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.dy) + mr1 * N + nr)[q];
      }
    }
    const int64_t wr = (int64_t)s * 64 + pr;
    const int64_t kk = k0 + 32 * hk;
    if (BF16W) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        st.wq[0][q] = reinterpret_cast<const uint4*>(a.wbf + wr * K + kk)[q];
        st.wq[1][q] = reinterpret_cast<const uint4*>(a.wbf + (wr + 1) * K + kk)[q];
      }
    } else {
      st.wq[0][0] = *reinterpret_cast<const uint4*>(a.codes + wr * (K / 2) + kk / 2);
      st.wq[1][0] = *reinterpret_cast<const uint4*>(a.codes + (wr + 1) * (K / 2) + kk / 2);
      st.ws[0] = a.absmax[wr * (K / 64) + k0 / 64];
      st.ws[1] = a.absmax[(wr + 1) * (K / 64) + k0 / 64];
    }
    if (lora) {
      // B row bn: pieces past r re-read the last one (in bounds) and are zeroed at use
      const int64_t bn = (int64_t)s * 64 + lane;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(a.B + bn * r + 4 * min(q, rq - 1));
        st.bq[4 * q] = v.x;
        st.bq[4 * q + 1] = v.y;
        st.bq[4 * q + 2] = v.z;
        st.bq[4 * q + 3] = v.w;
      }
    }
  };
  auto compute = [&](const Stage& st) {
    // W^T: input column 32 hk + e gets the bf16 pair (row 2 r32, row 2 r32 + 1) at pair r32
    uint32_t w0[16], w1[16];
    if (BF16W) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w0[4 * q] = st.wq[0][q].x; w0[4 * q + 1] = st.wq[0][q].y; w0[4 * q + 2] = st.wq[0][q].z; w0[4 * q + 3] = st.wq[0][q].w;
        w1[4 * q] = st.wq[1][q].x; w1[4 * q + 1] = st.wq[1][q].y; w1[4 * q + 2] = st.wq[1][q].z; w1[4 * q + 3] = st.wq[1][q].w;
      }
    } else {
      nf4_dequant32(nf4_planes(a.lut, st.ws[0]), st.wq[0][0], w0);
      nf4_dequant32(nf4_planes(a.lut, st.ws[1]), st.wq[1][0], w1);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      wt[(32 * hk + 2 * q) * 36 + r32] = __builtin_amdgcn_perm(w1[q], w0[q], 0x05040100u);
      wt[(32 * hk + 2 * q + 1) * 36 + r32] = __builtin_amdgcn_perm(w1[q], w0[q], 0x07060302u);
    }
    if (lora) {
#pragma unroll
      for (int j = 0; j < 32; ++j) bt[j * 68 + lane] = j < r ? st.bq[j] : 0.0f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t ax[2], axl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (XF32) {
          const uint4 p0 = st.xq[i][2 * c], p1 = st.xq[i][2 * c + 1];
          const uint32_t w8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
          float xv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[e] = __uint_as_float(w8[e]);
          sm_split8(xv, ax[i], axl[i]);
        } else {
          ax[i] = __builtin_bit_cast(bf16x8_t, st.xq[i][c]);
        }
      }
      // W^T operand of column block j: column 32 j + r32, reduction rows 32 hk + 8 c .. + 7
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&wt[(32 * j + r32) * 36 + 16 * hk + 4 * c]);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[i], b, acc[i][j], 0, 0, 0);
      }
      if (lora) {
        float bv[8];
        const float4 b0 = *reinterpret_cast<const float4*>(&bt[r32 * 68 + 32 * hk + 8 * c]);
        const float4 b1 = *reinterpret_cast<const float4*>(&bt[r32 * 68 + 32 * hk + 8 * c + 4]);
        bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
        bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
        bf16x8_t bh, bl;
        sm_split8(bv, bh, bl);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[i], bh, ua[i], 0, 0, 0);
          ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[i], bl, ua[i], 0, 0, 0);
          if (XF32) ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(axl[i], bh, ua[i], 0, 0, 0);
        }
      }
    }
    // the tiles are rewritten by this wave's next step: its reads complete first
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  {
    Stage s0, s1;
    int s = wave;
    if (s < steps) load(s0, s);
    while (s < steps) {
      // the next step's loads (past the end: the last step again, loaded and not used)
      const int s1i = s + SM_WAVES;
      load(s1, min(s1i, steps - 1));
      compute(s0);
      if (s1i >= steps) break;
      const int s2i = s1i + SM_WAVES;
      load(s0, min(s2i, steps - 1));
      compute(s1);
      s = s2i;
    }
  }

  // ---- the waves' partials, summed in wave order ------------------------------------
  __syncthreads();  // every wave is done with its loop tiles, which the partials overwrite
  float* red = reinterpret_cast<float*>(lds);
  float* mine = red + wave * 6 * SM_BLK;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    mine[(0 * 16 + v) * 64 + lane] = acc[0][0][v];
    mine[(1 * 16 + v) * 64 + lane] = acc[1][0][v];
    mine[(2 * 16 + v) * 64 + lane] = acc[0][1][v];
    mine[(3 * 16 + v) * 64 + lane] = acc[1][1][v];
    mine[(4 * 16 + v) * 64 + lane] = ua[0][v];
    mine[(5 * 16 + v) * 64 + lane] = ua[1][v];
  }
  __syncthreads();
  auto wsum = [&](int blk, int v) {
    const int o = (blk * 16 + v) * 64 + lane;
    return ((red[o] + red[6 * SM_BLK + o]) + red[12 * SM_BLK + o]) + red[18 * SM_BLK + o];
  };
  f32x16_t g, duf;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    g[v] = wsum(oi + 2 * oj, v);
    duf[v] = lora ? a.lscale * wsum(4 + oi, v) : 0.0f;
  }
  const int64_t rb = m0 + 32 * oi;
  if (lora && a.du && blockIdx.x == 0 && oj == 0 && r32 < r) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = rb + sm_row(v, hk);
      if (m < T) a.du[m * r + r32] = duf[v];
    }
  }

  // ---- LoRA input gradient: dx += keep * sigma * (du A) -------------------------------
  if (lora) {
    float* us = red + SM_WAVES * 6 * SM_BLK + wave * 32 * 33;
#pragma unroll
    for (int v = 0; v < 16; ++v) us[sm_row(v, hk) * 33 + r32] = duf[v];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    f32x16_t t;
#pragma unroll
    for (int v = 0; v < 16; ++v) t[v] = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (16 * h >= r) break;
      float uv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * h + 8 * hk + e;
        uv[e] = j < r ? us[r32 * 33 + j] : 0.0f;
      }
      bf16x8_t uh, ul, ah, al;
      sm_split8(uv, uh, ul);
      sm_split8(apre[h], ah, al);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uh, ah, t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uh, al, t, 0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ul, ah, t, 0, 0, 0);
    }
    const Dropout d = a.d;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      if (d.threshold == 0u) {
        g[v] += t[v];
      } else {
        const int64_t m = min(rb + sm_row(v, hk), T - 1);
        const uint64_t e = (uint64_t)m * (uint64_t)K + (uint64_t)kc;
        if ((keep4(d, e & ~(uint64_t)3) >> (e & 3)) & 1u) g[v] += d.sigma * t[v];
      }
    }
  }

  // ---- output: [old dx +] dx, one rounding ------------------------------------------
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t m = rb + sm_row(v, hk);
    if (m >= T) continue;
    float val = g[v];
    if (a.out_f32) {
      float* po = reinterpret_cast<float*>(a.dx) + m * K + kc;
      *po = a.accumulate ? *po + val : val;
    } else {
      uint16_t* po = reinterpret_cast<uint16_t*>(a.dx) + m * K + kc;
      if (a.accumulate) val = bf16_to_f32(*po) + val;
      *po = (uint16_t)bf16_rne(val);
    }
  }
}

template <typename K_, typename A_>
hipError_t small_launch(const char* name, const char* shape, double flops, double bytes, K_ kern, dim3 grid,
                        hipStream_t s, const A_& a) {
  return timed_launch(name, shape, flops, bytes, kern, grid, dim3(256), s, a);
}

}  // namespace

bool small_path_fits(int64_t t, int64_t k, int64_t n, int r) {
  return r <= SMALL_MAX_R && r % 4 == 0 && t <= SMALL_MAX_T && k <= SMALL_MAX_KN && n <= SMALL_MAX_KN;
}

hipError_t launch_small_fwd(const SmallLinear& L, const void* x, const uint16_t* bias, const void* residual, void* y,
                            float* u, bool u_only, hipStream_t s) {
  if (L.t == 0) return hipSuccess;
  if (L.r > SMALL_MAX_R || L.r % 4 || L.k % 64 || L.n % 64) return hipErrorInvalidValue;
  SmallFwdArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.codes = L.codes;
  a.absmax = L.absmax;
  a.wbf = L.wbf;
  a.bias = bias;
  a.residual = residual;
  a.A = L.A;
  a.B = L.B;
  a.y = y;
  a.u = u;
  a.T = L.t;
  a.K = L.k;
  a.N = L.n;
  a.r = L.r;
  a.lscale = L.lscale;
  a.out_f32 = L.out_f32;
  a.u_only = u_only;
  a.d = L.drop;
  a.lut = nf4_lut();
  const dim3 grid(u_only ? 1u : (unsigned)(L.n / SM_C), (unsigned)((L.t + SM_T - 1) / SM_T));
  const double flops = u_only ? 0.0 : 2.0 * L.t * L.k * L.n;
  const double wb = L.wbf ? 2.0 * L.n * L.k : 0.5625 * L.n * L.k;
  const double bytes = (double)L.t * L.k * (L.act_f32 ? 4 : 2) + (u_only ? 0.0 : wb + (double)L.t * L.n * (L.out_f32 ? 4 : 2)) +
                       (L.r > 0 ? 4.0 * L.r * (L.k + L.n + L.t) : 0.0);
  char shape[48];
  snprintf(shape, sizeof(shape), "%lldx%lldx%lld r%d%s", (long long)L.t, (long long)L.n, (long long)L.k, L.r,
           u_only ? " u" : "");
  const char* name = "small_fwd";
  if (u_only)  // u alone: no W read, so no base variant
    return L.act_f32 ? small_launch(name, shape, flops, bytes, small_fwd<true, false, false, true>, grid, s, a)
                     : small_launch(name, shape, flops, bytes, small_fwd<false, false, false, true>, grid, s, a);
  const int v = (L.act_f32 ? 4 : 0) | (L.wbf ? 2 : 0) | (L.r > 0 ? 1 : 0);
  switch (v) {
    case 0: return small_launch(name, shape, flops, bytes, small_fwd<false, false, true, false>, grid, s, a);
    case 1: return small_launch(name, shape, flops, bytes, small_fwd<false, false, true, true>, grid, s, a);
    case 2: return small_launch(name, shape, flops, bytes, small_fwd<false, true, true, false>, grid, s, a);
    case 3: return small_launch(name, shape, flops, bytes, small_fwd<false, true, true, true>, grid, s, a);
    case 4: return small_launch(name, shape, flops, bytes, small_fwd<true, false, true, false>, grid, s, a);
    case 5: return small_launch(name, shape, flops, bytes, small_fwd<true, false, true, true>, grid, s, a);
    case 6: return small_launch(name, shape, flops, bytes, small_fwd<true, true, true, false>, grid, s, a);
    default: return small_launch(name, shape, flops, bytes, small_fwd<true, true, true, true>, grid, s, a);
  }
}

hipError_t launch_small_bwd(const SmallLinear& L, const void* dy, void* dx, int accumulate, float* du, hipStream_t s) {
  if (L.t == 0) return hipSuccess;
  if (L.r > SMALL_MAX_R || L.r % 4 || L.k % 64 || L.n % 64) return hipErrorInvalidValue;
  SmallBwdArgs a;
  memset(&a, 0, sizeof(a));
  a.dy = dy;
  a.codes = L.codes;
  a.absmax = L.absmax;
  a.wbf = L.wbf;
  a.A = L.A;
  a.B = L.B;
  a.dx = dx;
  a.du = du;
  a.T = L.t;
  a.K = L.k;
  a.N = L.n;
  a.r = L.r;
  a.lscale = L.lscale;
  a.out_f32 = L.out_f32;
  a.accumulate = accumulate;
  a.d = L.drop;
  a.lut = nf4_lut();
  const dim3 grid((unsigned)(L.k / SM_C), (unsigned)((L.t + SM_T - 1) / SM_T));
  const double flops = 2.0 * L.t * L.k * L.n;
  const double wb = L.wbf ? 2.0 * L.n * L.k : 0.5625 * L.n * L.k;
  const double ob = L.out_f32 ? 4.0 : 2.0;
  const double bytes = (double)L.t * L.n * (L.act_f32 ? 4 : 2) + wb + (double)L.t * L.k * ob * (accumulate ? 2 : 1) +
                       (L.r > 0 ? 4.0 * L.r * (L.k + L.n + L.t) : 0.0);
  char shape[48];
  snprintf(shape, sizeof(shape), "%lldx%lldx%lld r%d", (long long)L.t, (long long)L.k, (long long)L.n, L.r);
  const char* name = "small_bwd";
  const int v = (L.act_f32 ? 4 : 0) | (L.wbf ? 2 : 0) | (L.r > 0 ? 1 : 0);
  switch (v) {
    case 0: return small_launch(name, shape, flops, bytes, small_bwd<false, false, false>, grid, s, a);
    case 1: return small_launch(name, shape, flops, bytes, small_bwd<false, false, true>, grid, s, a);
    case 2: return small_launch(name, shape, flops, bytes, small_bwd<false, true, false>, grid, s, a);
    case 3: return small_launch(name, shape, flops, bytes, small_bwd<false, true, true>, grid, s, a);
    case 4: return small_launch(name, shape, flops, bytes, small_bwd<true, false, false>, grid, s, a);
    case 5: return small_launch(name, shape, flops, bytes, small_bwd<true, false, true>, grid, s, a);
    case 6: return small_launch(name, shape, flops, bytes, small_bwd<true, true, false>, grid, s, a);
    default: return small_launch(name, shape, flops, bytes, small_bwd<true, true, true>, grid, s, a);
  }
}

}  // namespace msq
