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
#include "split_bf16.hpp"

namespace msq {
namespace {

constexpr int SM_T = 64;       // tokens per workgroup
constexpr int SM_C = 64;       // output (forward) or input (backward) columns per workgroup
constexpr int SM_WAVES = 4;
constexpr int SM_BLK = 16 * 64;  // one 32 x 32 fp32 block in register order: [v][lane]


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

// The activation tile of a k-step (64 tokens x 64 columns, bf16 or fp32) is loaded with
// whole rows per instruction (8 or 4 rows of 128 or 256 bytes per 64 lanes) into the wave's
// own LDS tile, and the MFMA operands are read from there: a load whose 64 lanes each
// fetch 16 bytes of a different row touches 32 cache lines and runs the vector memory
// path at a fraction of its rate, which bounded the k-step before.  The LoRA factor's
// rows (A in the forward, B in the backward) go through LDS the same way.  Each wave uses
// only its own tiles: a fence and a wave barrier order its LDS stores before its reads
// and its reads before the next k-step's stores.
template <bool XF32>
struct ActTile {
  static constexpr int PITCH = XF32 ? 68 : 36;     // dwords per row (16-byte aligned rows)
  static constexpr int WORDS = 64 * PITCH;
  static constexpr int PIECES = XF32 ? 16 : 8;     // 16-byte loads per lane for the tile
  static constexpr int ROWS_PER = XF32 ? 4 : 8;    // rows per 64-lane load
  static constexpr int LANES_PER_ROW = XF32 ? 16 : 8;
};
constexpr int SM_FT = 32 * 68;  // a factor tile in floats: 32 ranks x 64 columns (+4 pad)
// 16 bytes as a plain vector (a struct-typed copy of HIP's uint4 is lowered to a memory
// copy that keeps the staged tile in scratch)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Loads of a tile: lane l, piece p -> row p * ROWS_PER + l / LANES_PER_ROW, 16 bytes at
// column (l % LANES_PER_ROW) * 16 bytes.  Rows past `last` re-read `last` (in bounds).
template <bool XF32>
__device__ __forceinline__ void act_tile_load(u32x4_t (&q)[ActTile<XF32>::PIECES], const void* base, int64_t row0,
                                              int64_t last, int64_t stride, int64_t col0, int lane) {
  using AT = ActTile<XF32>;
#pragma unroll
  for (int p = 0; p < AT::PIECES; ++p) {
    const int64_t row = min(row0 + p * AT::ROWS_PER + lane / AT::LANES_PER_ROW, last);
    const int64_t e = row * stride + col0 + (lane % AT::LANES_PER_ROW) * (XF32 ? 4 : 8);  // element index
    if (XF32)
      q[p] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const float*>(base) + e);
    else
      q[p] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(base) + e);
  }
}
template <bool XF32>
__device__ __forceinline__ void act_tile_store(uint32_t* t, const u32x4_t (&q)[ActTile<XF32>::PIECES], int lane) {
  using AT = ActTile<XF32>;
#pragma unroll
  for (int p = 0; p < AT::PIECES; ++p) {
    const int row = p * AT::ROWS_PER + lane / AT::LANES_PER_ROW;
    *reinterpret_cast<u32x4_t*>(&t[row * AT::PITCH + (lane % AT::LANES_PER_ROW) * 4]) = q[p];
  }
}
// The 8 activation values of (tile row `row`, columns 32 hk + 8 c .. + 7) as the bf16
// MFMA operand: the values themselves (bf16 tile), or their hi and lo parts (fp32 tile).
template <bool XF32>
__device__ __forceinline__ void act_operand(const uint32_t* t, int row, int hk, int c, bf16x8_t& hi, bf16x8_t& lo) {
  using AT = ActTile<XF32>;
  if (XF32) {
    const float4 v0 = *reinterpret_cast<const float4*>(&t[row * AT::PITCH + 32 * hk + 8 * c]);
    const float4 v1 = *reinterpret_cast<const float4*>(&t[row * AT::PITCH + 32 * hk + 8 * c + 4]);
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    split8_bf16(v, hi, lo);
  } else {
    hi = *reinterpret_cast<const bf16x8_t*>(&t[row * AT::PITCH + 16 * hk + 4 * c]);
  }
}
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

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
  int out_f32, u_only, u_given;  // u_given: u holds u (read, not written)
  Dropout d;
  Nf4Lut lut;
};

// LDS of small_fwd: in the loop each wave has its activation tile and its A tile; after
// it, the waves' partial blocks (6 per wave) and a u staging block per wave.
template <bool XF32>
struct FwdLds {
  static constexpr int LOOP = SM_WAVES * (ActTile<XF32>::WORDS + SM_FT);
  static constexpr int END = SM_WAVES * 6 * SM_BLK + SM_WAVES * 32 * 33;
  static constexpr int WORDS = LOOP > END ? LOOP : END;
};

// MAIN: y is formed (false: u alone); LORA: r > 0.  Both are template parameters so that
// every load of a k-step is unconditional and the compiler counts them exactly (a load
// under a runtime branch makes it wait for all of them, the prefetched step included).
template <bool XF32, bool BF16W, bool MAIN, bool LORA>
__global__ __launch_bounds__(256) void small_fwd(SmallFwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[FwdLds<XF32>::WORDS];
  using AT = ActTile<XF32>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hk = lane >> 5, r32 = lane & 31;
  const int64_t n0 = (int64_t)blockIdx.x * SM_C, m0 = (int64_t)blockIdx.y * SM_T;
  const int64_t T = a.T, K = a.K, N = a.N;
  const int steps = (int)(K / 64), r = a.r;
  constexpr bool main = MAIN, lora = LORA;
  const Dropout d = a.d;
  uint32_t* xt = lds + wave * (AT::WORDS + SM_FT);
  float* at = reinterpret_cast<float*>(xt + AT::WORDS);
  // the lane's two W rows; its rank in the u product; the rows of its activation operand
  const int64_t wn0 = n0 + r32, wn1 = n0 + 32 + r32;
  const bool rk_ok = r32 < r;
  const int rkc = min(r32, max(r - 1, 0));
  const int64_t mr0 = min(m0 + r32, T - 1), mr1 = min(m0 + 32 + r32, T - 1);

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

  // One k-step's loads: the activation tile (whole rows), the lane's two W rows (codes and
  // scales, or bf16 values), the A tile (4 rank rows of 64 columns per 64-lane load; rows
  // past r re-read row r - 1 and are never used).  The next k-step of the wave is loaded
  // before this one is multiplied.
  constexpr int WQ = BF16W ? 4 : 1;
  struct Stage {
    u32x4_t xq[AT::PIECES];
    u32x4_t wq[2][WQ];
    float ws[2];
    f32x4_t aq[8];
  };
  auto load = [&](Stage& st, int s) {
    const int64_t k0 = (int64_t)s * 64, kc = k0 + 32 * hk;
    act_tile_load<XF32>(st.xq, a.x, m0, T - 1, K, k0, lane);
    if (main) {
#pragma unroll
      for (int q = 0; q < WQ; ++q) {
        if (BF16W) {
          st.wq[0][q] = reinterpret_cast<const u32x4_t*>(a.wbf + wn0 * K + kc)[q];
          st.wq[1][q] = reinterpret_cast<const u32x4_t*>(a.wbf + wn1 * K + kc)[q];
        } else {
          st.wq[0][q] = *reinterpret_cast<const u32x4_t*>(a.codes + wn0 * (K / 2) + kc / 2);
          st.wq[1][q] = *reinterpret_cast<const u32x4_t*>(a.codes + wn1 * (K / 2) + kc / 2);
        }
      }
      if (!BF16W) {
        st.ws[0] = a.absmax[wn0 * (K / 64) + s];
        st.ws[1] = a.absmax[wn1 * (K / 64) + s];
      }
    }
    if (lora) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int rank = min(4 * q + (lane >> 4), r - 1);
        st.aq[q] = *reinterpret_cast<const f32x4_t*>(a.A + (int64_t)rank * K + k0 + 4 * (lane & 15));
      }
    }
  };
  auto compute = [&](const Stage& st, int s) {
    const int64_t kc = (int64_t)s * 64 + 32 * hk;
    // the tiles into LDS (the previous k-step's reads of them are complete)
    act_tile_store<XF32>(xt, st.xq, lane);
    if (lora) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        *reinterpret_cast<f32x4_t*>(&at[(4 * q + (lane >> 4)) * 68 + 4 * (lane & 15)]) = st.aq[q];
    }
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
          nf4_dequant32(P, make_uint4(st.wq[j][0].x, st.wq[j][0].y, st.wq[j][0].z, st.wq[j][0].w), wb[j]);
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
    wave_sync_lds();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t ax[2], axl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) act_operand<XF32>(xt, 32 * i + r32, hk, c, ax[i], axl[i]);
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
        const float4 a0 = *reinterpret_cast<const float4*>(&at[rkc * 68 + 32 * hk + 8 * c]);
        const float4 a1 = *reinterpret_cast<const float4*>(&at[rkc * 68 + 32 * hk + 8 * c + 4]);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        float avz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) avz[e] = rk_ok ? av[e] : 0.0f;
        bf16x8_t ah, al;
        split8_bf16(avz, ah, al);
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
    wave_sync_lds();  // this k-step's tile reads are complete before the next one's stores
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
  f32x16_t y, uf;
  const float usig = d.threshold != 0u ? d.sigma : 1.0f;
  const int64_t rb = m0 + 32 * oi;  // first token row of the block
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    y[v] = wsum(oi + 2 * oj, v);
    uf[v] = lora ? usig * wsum(4 + oi, v) : 0.0f;
  }
  if (lora && a.u_given) {  // u from an earlier call in place of the one formed above
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = rb + sm_row(v, hk);
      uf[v] = (rk_ok && m < T) ? a.u[m * r + r32] : 0.0f;
    }
  }
  if (lora && a.u && !a.u_given && blockIdx.x == 0 && oj == 0 && rk_ok) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = rb + sm_row(v, hk);
      if (m < T) a.u[m * r + r32] = uf[v];
    }
  }
  if (!main) return;

  // ---- LoRA term: y += (alpha / r) u B^T, u through LDS into the operand layout -------
  if (lora) {
    float* us = red + SM_WAVES * 6 * SM_BLK + wave * 32 * 33;
#pragma unroll
    for (int v = 0; v < 16; ++v) us[sm_row(v, hk) * 33 + r32] = a.lscale * uf[v];
    wave_sync_lds();
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
      split8_bf16(uv, uh, ul);
      split8_bf16(bpre[h], bh, bl);
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

// LDS of small_bwd: in the loop each wave has its dy tile, a W^T tile (64 input columns x
// 32 bf16 pairs of W rows, pitch 36 dwords) and a B^T tile (32 ranks x 64 W rows fp32,
// pitch 68); after it, the waves' partial blocks (6 per wave) and a du staging block per
// wave.
constexpr int SB_WT = 64 * 36;  // dwords per wave
template <bool XF32>
struct BwdLds {
  static constexpr int LOOP = SM_WAVES * (ActTile<XF32>::WORDS + SB_WT + SM_FT);
  static constexpr int END = SM_WAVES * 6 * SM_BLK + SM_WAVES * 32 * 33;
  static constexpr int WORDS = LOOP > END ? LOOP : END;
};

// LORA: r > 0 (then r % 4 == 0).  A template parameter for the reason given at small_fwd.
template <bool XF32, bool BF16W, bool LORA>
__global__ __launch_bounds__(256) void small_bwd(SmallBwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[BwdLds<XF32>::WORDS];
  using AT = ActTile<XF32>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hk = lane >> 5, r32 = lane & 31;
  const int64_t k0 = (int64_t)blockIdx.x * SM_C, m0 = (int64_t)blockIdx.y * SM_T;
  const int64_t T = a.T, K = a.K, N = a.N;
  const int steps = (int)(N / 64), r = a.r;
  constexpr bool lora = LORA;
  uint32_t* yt = lds + wave * (AT::WORDS + SB_WT + SM_FT);
  uint32_t* wt = yt + AT::WORDS;
  float* bt = reinterpret_cast<float*>(wt + SB_WT);
  // the W rows this lane dequantizes: 2 (lane & 31) and the next, columns k0 + 32 hk ..
  const int pr = 2 * r32;
  const bool rk_ok = r32 < r;
  const int rkc = min(r32, max(r - 1, 0));
  const int rq = max(r / 4, 1);  // 16-byte pieces of a B row

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

  // One reduction step's loads: the dy tile (whole rows), two W rows over the lane's 32
  // input columns, the step's 64 rows of B (one contiguous block of 64 r floats: 16 bytes
  // per lane and piece, pieces past the block re-read its last one and are not stored).
  constexpr int WQ = BF16W ? 8 : 1;
  struct Stage {
    u32x4_t xq[AT::PIECES];
    u32x4_t wq[2][WQ];
    float ws[2];
    f32x4_t bq[8];
  };
  auto load = [&](Stage& st, int s) {
    act_tile_load<XF32>(st.xq, a.dy, m0, T - 1, N, (int64_t)s * 64, lane);
    const int64_t wr = (int64_t)s * 64 + pr;
    const int64_t kk = k0 + 32 * hk;
    if (BF16W) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        st.wq[0][q] = reinterpret_cast<const u32x4_t*>(a.wbf + wr * K + kk)[q];
        st.wq[1][q] = reinterpret_cast<const u32x4_t*>(a.wbf + (wr + 1) * K + kk)[q];
      }
    } else {
      st.wq[0][0] = *reinterpret_cast<const u32x4_t*>(a.codes + wr * (K / 2) + kk / 2);
      st.wq[1][0] = *reinterpret_cast<const u32x4_t*>(a.codes + (wr + 1) * (K / 2) + kk / 2);
      st.ws[0] = a.absmax[wr * (K / 64) + k0 / 64];
      st.ws[1] = a.absmax[(wr + 1) * (K / 64) + k0 / 64];
    }
    if (lora) {
      const float* blk = a.B + (int64_t)s * 64 * r;
#pragma unroll
      for (int q = 0; q < 8; ++q) st.bq[q] = *reinterpret_cast<const f32x4_t*>(blk + 4 * (64 * min(q, rq - 1) + lane));
    }
  };
  auto compute = [&](const Stage& st) {
    act_tile_store<XF32>(yt, st.xq, lane);
    // W^T: input column 32 hk + e gets the bf16 pair (row 2 r32, row 2 r32 + 1) at pair r32
    uint32_t w0[16], w1[16];
    if (BF16W) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w0[4 * q] = st.wq[0][q].x; w0[4 * q + 1] = st.wq[0][q].y; w0[4 * q + 2] = st.wq[0][q].z; w0[4 * q + 3] = st.wq[0][q].w;
        w1[4 * q] = st.wq[1][q].x; w1[4 * q + 1] = st.wq[1][q].y; w1[4 * q + 2] = st.wq[1][q].z; w1[4 * q + 3] = st.wq[1][q].w;
      }
    } else {
      nf4_dequant32(nf4_planes(a.lut, st.ws[0]),
                    make_uint4(st.wq[0][0].x, st.wq[0][0].y, st.wq[0][0].z, st.wq[0][0].w), w0);
      nf4_dequant32(nf4_planes(a.lut, st.ws[1]),
                    make_uint4(st.wq[1][0].x, st.wq[1][0].y, st.wq[1][0].z, st.wq[1][0].w), w1);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      wt[(32 * hk + 2 * q) * 36 + r32] = __builtin_amdgcn_perm(w1[q], w0[q], 0x05040100u);
      wt[(32 * hk + 2 * q + 1) * 36 + r32] = __builtin_amdgcn_perm(w1[q], w0[q], 0x07060302u);
    }
    if (lora) {
      // B block floats f = 4 (64 q + lane) + e: W row f / r of the step, rank f % r
      // pieces past the block hold piece rq - 1 again and store the same values to the
      // same places (unconditional: a load consumed under a branch would make the compiler
      // wait for every load in flight at the top of the next step)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int f = 4 * (64 * min(q, rq - 1) + lane);
        const int row = f / r, j = f - row * r;
        bt[j * 68 + row] = st.bq[q].x;
        bt[(j + 1) * 68 + row] = st.bq[q].y;
        bt[(j + 2) * 68 + row] = st.bq[q].z;
        bt[(j + 3) * 68 + row] = st.bq[q].w;
      }
    }
    wave_sync_lds();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t ax[2], axl[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) act_operand<XF32>(yt, 32 * i + r32, hk, c, ax[i], axl[i]);
      // W^T operand of column block j: column 32 j + r32, reduction rows 32 hk + 8 c .. + 7
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(&wt[(32 * j + r32) * 36 + 16 * hk + 4 * c]);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[i], b, acc[i][j], 0, 0, 0);
      }
      if (lora) {
        const float4 b0 = *reinterpret_cast<const float4*>(&bt[rkc * 68 + 32 * hk + 8 * c]);
        const float4 b1 = *reinterpret_cast<const float4*>(&bt[rkc * 68 + 32 * hk + 8 * c + 4]);
        float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = rk_ok ? bv[e] : 0.0f;
        bf16x8_t bh, bl;
        split8_bf16(bv, bh, bl);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[i], bh, ua[i], 0, 0, 0);
          ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax[i], bl, ua[i], 0, 0, 0);
          if (XF32) ua[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(axl[i], bh, ua[i], 0, 0, 0);
        }
      }
    }
    wave_sync_lds();  // this step's tile reads are complete before the next one's stores
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
      split8_bf16(uv, uh, ul);
      split8_bf16(apre[h], ah, al);
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
                            float* u, bool u_only, bool u_given, hipStream_t s) {
  if (L.t == 0) return hipSuccess;
  if (L.r > SMALL_MAX_R || L.r % 4 || L.k % 64 || L.n % 64) return hipErrorInvalidValue;
  if (u_given && (u_only || !u || L.r == 0)) return hipErrorInvalidValue;
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
  a.u_given = u_given;
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
