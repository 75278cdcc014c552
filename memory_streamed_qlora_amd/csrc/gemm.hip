// Fused NF4-dequant + bf16 MFMA GEMMs of the frozen base.
//
// Forward:  P[s][t][n] = sum_{k in split s} x[t][k]  * W[n][k]    ("NT")
// Backward: P[s][t][k] = sum_{n in split s} dy[t][n] * W[n][k]    ("NN", dx of the base)
// W is never materialised: each workgroup reads NF4 codes and per-64 absmax straight
// from HBM, builds the block's 16-entry bf16 table bf16_rne(L[c] * absmax), looks codes
// up four at a time with v_perm, and writes the bf16 tile into LDS in the layout the
// MFMA operand reads want; the contraction runs on v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  The pages' base is frozen (never differentiated: "Poros" research
// post, training-step paragraph), so there is no dW kernel.  The bf16_* kernels are the
// same GEMMs over a base kept in bf16 (the pages' bf16 streaming variant, "Current
// limitations", "bf16 LoRA"): each thread loads its 16 bf16 values of the tile and
// stores them into the same LDS layout, with no dequantization.
//
// Tile: BM=512 rows of t x BN=128 output columns x BK=64 reduction, 512 threads = 8
// waves; wave w owns rows 64w..64w+63 and all 128 columns (2x4 MFMA 32x32 blocks).
// The activation operand comes straight from global memory into registers, packed in
// MFMA-fragment order beforehand (launch_pack_lora) so that each load is one contiguous
// 1 KB block; only the dequantized W tile goes through LDS (three buffers, one
// barrier per k-step), and each dequantized element feeds all 512 rows.  Within a k-step,
// the dequantization of the next tile is interleaved with the MFMAs of this one.
// The rank-r LoRA term of the same output tile is one more MFMA k-step per 16 ranks
// (operands split into bf16 hi/lo pairs for ~fp32 accuracy); in the backward the
// dropout keep-mask is applied per element of that term.  Unsplit launches write the
// final output (bias added, then a residual or the old dx, rounded once); the reduction
// can instead be split over gridDim.z, in which case split 0 carries the LoRA term and
// fp32 partial tiles go to a workspace summed in split order by a separate kernel, so
// results never depend on timing.
#include <string.h>

#include <algorithm>

#include "internal.hpp"

namespace msq {
namespace {

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int PAD = 8;              // bf16 elements of row padding in LDS
constexpr int LDW = BK + PAD;       // LDS row pitch in bf16 elements (144 bytes)
static_assert(BM == 512 && BN == 128 && BK == 64, "the thread mappings below assume this tile");
constexpr int THREADS = 512;  // 8 waves, one per 64 rows

// One projection of a launch.  A forward launch may group up to GEMM_MAX_SEGS projections
// that share the activation (same K): their column tiles are concatenated in the grid and
// each workgroup finds its projection from its tile.  A backward launch may group the
// projections whose dx add up: their W rows are concatenated along the reduction, k-steps
// step0 .. of the packed dy belong to projection i, and every workgroup runs through all
// of them; the output fields of segment 0 describe dx.
struct GemmSeg {
  const uint8_t* codes;  // [N][K/2] NF4 base, or
  const float* absmax;   // [N][K/64]
  const uint16_t* wbf;   // [N][K] bf16 base (the bf16 kernels)
  // LoRA term, added once (by split 0):
  //   forward  lscale * lu[m][:] . lw[n][:]          lu = u [M][r], lw = B [N][r]
  //   backward keep(m,k) * sigma * lu[m][:] . lw[:][k]  lu = du [M][r], lw = A [r][K]
  const float* lu;
  const float* lw;
  Dropout drop;  // backward: keep mask of this projection's LoRA input gradient
  int step0;     // backward: first k-step of this projection's rows in the reduction
  // output: splits == 1 -> y / dx directly (bf16 or fp32): acc + bias, then addend + that
  //         when addend is set (forward: a residual input, added to y after y's own
  //         rounding; backward: the old dx, one rounding of the sum);
  //         splits  > 1 -> fp32 partials [splits][M][Nc]
  const uint16_t* bias;
  const void* addend;  // [M][Nc] in the output's type, may equal out
  void* out;
  int64_t Nc;          // output columns
  int tile0;           // first column tile of this projection in the grid
};

struct GemmArgs {
  const uint16_t* act;   // [M][R] bf16, packed
  int64_t M, K;          // every W is [N][K]
  int64_t R;             // reduction length
  int steps, steps_per_split, splits;
  Nf4Lut lut;
  int r;
  float lscale;
  int out_f32;
  int nseg;
  GemmSeg seg[GEMM_MAX_SEGS];
};

// The launch as the workgroup's projection sees it.
struct GemmView {
  const uint16_t* act;
  const uint8_t* codes;
  const float* absmax;
  const uint16_t* wbf;
  int64_t M, K, Nc;
  int steps;
  int r;
  float lscale;
  const uint16_t* bias;
  const void* addend;
  void* out;
  int out_f32;
};

// Eight fp32 values -> hi and lo bf16 MFMA operands, hi = rne(v), lo = rne(v - hi), so
// hi + lo = v to ~2^-16 relative; products of the pairs are exact in fp32, so
// hi*hi + hi*lo + lo*hi carries ~fp32 accuracy on the MFMA.
__device__ __forceinline__ void split8(const float (&v)[8], bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    l[i] = pack_bf16x2(v[2 * i] - bf16_to_f32(h[i] & 0xffffu), v[2 * i + 1] - bf16_to_f32(h[i] >> 16));
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
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

// Keep bits of the 16 accumulator rows a lane holds in one 32x32 block (bit v for
// register v), for output column n.  Element (m, n) draws word (m*Nc + n) % 4 of the
// Philox block (m*Nc + n) / 4; since Nc % 4 == 0, the four lanes of a quad (columns
// 4q..4q+3) share each row's block.  Lane p of the quad draws the blocks of rows
// 4p..4p+3 of the lane's register layout and the quad swaps results through DPP.
__device__ __forceinline__ uint32_t keep_rows16(const Dropout& d, int64_t mrow0, int hk, int64_t ncol,
                                                int64_t Nc, int lane) {
  const int p = lane & 3;
  const int64_t nq = ncol & ~(int64_t)3;
  uint32_t w = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int64_t m = mrow0 + 8 * p + 4 * hk + x;  // register v = 4p + x
    w |= keep4(d, (uint64_t)m * (uint64_t)Nc + (uint64_t)nq) << (4 * x);
  }
  const uint32_t w0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x00, 0xf, 0xf, false);
  const uint32_t w1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x55, 0xf, 0xf, false);
  const uint32_t w2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xaa, 0xf, 0xf, false);
  const uint32_t w3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xff, 0xf, 0xf, false);
  uint32_t bits = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    bits |= ((w0 >> (4 * x + p)) & 1u) << x;
    bits |= ((w1 >> (4 * x + p)) & 1u) << (4 + x);
    bits |= ((w2 >> (4 * x + p)) & 1u) << (8 + x);
    bits |= ((w3 >> (4 * x + p)) & 1u) << (12 + x);
  }
  return bits;
}

// One k-step's share of the W tile held in registers by one thread: 16 NF4 codes and
// their block's absmax, or 16 bf16 values.
template <bool BF16W>
struct WShare {
  uint2 q;
  float s;
};
template <>
struct WShare<true> {
  uint4 q[2];
};

template <int MODE, bool DROP, bool BF16W>
__device__ __forceinline__ void gemm_body(const GemmArgs& ga) {
  // W tiles [output column][k] with row pitch LDW; the backward's also start each group
  // of 16 columns 8 elements further (BSKEW), so that the transposed stores of a wave's
  // 8 column groups land on different banks
  constexpr int BSKEW = MODE == 1 ? 8 : 0;
  __shared__ __attribute__((aligned(16))) uint16_t sB[3][BN * LDW + BSKEW * (BN / 16)];
  // NF4: the codebook, and each thread's quarter of its row's bf16 table planes
  constexpr bool QUAD_TABLE = !BF16W;
  __shared__ __attribute__((aligned(16))) float sLut[QUAD_TABLE ? 16 : 1];
  __shared__ __attribute__((aligned(16))) uint2 sPl[QUAD_TABLE ? THREADS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hk = lane >> 5, r32 = lane & 31;
  if constexpr (QUAD_TABLE) {
    if (tid < 16) sLut[tid] = ga.lut.v[tid];
    __syncthreads();
  }
  int64_t n0, m0;
  int split;
  tile_of(n0, m0, split);
  // forward: this workgroup's projection (uniform), the last segment whose tiles start at
  // or before the tile; n0 becomes the column within it.  Backward: segment 0 holds dx.
  int sgi = 0;
  if (MODE == 0 && ga.nseg > 1 && n0 >= (int64_t)ga.seg[1].tile0 * BN) sgi = 1;
  if (MODE == 0 && ga.nseg > 2 && n0 >= (int64_t)ga.seg[2].tile0 * BN) sgi = 2;
  const GemmSeg& sg = ga.seg[sgi];
  n0 -= (int64_t)sg.tile0 * BN;
  const GemmView g{ga.act, sg.codes, sg.absmax, sg.wbf, ga.M, ga.K, sg.Nc, ga.steps, ga.r,
                   ga.lscale, sg.bias, sg.addend, sg.out, ga.out_f32};
  const int s_begin = split * ga.steps_per_split;
  const int s_end = min(ga.steps, s_begin + ga.steps_per_split);
  const int64_t mw = m0 + 64 * wave;  // first row of this wave

  // An asm operand in an AGPR lets the compiler place the MFMA accumulators in AGPRs
  // (128 AGPR + 128 VGPR at two waves per SIMD), which keeps the accumulator traffic of
  // every MFMA off the VGPR file that the dequantization and the loads use.  The
  // dropout variant needs more VGPRs in its epilogue and keeps them in VGPRs.
  if constexpr (!DROP) asm volatile("; mfma accumulators in AGPRs" ::"a"(0.0f));
  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  if (s_begin < s_end) {
    // Activation operand, straight from global memory into MFMA registers.  The operand
    // is packed in fragment order: within a k-step, MFMA sub-step c of lane half hk
    // reduces over k = 32*hk + 8*c + (0..7), and the 64 lanes' 16-byte pieces of one
    // (32-row group, k-step, sub-step) are one contiguous 1 KB block, so every load is
    // fully coalesced.  The W tile is read from LDS in the same k order.  Row groups past
    // the packed rows are clamped onto the last one: they only feed accumulator rows
    // that are never stored.
    const int64_t ngrp = (g.M + 31) / 32;
    const uint16_t* ap0 = g.act + min(mw / 32, ngrp - 1) * g.steps * 2048 + lane * 8;
    const uint16_t* ap1 = g.act + min(mw / 32 + 1, ngrp - 1) * g.steps * 2048 + lane * 8;

    // Source of this thread's share of the W tile (clamped like the rows above): 16
    // elements per k-step, as NF4 codes (one 8-byte load + the block's absmax) or bf16
    // values (two 16-byte loads).
    //   forward:  W row n0 + (tid >> 2), elements 16*(tid & 3) .. +15 of the step's block
    //   backward: reduction row 8*wave + (lane >> 3) of the step, output columns
    //             n0 + 16*(lane & 7) .. +15 (the 8 lanes of a row read its 64 code bytes, or
    //             256 bf16 bytes, as one piece; the 4 lanes of a 64-column block share its
    //             absmax, as in the forward)
    const uint8_t* cbase = nullptr;
    const float* sbase = nullptr;
    const uint16_t* wbase = nullptr;
    int64_t cstride = 0, sstride = 0, wstride = 0;
    int64_t coff = 0, soff = 0, woff = 0;  // backward: the thread's offsets within a projection's W
    if (MODE == 0) {
      const int64_t wn = min(n0 + (tid >> 2), g.Nc - 1);
      if constexpr (BF16W) {
        wbase = g.wbf + wn * g.K + 16 * (tid & 3);
        wstride = BK;
      } else {
        cbase = g.codes + wn * (g.K / 2) + 8 * (tid & 3);
        sbase = g.absmax + wn * (g.K / 64);
        cstride = BK / 2;
        sstride = 1;
      }
    } else {
      // offsets within a projection's W; the projection and its row base follow the step
      const int64_t wrow = 8 * wave + (lane >> 3), colq = n0 + 16 * (lane & 7);
      const int64_t col = colq < g.Nc ? colq : 0;
      if constexpr (BF16W) {
        woff = wrow * g.K + col;
        wstride = (int64_t)BK * g.K;
      } else {
        coff = wrow * (g.K / 2) + col / 2;
        soff = wrow * (g.K / 64) + col / 64;
        cstride = (int64_t)BK * (g.K / 2);
        sstride = (int64_t)BK * (g.K / 64);
      }
    }

    uint4 a[2][4];            // activation operand of the current k-step, refilled per sub-step
    WShare<BF16W> qa, qb;     // this thread's W share, alternating between k-steps
    auto load_a = [&](int step, int c) {
      const int64_t o = ((int64_t)step * 4 + c) * 512;
      a[0][c] = *reinterpret_cast<const uint4*>(ap0 + o);
      a[1][c] = *reinterpret_cast<const uint4*>(ap1 + o);
    };
    auto load_w = [&](WShare<BF16W>& w, int step) {
      if (MODE == 1) {
        // the projection whose rows the step covers (uniform): base + lane offset + rows
        const bool in2 = ga.nseg > 2 && step >= ga.seg[2].step0;
        const bool in1 = !in2 && ga.nseg > 1 && step >= ga.seg[1].step0;
        const int64_t ls = step - (in2 ? ga.seg[2].step0 : in1 ? ga.seg[1].step0 : 0);
        if constexpr (BF16W) {
          const uint16_t* wb = in2 ? ga.seg[2].wbf : in1 ? ga.seg[1].wbf : ga.seg[0].wbf;
          const uint16_t* p = wb + (woff + ls * wstride);
          w.q[0] = *reinterpret_cast<const uint4*>(p);
          w.q[1] = *reinterpret_cast<const uint4*>(p + 8);
        } else {
          const uint8_t* cb = in2 ? ga.seg[2].codes : in1 ? ga.seg[1].codes : ga.seg[0].codes;
          const float* sb = in2 ? ga.seg[2].absmax : in1 ? ga.seg[1].absmax : ga.seg[0].absmax;
          w.q = *reinterpret_cast<const uint2*>(cb + (coff + ls * cstride));
          w.s = sb[soff + ls * sstride];
        }
        return;
      }
      if constexpr (BF16W) {
        const uint16_t* p = wbase + (int64_t)step * wstride;
        w.q[0] = *reinterpret_cast<const uint4*>(p);
        w.q[1] = *reinterpret_cast<const uint4*>(p + 8);
      } else {
        w.q = *reinterpret_cast<const uint2*>(cbase + (int64_t)step * cstride);
        w.s = sbase[(int64_t)step * sstride];
      }
    };
    // Eight bf16 values (elements 8h .. 8h+7 of this thread's share, packed in pairs)
    // into LDS buffer `buf`.
    auto store8 = [&](const uint32_t (&out)[4], int h, int buf) {
      if (MODE == 0) {
        *reinterpret_cast<uint4*>(&sB[buf][(tid >> 2) * LDW + 16 * (tid & 3) + 8 * h]) =
            make_uint4(out[0], out[1], out[2], out[3]);
      } else {
        // transpose into [output column][reduction row]
        const int cg = lane & 7;
        uint16_t* dst = &sB[buf][(16 * cg + 8 * h) * LDW + BSKEW * cg + 8 * wave + (lane >> 3)];
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e * LDW] = (uint16_t)((e & 1) ? (out[e >> 1] >> 16) : out[e >> 1]);
      }
    };
    // Half h of a share -> bf16 in LDS: eight codes dequantized through the block's
    // planes, or eight bf16 values stored as they are.
    auto fill = [&](const Nf4Planes& P, const WShare<BF16W>& w, int h, int buf) {
      uint32_t out[4];
      if constexpr (BF16W) {
        const uint4 v = w.q[h];
        out[0] = v.x;
        out[1] = v.y;
        out[2] = v.z;
        out[3] = v.w;
      } else {
        nf4_dequant8(P, h ? w.q.y : w.q.x, out);
      }
      store8(out, h, buf);
    };
    // The four threads of a quad (lanes 4r .. 4r+3 of one wave) hold the same W row's
    // block (forward: the row's four 16-element pieces; backward: four 16-column pieces of
    // one 64-column block): each builds the table entries of codes 4q .. 4q+3 (q = tid & 3)
    // and the quad exchanges them through LDS, in place of each building all 16.  A wave's
    // LDS operations complete in order, so no barrier.
    auto planes = [&](const WShare<BF16W>& w) {
      Nf4Planes P;
      if constexpr (QUAD_TABLE) {
        const float4 L = *reinterpret_cast<const float4*>(&sLut[4 * (tid & 3)]);
        const uint32_t pk0 = pack_bf16x2(L.x * w.s, L.y * w.s), pk1 = pack_bf16x2(L.z * w.s, L.w * w.s);
        sPl[tid] = make_uint2(__builtin_amdgcn_perm(pk1, pk0, 0x06040200u), __builtin_amdgcn_perm(pk1, pk0, 0x07050301u));
        const uint4 r0 = *reinterpret_cast<const uint4*>(&sPl[tid & ~3]);
        const uint4 r1 = *reinterpret_cast<const uint4*>(&sPl[(tid & ~3) + 2]);
        P.lo[0] = r0.x;
        P.hi[0] = r0.y;
        P.lo[1] = r0.z;
        P.hi[1] = r0.w;
        P.lo[2] = r1.x;
        P.hi[2] = r1.y;
        P.lo[3] = r1.z;
        P.hi[3] = r1.w;
      } else if constexpr (!BF16W) {
        P = nf4_planes(ga.lut, w.s);
      }
      return P;
    };
    auto read_b = [&](bf16x8_t(&b)[4], int c, int buf) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(
            &sB[buf][(32 * j + r32) * LDW + BSKEW * ((32 * j + r32) >> 4) + 32 * hk + 8 * c]);
    };
    // Column-major MFMA order: operand b[j] is dead after its second MFMA, so the LDS
    // read that refills it for the next sub-step can be issued six MFMAs before use.
    auto mfma_sub = [&](const bf16x8_t(&b)[4], int c) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[i][c]), b[j], acc[i][j],
                                                              0, 0, 0);
    };
    // One k-step in four sub-steps.  The dequantized W tiles rotate through three LDS
    // buffers: k-step s multiplies on tile s while dequantizing tile s+2 (codes fetched
    // one k-step earlier) into the buffer tile s-1 has left, so tile s+1 is complete a
    // whole k-step before it is needed.  Sub-step c multiplies with operand column c
    // while the LDS operand of sub-step c+1 is read (for c = 3: sub-step 0 of tile s+1),
    // then refills a[][c] with the next k-step's activations (a full k-step ahead of
    // their use); sub-step 0 builds tile s+2's lookup table and sub-steps 1 and 2
    // dequantize its codes, so one wave's VALU work sits between its MFMAs.  The codes of tile s+3 go to the other register set (qn):
    // no register copies, so no wait on loads issued in this k-step.  Sub-steps are
    // fenced off from each other for the scheduler; nothing branches (past-the-end
    // fetches are clamped onto the last step and never read).
    bf16x8_t b0[4];
    int cur = 0;  // LDS buffer of the current tile
    auto kstep = [&](int step, const WShare<BF16W>& qc, WShare<BF16W>& qn) {
      const int nxt = min(step + 1, s_end - 1);
      const int b_next = cur == 2 ? 0 : cur + 1, b_fill = b_next == 2 ? 0 : b_next + 1;
      load_w(qn, min(step + 3, s_end - 1));
      Nf4Planes P;
      bf16x8_t b1[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        if (c == 0) P = planes(qc);
        if (c < 3)
          read_b((c & 1) ? b0 : b1, c + 1, cur);
        else
          read_b(b0, 0, b_next);  // tile s+1 is complete: its first operands load under these MFMAs
        mfma_sub((c & 1) ? b1 : b0, c);
        load_a(nxt, c);
        if (c == 1) fill(P, qc, 0, b_fill);
        if (c == 2) fill(P, qc, 1, b_fill);
        if (c < 3) {
          // one MFMA, then up to four of the sub-step's other VALU instructions (the table
          // build, the code lookups): both waves of a SIMD leave the barrier together, and a
          // wave that ran its VALU block first would leave the matrix core idle meanwhile
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      cur = b_next;
    };

    // Prologue: tiles s_begin and s_begin+1 into buffers 0 and 1; the codes of tile
    // s_begin+2 are fetched before the activations, the order the loop keeps them in
    // flight, so the wait counts the compiler derives at the loop head hold on entry
    // as well as on the back edge.
    {
      WShare<BF16W> t0, t1;
      load_w(t0, s_begin);
      load_w(t1, min(s_begin + 1, s_end - 1));
      load_w(qa, min(s_begin + 2, s_end - 1));
#pragma unroll
      for (int c = 0; c < 4; ++c) load_a(s_begin, c);
      const Nf4Planes P0 = planes(t0);
      fill(P0, t0, 0, 0);
      fill(P0, t0, 1, 0);
      const Nf4Planes P1 = planes(t1);
      fill(P1, t1, 0, 1);
      fill(P1, t1, 1, 1);
    }
    __syncthreads();
    read_b(b0, 0, 0);
    int step = s_begin;
    for (; step + 1 < s_end; step += 2) {
      kstep(step, qa, qb);
      kstep(step + 1, qb, qa);
    }
    if (step < s_end) kstep(step, qa, qb);
  }

  // ---- LoRA term: one extra MFMA k-step per 16 ranks, operands split hi/lo ---------------
  // Operands come straight from global memory in the MFMA lane layout: lane half hk
  // holds ranks rc + 8*hk .. +7 of its row (u side) or column (B / A side).
  // One projection's term, added by split 0; in a backward group split p adds projection
  // p's with its own factors and keep mask (a group's plan has a split per projection), so
  // no workgroup adds more than one (several terms in one workgroup keep enough values
  // live that the dropout variant spills).
  auto lora_term = [&](const float* lu, const float* lw, const Dropout& dr) {
      for (int rc = 0; rc < g.r; rc += 16) {
        bf16x8_t ah[2], al[2], bh[4], bl[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int64_t m = min(mw + 32 * i + r32, g.M - 1);
          float v[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int j = rc + 8 * hk + jj;
            const float x = lu[m * g.r + min(j, g.r - 1)];
            v[jj] = j < g.r ? g.lscale * x : 0.0f;
          }
          split8(v, ah[i], al[i]);
        }
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) {
          const int64_t n = min(n0 + 32 * jn + r32, g.Nc - 1);
          float v[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int j = rc + 8 * hk + jj;
            const int jc = min(j, g.r - 1);
            const float x = (MODE == 0) ? lw[n * g.r + jc] : lw[(int64_t)jc * g.K + n];
            v[jj] = j < g.r ? x : 0.0f;
          }
          split8(v, bh[jn], bl[jn]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jn = 0; jn < 4; ++jn) {
            if (!DROP) {
              f32x16_t t = acc[i][jn];
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[jn], t, 0, 0, 0);
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[jn], t, 0, 0, 0);
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[jn], t, 0, 0, 0);
              acc[i][jn] = t;
            } else {
              // masked LoRA input gradient: acc += keep * sigma * (du . A)
              f32x16_t t;
#pragma unroll
              for (int v = 0; v < 16; ++v) t[v] = 0.0f;
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[jn], t, 0, 0, 0);
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[jn], t, 0, 0, 0);
              t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[jn], t, 0, 0, 0);
              const uint32_t keep = keep_rows16(dr, mw + 32 * i, hk, n0 + 32 * jn + r32, g.Nc, lane);
#pragma unroll
              for (int v = 0; v < 16; ++v)
                if ((keep >> v) & 1u) acc[i][jn][v] += dr.sigma * t[v];
              __builtin_amdgcn_sched_barrier(0);  // one block's term live at a time
            }
          }
      }
  };
  if (g.r > 0) {
    if (MODE == 0) {
      if (split == 0) lora_term(sg.lu, sg.lw, sg.drop);
    } else {
      if (split < ga.nseg) {
        const bool s1 = split == 1, s2 = split == 2;  // uniform picks, no indexed segment
        Dropout dr;
        dr.k0 = s2 ? ga.seg[2].drop.k0 : s1 ? ga.seg[1].drop.k0 : ga.seg[0].drop.k0;
        dr.k1 = s2 ? ga.seg[2].drop.k1 : s1 ? ga.seg[1].drop.k1 : ga.seg[0].drop.k1;
        dr.c1 = s2 ? ga.seg[2].drop.c1 : s1 ? ga.seg[1].drop.c1 : ga.seg[0].drop.c1;
        dr.c2 = s2 ? ga.seg[2].drop.c2 : s1 ? ga.seg[1].drop.c2 : ga.seg[0].drop.c2;
        dr.c3 = s2 ? ga.seg[2].drop.c3 : s1 ? ga.seg[1].drop.c3 : ga.seg[0].drop.c3;
        dr.threshold = s2 ? ga.seg[2].drop.threshold : s1 ? ga.seg[1].drop.threshold : ga.seg[0].drop.threshold;
        dr.sigma = s2 ? ga.seg[2].drop.sigma : s1 ? ga.seg[1].drop.sigma : ga.seg[0].drop.sigma;
        lora_term(s2 ? ga.seg[2].lu : s1 ? ga.seg[1].lu : ga.seg[0].lu,
                  s2 ? ga.seg[2].lw : s1 ? ga.seg[1].lw : ga.seg[0].lw, dr);
      }
    }
  }

  // ---- output ---------------------------------------------------------------------------
  // One 32x32 block at a time through LDS: the wave writes its block into a 32 x 36 fp32
  // staging area (the W buffers are free once every wave has left the main loop), then
  // stores whole rows as float4, four rows of the block per pass, guarded per row.  The
  // per-element stores straight from the accumulator layout needed a branch per element
  // and a separate copy of that code for each output form; the kernel then ran to ~15k
  // instructions, most of them executed once per workgroup from a cold instruction cache.
  // Column blocks are never partial: Nc is a multiple of 64.
  __syncthreads();
  constexpr int SP = 36;  // staging row pitch in floats (keeps float4 rows aligned)
  float* stage = reinterpret_cast<float*>(&sB[0][0]) + wave * (32 * SP);
  const int srow = lane >> 3, scol = 4 * (lane & 7);  // this lane's row (of 8) and column quad
  auto store_block = [&](const f32x16_t& blk, int i, int jn) {
    __builtin_amdgcn_sched_barrier(0);
    const int64_t nb = n0 + 32 * jn;  // first column of the block
    if (nb >= g.Nc) return;            // uniform
#pragma unroll
    for (int v = 0; v < 16; ++v) stage[(8 * (v >> 2) + 4 * hk + (v & 3)) * SP + r32] = blk[v];
    const int64_t n = nb + scol;
    float bn[4] = {0.f, 0.f, 0.f, 0.f};
    if (MODE == 0 && g.bias && ga.splits == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) bn[q] = bf16_to_f32(g.bias[n + q]);
    }
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int row = srow + 8 * pass;
      const int64_t m = mw + 32 * i + row;
      const float4 a4 = *reinterpret_cast<const float4*>(&stage[row * SP + scol]);
      if (m >= g.M) continue;
      if (ga.splits > 1) {
        float* po = reinterpret_cast<float*>(g.out) + ((int64_t)split * g.M + m) * g.Nc + n;
        *reinterpret_cast<float4*>(po) = a4;
        continue;
      }
      float val[4] = {a4.x + bn[0], a4.y + bn[1], a4.z + bn[2], a4.w + bn[3]};
      if (g.out_f32) {
        float* po = reinterpret_cast<float*>(g.out) + m * g.Nc + n;
        if (g.addend) {
          const float4 o = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(g.addend) + m * g.Nc + n);
          val[0] = o.x + val[0];
          val[1] = o.y + val[1];
          val[2] = o.z + val[2];
          val[3] = o.w + val[3];
        }
        *reinterpret_cast<float4*>(po) = make_float4(val[0], val[1], val[2], val[3]);
      } else {
        uint16_t* po = reinterpret_cast<uint16_t*>(g.out) + m * g.Nc + n;
        if (g.addend) {
          // forward residual: y is rounded first, as a separate add would see it;
          // backward accumulate: one rounding of the fp32 sum
          const uint2 o = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(g.addend) + m * g.Nc + n);
          const float old[4] = {bf16_to_f32(o.x & 0xffffu), bf16_to_f32(o.x >> 16), bf16_to_f32(o.y & 0xffffu),
                                bf16_to_f32(o.y >> 16)};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (MODE == 0) val[q] = bf16_to_f32(bf16_rne(val[q]));
            val[q] = old[q] + val[q];
          }
        }
        *reinterpret_cast<uint2*>(po) =
            make_uint2(bf16_rne(val[0]) | (bf16_rne(val[1]) << 16), bf16_rne(val[2]) | (bf16_rne(val[3]) << 16));
      }
    }
  };
  store_block(acc[0][0], 0, 0);
  store_block(acc[0][1], 0, 1);
  store_block(acc[0][2], 0, 2);
  store_block(acc[0][3], 0, 3);
  store_block(acc[1][0], 1, 0);
  store_block(acc[1][1], 1, 1);
  store_block(acc[1][2], 1, 2);
  store_block(acc[1][3], 1, 3);
}

#define MSQ_GEMM_KERNEL(name, MODE, DROP, BF16W) \
  __global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2))) void name(GemmArgs g) { \
    gemm_body<MODE, DROP, BF16W>(g);                                                                       \
  }
MSQ_GEMM_KERNEL(nf4_fwd_gemm, 0, false, false)
MSQ_GEMM_KERNEL(nf4_bwd_gemm, 1, false, false)
MSQ_GEMM_KERNEL(nf4_bwd_gemm_dropout, 1, true, false)
MSQ_GEMM_KERNEL(bf16_fwd_gemm, 0, false, true)
MSQ_GEMM_KERNEL(bf16_bwd_gemm, 1, false, true)
MSQ_GEMM_KERNEL(bf16_bwd_gemm_dropout, 1, true, true)
#undef MSQ_GEMM_KERNEL

}  // namespace

// Split of the reduction dimension.  Cost model per candidate split S: a k-step of one
// workgroup keeps its CU's matrix cores busy for ~1 us (64 MFMAs per SIMD), the
// workgroups spread evenly over the 256 CUs, and every extra split writes and re-reads
// an fp32 partial tile at ~8 TB/s (the partials are re-read while still in the L2 and
// last-level caches; measured at the 32B shapes, this rate picks the fastest S of every
// one of them).  The cheapest S wins; the smallest on ties.
GemmPlan gemm_plan_tiles(int64_t m, int64_t n_tiles, int64_t nc, int64_t red, int min_splits) {
  GemmPlan p;
  p.steps = (int)(red / BK);
  const int64_t tiles = ((m + BM - 1) / BM) * n_tiles;
  const int s0 = std::max(1, std::min(min_splits, p.steps));
  double best = 0.0;
  int best_s = s0;
  for (int s = s0; s <= 32 && s <= p.steps; ++s) {
    const int64_t per = (p.steps + s - 1) / s;
    if (s > s0 && (per < 4 || (int64_t)(s - 1) * per >= p.steps)) continue;  // no empty or tiny splits
    const double per_cu = (double)((tiles * s + 255) / 256);
    const double t = per_cu * (double)per * 1.0 + (s > 1 ? (double)s * (double)m * (double)nc * 8.0 / 8e6 : 0.0);
    if (s == s0 || t < best) {
      best = t;
      best_s = s;
    }
  }
  p.splits = best_s;
  p.steps_per_split = (p.steps + best_s - 1) / best_s;
  return p;
}

GemmPlan gemm_plan(int64_t m, int64_t nc, int64_t red, int min_splits) {
  return gemm_plan_tiles(m, (nc + BN - 1) / BN, nc, red, min_splits);
}

GemmPlan gemm_plan_group(int64_t m, const int64_t* ns, int nseg, int64_t red) {
  int64_t tiles = 0, nc = 0;
  for (int i = 0; i < nseg; ++i) {
    tiles += (ns[i] + BN - 1) / BN;
    nc += ns[i];
  }
  return gemm_plan_tiles(m, tiles, nc, red, 1);
}

hipError_t launch_gemm(const GemmLaunch& L, hipStream_t s) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  if (L.nseg < 1 || L.nseg > GEMM_MAX_SEGS) return hipErrorInvalidValue;
  const bool bf = L.seg[0].wbf != nullptr;
  g.act = L.act;
  g.M = L.M;
  g.K = L.K;
  g.R = 0;
  for (int i = 0; i < L.nseg && L.mode == 1; ++i) {
    if (L.seg[i].N % BK) return hipErrorInvalidValue;  // a k-step never straddles two projections
    g.seg[i].step0 = (int)(g.R / BK);
    g.R += L.seg[i].N;
  }
  if (L.mode == 0) g.R = L.K;
  g.steps = L.plan.steps;
  g.steps_per_split = L.plan.steps_per_split;
  g.splits = L.plan.splits;
  g.lut = nf4_lut();
  g.r = L.r;
  g.lscale = L.lscale;
  g.out_f32 = L.out_f32;
  g.nseg = L.nseg;
  int tiles = 0;
  int64_t n_total = 0;
  bool drop_any = false;
  for (int i = 0; i < L.nseg; ++i) {
    const GemmSegment& S = L.seg[i];
    if ((S.wbf != nullptr) != bf || (S.codes != nullptr) == bf) return hipErrorInvalidValue;  // one base format
    GemmSeg& d = g.seg[i];
    d.codes = S.codes;
    d.absmax = S.absmax;
    d.wbf = S.wbf;
    d.lu = S.lu;
    d.lw = S.lw;
    d.drop = S.drop;
    d.bias = S.bias;
    d.addend = S.addend;
    d.out = S.out;
    d.Nc = L.mode == 0 ? S.N : L.K;
    d.tile0 = L.mode == 0 ? tiles : 0;
    if (d.Nc < 1) return hipErrorInvalidValue;
    if (L.mode == 0 || i == 0) tiles += (int)((d.Nc + BN - 1) / BN);
    if (S.drop.threshold != 0u) drop_any = true;
    n_total += S.N;
  }
  // The kernel clamps rows and columns onto [0, M) x [0, Nc) and reads whole k-steps; a
  // backward group's split p adds projection p's LoRA term.
  if (g.M < 1 || g.R % BK || g.K % 64 || g.steps != (int)(g.R / BK)) return hipErrorInvalidValue;
  if (L.mode == 1 && g.splits < g.nseg) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles, (unsigned)((g.M + BM - 1) / BM), (unsigned)g.splits);
  const double flops = 2.0 * (double)g.M * (double)n_total * (double)g.K;
  void (*kern)(GemmArgs);
  const char* name;
  if (L.mode == 0) {
    kern = bf ? bf16_fwd_gemm : nf4_fwd_gemm;
    name = bf ? "bf16_fwd_gemm" : "nf4_fwd_gemm";
  } else if (L.r > 0 && drop_any) {
    kern = bf ? bf16_bwd_gemm_dropout : nf4_bwd_gemm_dropout;
    name = bf ? "bf16_bwd_gemm" : "nf4_bwd_gemm";
  } else {
    kern = bf ? bf16_bwd_gemm : nf4_bwd_gemm;
    name = bf ? "bf16_bwd_gemm" : "nf4_bwd_gemm";
  }
  // algorithmic bytes: the base (NF4 codes + scales, or bf16), the packed activation, the
  // output (or split partials)
  double out_bytes = 0.0;
  for (int i = 0; i < (L.mode == 0 ? L.nseg : 1); ++i)
    out_bytes += (double)g.M * g.seg[i].Nc *
                 (g.splits > 1 ? 4.0 * g.splits : (g.out_f32 ? 4.0 : 2.0) * (g.seg[i].addend ? 2 : 1));
  const double bytes = (double)n_total * g.K * (bf ? 2.0 : 0.5625) + (double)frag_rows(g.M) * g.R * 2 + out_bytes;
  char shape[40];
  snprintf(shape, sizeof(shape), "%lldx%lldx%lld", (long long)L.M, (long long)n_total, (long long)L.K);
  return timed_launch(name, shape, flops, bytes, kern, grid, dim3(THREADS), s, g);
}

}  // namespace msq
