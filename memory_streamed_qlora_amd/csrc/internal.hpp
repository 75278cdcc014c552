// Host-side internals of libmsq: launch wrappers, planning, errors, timing.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "device_common.hpp"

namespace msq {

// ---- errors ---------------------------------------------------------------
int set_error(int code, const char* fmt, ...);  // records thread-local text, returns code
int hip_error(hipError_t e, const char* what);   // MSQ_E_HIP with the HIP error string

// ---- codebook (computed on the host from the NormalFloat construction) -----
const Nf4Lut& nf4_lut();
const Nf4Mid& nf4_mid();

// ---- workspace planning ----------------------------------------------------
constexpr int GEMM_BM = 512;
constexpr int GEMM_BN = 128;
constexpr int GEMM_BK = 64;

struct GemmPlan {
  int splits;          // split of the reduction dimension
  int steps;           // reduction steps of GEMM_BK
  int steps_per_split;
};
// Split plan of an m x nc output over a reduction of red; min_splits (at most the k-step
// count) is the fewest splits allowed: a backward group needs one per projection.
GemmPlan gemm_plan(int64_t m, int64_t nc, int64_t red, int min_splits = 1);
GemmPlan gemm_plan_group(int64_t m, const int64_t* ns, int nseg, int64_t red);

struct LoraPlan {
  GemmPlan fwd, bwd;
  size_t off_part_fwd, off_u_fwd, off_act_fwd, off_sk_fwd;                   // fwd layout
  size_t off_part_bwd, off_u_bwd, off_du, off_act_bwd, off_sk_bwd;  // bwd layout
  size_t fwd_bytes, bwd_bytes;
};
LoraPlan lora_plan(int64_t t, int64_t k, int64_t n, int32_t r);

// ---- launch wrappers (all asynchronous on `s`) -------------------------------
hipError_t launch_quantize(const uint16_t* w, int64_t nblocks, uint8_t* codes, float* absmax,
                           hipStream_t s);
hipError_t launch_dequantize(const uint8_t* codes, const float* absmax, int64_t nchunks32,
                             uint16_t* w, hipStream_t s);

// Fused dequant-MFMA product with the LoRA term of the same tile.
//   mode 0 (forward):  y[m][n]  = [addend +] (sum_k act[m][k] W[n][k] + lscale * lu[m] . lw[n] + bias[n])
//   mode 1 (backward): dx[m][k] = [addend +] (sum_n act[m][n] W[n][k] + keep*sigma * lu[m] . lw[:,k])
// addend ([M][Nc] in the output's type, NULL for none) may be `out` itself.
// With plan.splits > 1, `out` receives fp32 partials [splits][M][Nc] instead (split 0
// carrying the LoRA term) and launch_split_reduce finishes the output.
// A launch may group up to GEMM_MAX_SEGS projections of the same input (same K):
//   forward:  each with its own base, LoRA factors, bias, addend and output; one grid over
//             all their column tiles, one split plan (gemm_plan_group);
//   backward: their contributions to the one dx: the reduction runs over the projections'
//             rows in segment order (act holds each projection's dy in its k-steps, see
//             launch_pack_lora's step offset) and each adds its own LoRA term with its own
//             dropout key; out and addend are segment 0's.
constexpr int GEMM_MAX_SEGS = 3;
struct GemmSegment {
  const uint8_t* codes = nullptr;  // NF4 base (codes + absmax), or
  const float* absmax = nullptr;
  const uint16_t* wbf = nullptr;   // bf16 base [N][K]: exactly one of codes / wbf is set
  int64_t N = 0;                   // W rows (forward: output columns; backward: reduction)
  const float* lu = nullptr;
  const float* lw = nullptr;
  Dropout drop{0, 0, 0, 0, 0, 0, 1.0f};  // backward LoRA term's keep mask (threshold 0: none)
  const uint16_t* bias = nullptr;
  const void* addend = nullptr;
  void* out = nullptr;
};
struct GemmLaunch {
  int mode;
  const uint16_t* act;  // packed by launch_pack_lora
  int64_t M, K;
  GemmPlan plan;
  int r;
  float lscale;
  int out_f32;
  int nseg = 1;
  GemmSegment seg[GEMM_MAX_SEGS];
};
hipError_t launch_gemm(const GemmLaunch& L, hipStream_t s);

// One pass over an activation in [T][C] (bf16, or fp32 with in_f32; C % 64 == 0):
//  - if `packed`, writes its bf16 copy in MFMA-fragment order: block (g, s, c) of 512 bf16
//    holds, for lane l = 0..63, the 8 values of row 32*g + (l & 31) at reduction index
//    64*s + 32*(l >> 5) + 8*c + (0..7); blocks ordered g, then s, then c, so the GEMM loads
//    each 32-row operand fragment as one contiguous 1 KB piece; rows padded with zeros up
//    to a multiple of 32 (`packed` holds frag_rows(T) * C bf16);
//  - if r > 0, out[t][j] = scale * sum_c h[t][c] * mat(j, c), h = drop(in) (the dropout
//    mask only touches this rank-r copy); mat_kind 0: mat is [r][C] (LoRA A), 1: [C][r]
//    (LoRA B).  Partials per LORA_CHUNK columns go to part ([ceil(C / LORA_CHUNK)][T][r]
//    floats) and are summed in chunk order.
constexpr int LORA_CHUNK = 256;
inline int64_t frag_rows(int64_t M) { return (M + 31) / 32 * 32; }
//  - pack_steps / pack_step0: the packed buffer holds pack_steps k-steps per 32-row group
//    and this activation fills k-steps pack_step0 .. pack_step0 + C/64 - 1 of each group (a
//    grouped backward packs its projections' dy side by side); 0 / 0: C/64 and 0.
hipError_t launch_pack_lora(const void* in, bool in_f32, int64_t T, int64_t C, const float* mat, int mat_kind,
                            int r, float scale, const Dropout& d, uint16_t* packed, float* part, float* out,
                            hipStream_t s, int pack_steps = 0, int pack_step0 = 0);

// The same pass over up to GEMM_MAX_SEGS activations in one launch (PackInput: input i
// has C_i columns, fills k-steps pstep0_i .. of each group of `packed`, whose stride is
// pack_steps (0: the inputs' k-steps summed), and owns the next nprod_i of prods), with the
// rank-r products of up to GEMM_MAX_SEGS projections in all (each its own matrix, dropout
// mask, partial buffer and output): launch_pack (the packing and every product's chunk
// partials; sets each nck), then launch_product_reduce (every product's chunks summed in
// order, scaled; it may also take products of different packing passes).
struct LoraProduct {
  const float* mat;  // [r][C] (mat_kind 0) or [C][r] (mat_kind 1)
  Dropout drop;
  float scale;
  float* part;       // [ceil(C / LORA_CHUNK)][T][r] floats of its own
  float* out;        // [T][r]
  int nck;
};
struct PackInput {
  const void* in;
  int64_t C;
  int pstep0;
  int nprod;
};
hipError_t launch_pack(const PackInput* ins, int nin, bool in_f32, int64_t T, int mat_kind, int r,
                       LoraProduct* prods, uint16_t* packed, int pack_steps, hipStream_t s);
hipError_t launch_product_reduce(const LoraProduct* prods, int nprod, int64_t T, int r, hipStream_t s);

// Column gradients of the LoRA factors, up to COLGRAD_MAX_TASKS in one launch, each
//   out[j][c] (out_cr 0: [r][C], LoRA dA) or out[c][j] (out_cr 1: [C][r], LoRA dB)
//     = [out +] scale * sum_t coef[t][j] * h[t][c],   h = drop(in) [T][C],  coef [T][r]
// summed over tokens in a fixed order in one pass (no workspace).  in is bf16, or fp32
// with in_f32, for every task; accumulate applies to every task.
constexpr int COLGRAD_MAX_TASKS = 2 * GEMM_MAX_SEGS;
struct ColgradTask {
  const void* in;
  const float* coef;
  float* out;
  int64_t C;
  float scale;
  int out_cr;
  Dropout drop;
};
hipError_t launch_colgrad(const ColgradTask* tasks, int ntask, bool in_f32, int64_t T, int r, int accumulate,
                          hipStream_t s);

// Sum of split partials [splits][T][N] in split order, then + bias[n] (bias may be NULL),
// then addend + that (addend [T][N] in the output's type, may be `out`, NULL for none),
// rounded into bf16 or stored as fp32.  round_first (bf16 output): the pre-addend value is
// rounded to bf16 before the add, as a separate add of a rounded output would do.
hipError_t launch_split_reduce(const float* part, int splits, int64_t T, int64_t N,
                               const uint16_t* bias, const void* addend, bool round_first, void* out,
                               bool out_f32, hipStream_t s);
// Pointwise block glue (glue.hip), fp32 throughout.
hipError_t launch_swiglu_fwd(const float* g, const float* u, int64_t n, float* a, hipStream_t s);
hipError_t launch_swiglu_bwd(const float* da, const float* g, const float* u, int64_t n, float* dg, float* du,
                             hipStream_t s);
hipError_t launch_rope(bool backward, const float* x, const float* cs, const float* sn, int64_t T, int H, int D,
                       float* y, hipStream_t s);
hipError_t launch_rmsnorm_apply(bool backward, const float* dy, const float* h, const float* r, const float* w,
                                int64_t T, int64_t D, float* out, float* hdot, hipStream_t s);

// Device <-> pinned host copy by a kernel (hostcopy.hip); src and dst are device-side
// addresses, bytes a multiple of 16.
hipError_t launch_kernel_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

// AdamW over fp32 tensors (optim.hip).  The hyperparameters in the form the kernel uses
// them, formed on the host in double precision for step t.
struct AdamwHyper {
  float decay, b1c, b2, b2c, bc2s, eps, step;
};
// Workgroups (= g^2 partials written) of one update over tensors of n[0..nt) elements.
int64_t adamw_workgroups(const int64_t* n, int nt);
hipError_t launch_adamw(float* const* p, const float* const* g, float* const* m, float* const* v,
                        const int64_t* n, int nt, const AdamwHyper& h, float* gsq, hipStream_t s);


// ---- small-tile path (small.hip) -------------------------------------------------
// One launch for the forward, one (+ lora_colgrad) for the backward, at shapes where the
// tiled path's launches are latency-bound: r <= SMALL_MAX_R with r % 4 == 0, t <= SMALL_MAX_T and k, n <=
// SMALL_MAX_KN (then each launch is one round of at most 256 workgroups, and a wave runs
// at most 4 of the 64-wide reduction steps).
constexpr int SMALL_MAX_R = 32;
constexpr int64_t SMALL_MAX_T = 1024;
constexpr int64_t SMALL_MAX_KN = 1024;
struct SmallLinear {
  int64_t t, k, n;
  const uint8_t* codes;   // NF4 base, or
  const float* absmax;
  const uint16_t* wbf;    // bf16 base
  const float* A;         // [r][k]
  const float* B;         // [n][r]
  int r;
  float lscale;
  Dropout drop;
  bool act_f32;
  int out_f32;
};
bool small_path_fits(int64_t t, int64_t k, int64_t n, int r);
// y = [residual +] (x W^T + bias + lscale u B^T) and u = drop(x) A^T (u may be null);
// u_only: u alone (y, bias, residual unused); u_given: u holds u, read instead of formed.
hipError_t launch_small_fwd(const SmallLinear& L, const void* x, const uint16_t* bias, const void* residual, void* y,
                            float* u, bool u_only, bool u_given, hipStream_t s);
// dx = [dx +] (dy W + keep * sigma * (du A)) with du = lscale dy B, written to du (may be
// null).
hipError_t launch_small_bwd(const SmallLinear& L, const void* dy, void* dx, int accumulate, float* du, hipStream_t s);


// ---- timing -------------------------------------------------------------------
bool timing_on();
// Whether a launch of this much algorithmic work is timed (timing on, and every launch or
// only the ones with flops).
bool timing_wants(double flops);
// When timing is on, returns a record id and the two events the launch must record
// (hipExtLaunchKernelGGL start/stop); otherwise -1 and null events.  flops and bytes
// are the launch's algorithmic work (0 where it does not apply).
int timing_begin(const char* label, double flops, double bytes, hipEvent_t* start, hipEvent_t* stop);

// Launch `kern` on `s`; when timing is on, under a record labelled "<name> <shape>" whose
// start/stop events the dispatch itself records.
template <typename F, typename... Args>
inline hipError_t timed_launch(const char* name, const char* shape, double flops, double bytes, F kern, dim3 grid,
                               dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (timing_wants(flops)) {
    char label[48];
    snprintf(label, sizeof(label), "%s %s", name, shape);
    timing_begin(label, flops, bytes, &e0, &e1);
  }
  if (e0)
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, 0, s, args...);
  return hipGetLastError();
}

}  // namespace msq
