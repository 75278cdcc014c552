// C-ABI entry points of libmsq: host-side validation, workspace planning and the
// launch sequence of each call.  Every check happens before the first HIP call, so
// an invalid call launches nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "../../include/msq.h"
#include "internal.hpp"

namespace msq {

namespace {
thread_local char g_last_error[512] = "";

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int64_t MAX_T = 65535;          // grid y limit of the epilogue launches
constexpr int64_t MAX_ELEMS = 1LL << 34;  // t*k: dropout counter word 0 holds e >> 2

Dropout make_dropout(const msq_rng_key& key, float p) {
  Dropout d;
  d.k0 = (uint32_t)(key.seed & 0xffffffffu);
  d.k1 = (uint32_t)(key.seed >> 32);
  d.c1 = (key.layer << 4) | key.proj;
  d.c2 = key.step;
  d.c3 = key.micro;
  d.threshold = (uint32_t)floor((double)p * 4294967296.0);
  const float one_minus = 1.0f - p;
  d.sigma = 1.0f / one_minus;
  return d;
}

Dropout no_dropout() {
  Dropout d;
  memset(&d, 0, sizeof(d));
  d.sigma = 1.0f;
  return d;
}

int check_linear(const char* fn, int64_t t, int64_t k, int64_t n, const msq_lora_cfg& cfg,
                 const msq_rng_key& key) {
  if (t < 0 || k <= 0 || n <= 0) return set_error(MSQ_E_INVAL, "%s: t=%lld k=%lld n=%lld must be t>=0, k>0, n>0", fn, (long long)t, (long long)k, (long long)n);
  if (k % 64 || n % 64) return set_error(MSQ_E_SHAPE, "%s: k=%lld and n=%lld must be multiples of 64", fn, (long long)k, (long long)n);
  if (cfg.r < 0 || cfg.r > 64) return set_error(MSQ_E_SHAPE, "%s: r=%d outside [0, 64]", fn, cfg.r);
  if (t > MAX_T) return set_error(MSQ_E_SHAPE, "%s: t=%lld exceeds %lld", fn, (long long)t, (long long)MAX_T);
  if (t * k >= MAX_ELEMS || t * n >= MAX_ELEMS) return set_error(MSQ_E_SHAPE, "%s: t*k or t*n reaches 2^34", fn);
  if (!(cfg.p_drop >= 0.0f && cfg.p_drop < 1.0f)) return set_error(MSQ_E_DROPOUT, "%s: p_drop=%g outside [0, 1)", fn, (double)cfg.p_drop);
  if (cfg.r > 0 && !isfinite(cfg.alpha)) return set_error(MSQ_E_DROPOUT, "%s: alpha is not finite", fn);
  if (key.proj >= 16 || key.layer >= (1u << 28)) return set_error(MSQ_E_INVAL, "%s: rng key proj must be < 16 and layer < 2^28", fn);
  if (cfg.flags & ~(MSQ_ACT_F32 | MSQ_OUT_F32 | MSQ_U_ONLY | MSQ_U_GIVEN | MSQ_PATH_TILED | MSQ_PATH_SMALL))
    return set_error(MSQ_E_INVAL, "%s: unknown flags 0x%x", fn, cfg.flags);
  if ((cfg.flags & MSQ_U_GIVEN) && (cfg.flags & MSQ_U_ONLY))
    return set_error(MSQ_E_INVAL, "%s: MSQ_U_GIVEN with MSQ_U_ONLY leaves nothing to compute", fn);
  if ((cfg.flags & MSQ_U_GIVEN) && cfg.r == 0) return set_error(MSQ_E_INVAL, "%s: MSQ_U_GIVEN needs r > 0", fn);
  if ((cfg.flags & MSQ_PATH_TILED) && (cfg.flags & MSQ_PATH_SMALL))
    return set_error(MSQ_E_INVAL, "%s: MSQ_PATH_TILED and MSQ_PATH_SMALL together", fn);
  if ((cfg.flags & MSQ_PATH_SMALL) && (cfg.r > SMALL_MAX_R || cfg.r % 4))
    return set_error(MSQ_E_SHAPE, "%s: the small-tile path holds r <= %d with r %% 4 == 0, not %d", fn, SMALL_MAX_R,
                     cfg.r);
  return MSQ_OK;
}

// The small-tile path (one launch per forward) where the call asks for it, or where the
// shape fits it and the call does not ask for the tiled path.
bool use_small_path(const msq_lora_cfg& cfg, int64_t t, int64_t k, int64_t n) {
  if (cfg.flags & MSQ_PATH_SMALL) return true;
  if (cfg.flags & MSQ_PATH_TILED) return false;
  return small_path_fits(t, k, n, cfg.r);
}

}  // namespace

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int hip_error(hipError_t e, const char* what) {
  return set_error(MSQ_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

LoraPlan lora_plan(int64_t t, int64_t k, int64_t n, int32_t r) {
  LoraPlan p;
  p.fwd = gemm_plan(t, n, k);
  p.bwd = gemm_plan(t, k, n);
  const size_t tr = (size_t)t * (size_t)r * sizeof(float);
  size_t o = 0;
  p.off_part_fwd = o;
  o = align256(o + (size_t)p.fwd.splits * t * n * sizeof(float));
  p.off_u_fwd = o;
  o = align256(o + tr);
  p.off_act_fwd = o;  // x packed into MFMA-fragment order (bf16)
  o = align256(o + (size_t)frag_rows(t) * k * sizeof(uint16_t));
  p.off_sk_fwd = o;   // chunk partials of the rank-r skinny products
  o = align256(o + (size_t)((k + LORA_CHUNK - 1) / LORA_CHUNK) * t * r * sizeof(float));
  p.fwd_bytes = o;
  o = 0;
  p.off_part_bwd = o;
  o = align256(o + (size_t)p.bwd.splits * t * k * sizeof(float));
  p.off_u_bwd = o;
  o = align256(o + tr);
  p.off_du = o;
  o = align256(o + tr);
  p.off_act_bwd = o;  // dy packed into MFMA-fragment order (bf16)
  o = align256(o + (size_t)frag_rows(t) * n * sizeof(uint16_t));
  p.off_sk_bwd = o;
  o = align256(o + (size_t)((std::max(k, n) + LORA_CHUNK - 1) / LORA_CHUNK) * t * r * sizeof(float));
  p.bwd_bytes = o;
  return p;
}

}  // namespace msq

using namespace msq;

extern "C" {

int msq_abi_version(void) { return MSQ_ABI_VERSION; }

const char* msq_strerror(int code) {
  switch (code) {
    case MSQ_OK: return "ok";
    case MSQ_E_INVAL: return "invalid argument";
    case MSQ_E_SHAPE: return "unsupported shape";
    case MSQ_E_DROPOUT: return "invalid dropout probability or LoRA scale";
    case MSQ_E_WORKSPACE: return "workspace too small";
    case MSQ_E_WINDOW: return "stream window does not fit the arena";
    case MSQ_E_ORDER: return "stream window protocol violation";
    case MSQ_E_HIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char* msq_last_error(void) { return g_last_error; }

int msq_nf4_codebook(float* out) {
  if (!out) return set_error(MSQ_E_INVAL, "msq_nf4_codebook: out is NULL");
  memcpy(out, nf4_lut().v, sizeof(float) * 16);
  return MSQ_OK;
}

int nf4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, float* absmax,
                 msq_stream_t stream) {
  if (n < 0 || k <= 0) return set_error(MSQ_E_INVAL, "nf4_quantize: n=%lld k=%lld", (long long)n, (long long)k);
  if (k % 64) return set_error(MSQ_E_SHAPE, "nf4_quantize: k=%lld is not a multiple of 64", (long long)k);
  if (n == 0) return MSQ_OK;
  if (!w || !codes || !absmax) return set_error(MSQ_E_INVAL, "nf4_quantize: null pointer");
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(absmax, 4))
    return set_error(MSQ_E_INVAL, "nf4_quantize: w and codes must be 16-byte aligned, absmax 4-byte");
  if (n == 0) return MSQ_OK;
  const hipError_t e = launch_quantize(w, n * (k / 64), codes, absmax, (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "nf4_quantize launch");
}

int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t n, int64_t k, uint16_t* w,
                   msq_stream_t stream) {
  if (n < 0 || k <= 0) return set_error(MSQ_E_INVAL, "nf4_dequantize: n=%lld k=%lld", (long long)n, (long long)k);
  if (k % 64) return set_error(MSQ_E_SHAPE, "nf4_dequantize: k=%lld is not a multiple of 64", (long long)k);
  if (n == 0) return MSQ_OK;
  if (!w || !codes || !absmax) return set_error(MSQ_E_INVAL, "nf4_dequantize: null pointer");
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(absmax, 4))
    return set_error(MSQ_E_INVAL, "nf4_dequantize: w and codes must be 16-byte aligned, absmax 4-byte");
  if (n == 0) return MSQ_OK;
  const hipError_t e = launch_dequantize(codes, absmax, n * (k / 32), w, (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "nf4_dequantize launch");
}

size_t nf4_lora_workspace_size(int64_t t, int64_t k, int64_t n, int32_t r) {
  if (t < 0 || k <= 0 || n <= 0 || k % 64 || n % 64 || r < 0 || r > 64 || t > 65535) return 0;
  const LoraPlan p = lora_plan(t, k, n, r);
  return std::max<size_t>(256, std::max(p.fwd_bytes, p.bwd_bytes));  // 0 is reserved for "invalid"
}

}  // extern "C"

namespace {

// The frozen base of one linear: NF4 (codes + absmax) or bf16 values; exactly one is set.
struct Base {
  const uint8_t* codes;
  const float* absmax;
  const uint16_t* wbf;
};

int check_base(const char* fn, const Base& b) {
  if (b.wbf ? (b.codes || b.absmax) : (!b.codes || !b.absmax)) return set_error(MSQ_E_INVAL, "%s: null pointer (base)", fn);
  if (!aligned(b.codes, 16) || !aligned(b.absmax, 4) || !aligned(b.wbf, 16))
    return set_error(MSQ_E_INVAL, "%s: misaligned base (codes, bf16 W: 16 bytes; absmax 4)", fn);
  return MSQ_OK;
}

int lora_fwd(const char* fn, const void* x, int64_t t, int64_t k, int64_t n, const Base& base,
             const uint16_t* bias, const void* residual, const float* A, const float* B, msq_lora_cfg cfg,
             msq_rng_key key, void* y, float* u_out, void* workspace, size_t workspace_bytes, msq_stream_t stream) {
  int rc = check_linear(fn, t, k, n, cfg, key);
  if (rc) return rc;
  rc = check_base(fn, base);
  if (rc) return rc;
  const bool u_only = cfg.flags & MSQ_U_ONLY, u_given = cfg.flags & MSQ_U_GIVEN;
  if (!workspace || (t > 0 && (!x || (!y && !u_only))))
    return set_error(MSQ_E_INVAL, "%s: null pointer", fn);
  if (u_only && (cfg.r == 0 || !u_out))
    return set_error(MSQ_E_INVAL, "%s: MSQ_U_ONLY needs r > 0 and u_out", fn);
  if (u_given && !u_out) return set_error(MSQ_E_INVAL, "%s: MSQ_U_GIVEN needs u_out (the given u)", fn);
  if (cfg.r > 0 && (!A || !B)) return set_error(MSQ_E_INVAL, "%s: r > 0 needs A and B", fn);
  if (u_only && residual) return set_error(MSQ_E_INVAL, "%s: MSQ_U_ONLY writes no y to add a residual to", fn);
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(bias, 8) || !aligned(residual, 16) || !aligned(A, 16) ||
      !aligned(B, 16) || !aligned(u_out, 4) || !aligned(workspace, 256))
    return set_error(MSQ_E_INVAL, "%s: misaligned pointer (x, y, residual, A, B: 16 bytes; bias 8; workspace 256)", fn);
  const LoraPlan p = lora_plan(t, k, n, cfg.r);
  if (workspace_bytes < std::max(p.fwd_bytes, p.bwd_bytes))
    return set_error(MSQ_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, std::max(p.fwd_bytes, p.bwd_bytes));
  if (t == 0) return MSQ_OK;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int r = cfg.r;
  const Dropout d = make_dropout(key, cfg.p_drop);
  const bool act_f32 = cfg.flags & MSQ_ACT_F32, out_f32 = cfg.flags & MSQ_OUT_F32;
  if (use_small_path(cfg, t, k, n)) {
    const SmallLinear L{t, k, n, base.codes, base.absmax, base.wbf, A, B, r, r > 0 ? cfg.alpha / (float)r : 0.0f,
                        d, act_f32, out_f32};
    const hipError_t e = launch_small_fwd(L, x, bias, residual, y, r > 0 ? u_out : nullptr, u_only, u_given, s);
    return e == hipSuccess ? MSQ_OK : hip_error(e, fn);
  }
  float* u = u_out ? u_out : (float*)(ws + p.off_u_fwd);
  float* part = (float*)(ws + p.off_part_fwd);
  const float lscale = r > 0 ? cfg.alpha / (float)r : 0.0f;
  hipError_t e = hipSuccess;
  uint16_t* xb = u_only ? nullptr : (uint16_t*)(ws + p.off_act_fwd);
  // with u given, the pass only packs x (no rank-r product, no chunk reduction)
  e = launch_pack_lora(x, act_f32, t, k, A, 0, u_given ? 0 : r, 1.0f, d, xb, (float*)(ws + p.off_sk_fwd), u, s);
  if (u_only) return e == hipSuccess ? MSQ_OK : hip_error(e, fn);

  if (e == hipSuccess) {
    GemmLaunch L;
    L.mode = 0;
    L.act = xb;
    L.M = t;
    L.K = k;
    L.plan = p.fwd;
    L.r = r;
    L.lscale = lscale;
    L.out_f32 = out_f32;
    GemmSegment& S = L.seg[0];
    S.codes = base.codes;
    S.absmax = base.absmax;
    S.wbf = base.wbf;
    S.N = n;
    S.lu = u;
    S.lw = B;
    S.bias = bias;
    S.addend = p.fwd.splits == 1 ? residual : nullptr;
    S.out = p.fwd.splits == 1 ? y : (void*)part;
    e = launch_gemm(L, s);
  }
  if (e == hipSuccess && p.fwd.splits > 1)
    e = launch_split_reduce(part, p.fwd.splits, t, n, bias, residual, true, y, out_f32, s);
  return e == hipSuccess ? MSQ_OK : hip_error(e, fn);
}

// Workspace of a grouped forward: fp32 split partials of every projection (consecutive
// [splits][t][n_i] blocks), u of each projection, the packed activation and the chunk
// partials of each projection's rank-r product (one packing pass forms them all).
struct GroupPlan {
  GemmPlan fwd;
  size_t off_part, off_u[GEMM_MAX_SEGS], off_act, off_sk[GEMM_MAX_SEGS], bytes;
};

GroupPlan group_plan(int64_t t, int64_t k, const int64_t* ns, int np, int32_t r) {
  GroupPlan p;
  p.fwd = gemm_plan_group(t, ns, np, k);
  int64_t ntot = 0;
  for (int i = 0; i < np; ++i) ntot += ns[i];
  size_t o = 0;
  p.off_part = o;
  o = align256(o + (p.fwd.splits > 1 ? (size_t)p.fwd.splits * t * ntot * sizeof(float) : 0));
  for (int i = 0; i < GEMM_MAX_SEGS; ++i) {
    p.off_u[i] = o;
    if (i < np) o = align256(o + (size_t)t * r * sizeof(float));
  }
  p.off_act = o;
  o = align256(o + (size_t)frag_rows(t) * k * sizeof(uint16_t));
  for (int i = 0; i < GEMM_MAX_SEGS; ++i) {
    p.off_sk[i] = o;
    if (i < np) o = align256(o + (size_t)((k + LORA_CHUNK - 1) / LORA_CHUNK) * t * r * sizeof(float));
  }
  p.bytes = o;
  return p;
}

int group_check(const char* fn, int64_t t, int64_t k, const msq_lora_proj* projs, int n_proj, const msq_lora_cfg& cfg,
                int64_t* ns) {
  if (n_proj < 1 || n_proj > GEMM_MAX_SEGS || !projs)
    return set_error(MSQ_E_INVAL, "%s: n_proj=%d outside [1, %d]", fn, n_proj, GEMM_MAX_SEGS);
  if (cfg.flags & MSQ_U_ONLY) return set_error(MSQ_E_INVAL, "%s: MSQ_U_ONLY is not available for groups", fn);
  if (cfg.flags & MSQ_U_GIVEN)
    for (int i = 0; i < n_proj; ++i)
      if (!projs[i].u_out) return set_error(MSQ_E_INVAL, "%s: MSQ_U_GIVEN needs every projection's u_out", fn);
  if (cfg.flags & MSQ_PATH_SMALL)
    return set_error(MSQ_E_INVAL, "%s: groups run on the tiled path (MSQ_PATH_SMALL is for single calls)", fn);
  int64_t ntot = 0;
  for (int i = 0; i < n_proj; ++i) {
    const msq_lora_proj& q = projs[i];
    int rc = check_linear(fn, t, k, q.n, cfg, q.key);
    if (rc) return rc;
    rc = check_base(fn, Base{q.codes, q.absmax, q.w});
    if (rc) return rc;
    if ((q.w != nullptr) != (projs[0].w != nullptr)) return set_error(MSQ_E_INVAL, "%s: mixed base formats in one group", fn);
    if (t > 0 && !q.y) return set_error(MSQ_E_INVAL, "%s: projection %d: null y", fn, i);
    if (cfg.r > 0 && (!q.A || !q.B)) return set_error(MSQ_E_INVAL, "%s: projection %d: r > 0 needs A and B", fn, i);
    if (!aligned(q.y, 16) || !aligned(q.bias, 8) || !aligned(q.residual, 16) || !aligned(q.A, 16) || !aligned(q.B, 16) ||
        !aligned(q.u_out, 4))
      return set_error(MSQ_E_INVAL, "%s: projection %d: misaligned pointer (y, residual, A, B: 16 bytes; bias 8)", fn, i);
    ns[i] = q.n;
    ntot += q.n;
  }
  if (t * ntot >= MAX_ELEMS) return set_error(MSQ_E_SHAPE, "%s: t * (sum of n) reaches 2^34", fn);
  return MSQ_OK;
}

int lora_bwd(const char* fn, const void* dy, const void* x, int64_t t, int64_t k, int64_t n, const Base& base,
             const float* A, const float* B, msq_lora_cfg cfg, msq_rng_key key, const float* u, void* dx,
             int dx_accumulate, float* dA, float* dB, int dAB_accumulate, void* workspace, size_t workspace_bytes,
             msq_stream_t stream) {
  int rc = check_linear(fn, t, k, n, cfg, key);
  if (rc) return rc;
  rc = check_base(fn, base);
  if (rc) return rc;
  if (!workspace || (t > 0 && (!dy || !x || !dx)))
    return set_error(MSQ_E_INVAL, "%s: null pointer", fn);
  if (cfg.r > 0 && (!A || !B || !dA || !dB)) return set_error(MSQ_E_INVAL, "%s: r > 0 needs A, B, dA, dB", fn);
  if (cfg.flags & (MSQ_U_ONLY | MSQ_U_GIVEN)) return set_error(MSQ_E_INVAL, "%s: MSQ_U_ONLY / MSQ_U_GIVEN are forward flags", fn);
  if ((dx_accumulate != 0 && dx_accumulate != 1) || (dAB_accumulate != 0 && dAB_accumulate != 1))
    return set_error(MSQ_E_INVAL, "%s: accumulate flags must be 0 or 1", fn);
  if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(dx, 16) || !aligned(A, 16) || !aligned(B, 16) ||
      !aligned(u, 4) || !aligned(dA, 4) || !aligned(dB, 4) || !aligned(workspace, 256))
    return set_error(MSQ_E_INVAL, "%s: misaligned pointer (dy, x, dx, A, B: 16 bytes; workspace 256)", fn);
  const LoraPlan p = lora_plan(t, k, n, cfg.r);
  if (workspace_bytes < std::max(p.fwd_bytes, p.bwd_bytes))
    return set_error(MSQ_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, std::max(p.fwd_bytes, p.bwd_bytes));
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int r = cfg.r;
  const Dropout d = make_dropout(key, cfg.p_drop);
  const float lscale = r > 0 ? cfg.alpha / (float)r : 0.0f;
  hipError_t e = hipSuccess;
  if (t > 0 && use_small_path(cfg, t, k, n)) {
    // u (recomputed when not passed), then dx with du, then dA and dB from du and u
    const bool act_f32 = cfg.flags & MSQ_ACT_F32, out_f32 = cfg.flags & MSQ_OUT_F32;
    const SmallLinear L{t, k, n, base.codes, base.absmax, base.wbf, A, B, r, lscale, d, act_f32, out_f32};
    float* du = (float*)(ws + p.off_du);
    const float* uu = u;
    if (r > 0 && !uu) {
      float* ut = (float*)(ws + p.off_u_bwd);
      e = launch_small_fwd(L, x, nullptr, nullptr, nullptr, ut, true, false, s);
      uu = ut;
    }
    if (e == hipSuccess) e = launch_small_bwd(L, dy, dx, dx_accumulate, r > 0 ? du : nullptr, s);
    if (e == hipSuccess && r > 0) {
      const ColgradTask tasks[2] = {{x, du, dA, k, 1.0f, 0, d}, {dy, uu, dB, n, lscale, 1, no_dropout()}};
      e = launch_colgrad(tasks, 2, act_f32, t, r, dAB_accumulate, s);
    }
  } else if (t > 0) {
    const bool act_f32 = cfg.flags & MSQ_ACT_F32, out_f32 = cfg.flags & MSQ_OUT_F32;
    float* part = (float*)(ws + p.off_part_bwd);
    float* du = (float*)(ws + p.off_du);
    float* sk = (float*)(ws + p.off_sk_bwd);
    const float* uu = u;
    uint16_t* dyb = (uint16_t*)(ws + p.off_act_bwd);
    if (e == hipSuccess && r > 0 && !uu) {
      float* ut = (float*)(ws + p.off_u_bwd);
      e = launch_pack_lora(x, act_f32, t, k, A, 0, r, 1.0f, d, nullptr, sk, ut, s);
      uu = ut;
    }
    if (e == hipSuccess) e = launch_pack_lora(dy, act_f32, t, n, B, 1, r, lscale, no_dropout(), dyb, sk, du, s);
    if (e == hipSuccess) {
      GemmLaunch L;
      L.mode = 1;
      L.act = dyb;
      L.M = t;
      L.K = k;
      L.plan = p.bwd;
      L.r = r;
      L.lscale = 1.0f;
      L.out_f32 = out_f32;
      GemmSegment& S = L.seg[0];
      S.codes = base.codes;
      S.absmax = base.absmax;
      S.wbf = base.wbf;
      S.N = n;
      S.lu = du;
      S.lw = A;
      S.drop = d;
      S.addend = dx_accumulate && p.bwd.splits == 1 ? dx : nullptr;
      S.out = p.bwd.splits == 1 ? dx : (void*)part;
      e = launch_gemm(L, s);
    }
    if (e == hipSuccess && p.bwd.splits > 1)
      e = launch_split_reduce(part, p.bwd.splits, t, k, nullptr, dx_accumulate ? dx : nullptr, false, dx, out_f32,
                              s);
    if (e == hipSuccess && r > 0) {
      const ColgradTask tasks[2] = {{x, du, dA, k, 1.0f, 0, d}, {dy, uu, dB, n, lscale, 1, no_dropout()}};
      e = launch_colgrad(tasks, 2, act_f32, t, r, dAB_accumulate, s);
    }
  } else if (r > 0) {
    // no tokens: the gradients are zero (or stay as they are when accumulating)
    const ColgradTask tasks[2] = {{nullptr, nullptr, dA, k, 1.0f, 0, no_dropout()},
                                  {nullptr, nullptr, dB, n, lscale, 1, no_dropout()}};
    e = launch_colgrad(tasks, 2, false, 0, r, dAB_accumulate, s);
  }
  return e == hipSuccess ? MSQ_OK : hip_error(e, fn);
}

// Workspace of a grouped backward: fp32 split partials of dx, u (when recomputed) and du
// of every projection, the projections' dy packed side by side along the reduction, and
// each projection's chunk partials of its rank-r products (the u pass is summed before
// the du pass reuses them).
struct GroupBwdPlan {
  GemmPlan bwd;
  int64_t red;  // concatenated reduction: the sum of the projections' n
  size_t off_part, off_u[GEMM_MAX_SEGS], off_du[GEMM_MAX_SEGS], off_act, off_sk[GEMM_MAX_SEGS], bytes;
};

GroupBwdPlan group_bwd_plan(int64_t t, int64_t k, const int64_t* ns, int np, int32_t r) {
  GroupBwdPlan p;
  p.red = 0;
  int64_t nmax = 0;
  for (int i = 0; i < np; ++i) {
    p.red += ns[i];
    nmax = std::max(nmax, ns[i]);
  }
  p.bwd = gemm_plan(t, k, p.red, np);  // split i adds projection i's LoRA term
  const size_t tr = (size_t)t * (size_t)r * sizeof(float);
  size_t o = 0;
  p.off_part = o;
  o = align256(o + (p.bwd.splits > 1 ? (size_t)p.bwd.splits * t * k * sizeof(float) : 0));
  for (int i = 0; i < GEMM_MAX_SEGS; ++i) {
    p.off_u[i] = o;
    if (i < np) o = align256(o + tr);
    p.off_du[i] = o;
    if (i < np) o = align256(o + tr);
  }
  p.off_act = o;
  o = align256(o + (size_t)frag_rows(t) * p.red * sizeof(uint16_t));
  for (int i = 0; i < GEMM_MAX_SEGS; ++i) {
    p.off_sk[i] = o;
    if (i < np) o = align256(o + (size_t)((std::max(k, ns[i]) + LORA_CHUNK - 1) / LORA_CHUNK) * t * r * sizeof(float));
  }
  p.bytes = o;
  return p;
}

int group_bwd_check(const char* fn, int64_t t, int64_t k, const msq_lora_proj_grad* projs, int n_proj,
                    const msq_lora_cfg& cfg, int64_t* ns) {
  if (n_proj < 1 || n_proj > GEMM_MAX_SEGS || !projs)
    return set_error(MSQ_E_INVAL, "%s: n_proj=%d outside [1, %d]", fn, n_proj, GEMM_MAX_SEGS);
  if (cfg.flags & (MSQ_U_ONLY | MSQ_U_GIVEN)) return set_error(MSQ_E_INVAL, "%s: MSQ_U_ONLY / MSQ_U_GIVEN are forward flags", fn);
  if (cfg.flags & MSQ_PATH_SMALL)
    return set_error(MSQ_E_INVAL, "%s: groups run on the tiled path (MSQ_PATH_SMALL is for single calls)", fn);
  int64_t red = 0;
  for (int i = 0; i < n_proj; ++i) {
    const msq_lora_proj_grad& q = projs[i];
    int rc = check_linear(fn, t, k, q.n, cfg, q.key);
    if (rc) return rc;
    rc = check_base(fn, Base{q.codes, q.absmax, q.w});
    if (rc) return rc;
    if ((q.w != nullptr) != (projs[0].w != nullptr)) return set_error(MSQ_E_INVAL, "%s: mixed base formats in one group", fn);
    if (t > 0 && !q.dy) return set_error(MSQ_E_INVAL, "%s: projection %d: null dy", fn, i);
    if (cfg.r > 0 && (!q.A || !q.B || !q.dA || !q.dB))
      return set_error(MSQ_E_INVAL, "%s: projection %d: r > 0 needs A, B, dA, dB", fn, i);
    if (!aligned(q.dy, 16) || !aligned(q.A, 16) || !aligned(q.B, 16) || !aligned(q.u, 4) || !aligned(q.dA, 4) ||
        !aligned(q.dB, 4))
      return set_error(MSQ_E_INVAL, "%s: projection %d: misaligned pointer (dy, A, B: 16 bytes; u, dA, dB: 4)", fn, i);
    ns[i] = q.n;
    red += q.n;
  }
  if (t * red >= MAX_ELEMS) return set_error(MSQ_E_SHAPE, "%s: t * (sum of n) reaches 2^34", fn);
  return MSQ_OK;
}

}  // namespace

extern "C" {

int nf4_lora_fwd(const void* x, int64_t t, int64_t k, int64_t n, const uint8_t* codes,
                 const float* absmax, const uint16_t* bias, const void* residual, const float* A,
                 const float* B, msq_lora_cfg cfg, msq_rng_key key, void* y, float* u_out,
                 void* workspace, size_t workspace_bytes, msq_stream_t stream) {
  if (!codes || !absmax) return set_error(MSQ_E_INVAL, "nf4_lora_fwd: null pointer (codes, absmax)");
  return lora_fwd("nf4_lora_fwd", x, t, k, n, Base{codes, absmax, nullptr}, bias, residual, A, B, cfg, key, y,
                  u_out, workspace, workspace_bytes, stream);
}

int nf4_lora_bwd(const void* dy, const void* x, int64_t t, int64_t k, int64_t n,
                 const uint8_t* codes, const float* absmax, const float* A, const float* B,
                 msq_lora_cfg cfg, msq_rng_key key, const float* u, void* dx,
                 int dx_accumulate, float* dA, float* dB, int dAB_accumulate, void* workspace,
                 size_t workspace_bytes, msq_stream_t stream) {
  if (!codes || !absmax) return set_error(MSQ_E_INVAL, "nf4_lora_bwd: null pointer (codes, absmax)");
  return lora_bwd("nf4_lora_bwd", dy, x, t, k, n, Base{codes, absmax, nullptr}, A, B, cfg, key, u, dx,
                  dx_accumulate, dA, dB, dAB_accumulate, workspace, workspace_bytes, stream);
}

size_t lora_group_workspace_size(int64_t t, int64_t k, const msq_lora_proj* projs, int n_proj, int32_t r) {
  int64_t ns[GEMM_MAX_SEGS];
  msq_lora_cfg cfg;
  memset(&cfg, 0, sizeof(cfg));
  cfg.r = r;
  cfg.alpha = 1.0f;
  if (group_check("lora_group_workspace_size", t, k, projs, n_proj, cfg, ns) != MSQ_OK) return 0;
  return group_plan(t, k, ns, n_proj, r).bytes;
}

int lora_fwd_group(const void* x, int64_t t, int64_t k, const msq_lora_proj* projs, int n_proj, msq_lora_cfg cfg,
                   void* workspace, size_t workspace_bytes, msq_stream_t stream) {
  const char* fn = "lora_fwd_group";
  int64_t ns[GEMM_MAX_SEGS];
  int rc = group_check(fn, t, k, projs, n_proj, cfg, ns);
  if (rc) return rc;
  if (!workspace || (t > 0 && !x)) return set_error(MSQ_E_INVAL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(workspace, 256))
    return set_error(MSQ_E_INVAL, "%s: misaligned pointer (x 16 bytes; workspace 256)", fn);
  const GroupPlan p = group_plan(t, k, ns, n_proj, cfg.r);
  if (workspace_bytes < p.bytes) return set_error(MSQ_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, p.bytes);
  if (t == 0) return MSQ_OK;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int r = cfg.r;
  const bool act_f32 = cfg.flags & MSQ_ACT_F32, out_f32 = cfg.flags & MSQ_OUT_F32;
  const float lscale = r > 0 ? cfg.alpha / (float)r : 0.0f;
  uint16_t* xb = (uint16_t*)(ws + p.off_act);
  float* u[GEMM_MAX_SEGS];
  hipError_t e = hipSuccess;
  // one pass over x packs it and forms every projection's rank-r product (each with its
  // own A and dropout mask), one launch sums their chunk partials
  LoraProduct prods[GEMM_MAX_SEGS];
  for (int i = 0; i < n_proj; ++i) {
    const msq_lora_proj& q = projs[i];
    u[i] = q.u_out ? q.u_out : (float*)(ws + p.off_u[i]);
    prods[i] = {q.A, make_dropout(q.key, cfg.p_drop), 1.0f, (float*)(ws + p.off_sk[i]), u[i], 0};
  }
  // with every u given (MSQ_U_GIVEN), the pass only packs x
  const bool u_given = cfg.flags & MSQ_U_GIVEN;
  const int rp = u_given ? 0 : r;
  const PackInput xin{x, k, 0, rp > 0 ? n_proj : 0};
  e = launch_pack(&xin, 1, act_f32, t, 0, rp, prods, xb, 0, s);
  if (e == hipSuccess) e = launch_product_reduce(prods, rp > 0 ? n_proj : 0, t, rp, s);
  float* part = (float*)(ws + p.off_part);
  size_t part_off[GEMM_MAX_SEGS];
  if (e == hipSuccess) {
    GemmLaunch L;
    L.mode = 0;
    L.act = xb;
    L.M = t;
    L.K = k;
    L.plan = p.fwd;
    L.r = r;
    L.lscale = lscale;
    L.out_f32 = out_f32;
    L.nseg = n_proj;
    size_t o = 0;
    for (int i = 0; i < n_proj; ++i) {
      const msq_lora_proj& q = projs[i];
      GemmSegment& S = L.seg[i];
      S.codes = q.codes;
      S.absmax = q.absmax;
      S.wbf = q.w;
      S.N = q.n;
      S.lu = u[i];
      S.lw = q.B;
      S.bias = q.bias;
      part_off[i] = o;
      S.addend = p.fwd.splits == 1 ? q.residual : nullptr;
      S.out = p.fwd.splits == 1 ? q.y : (void*)(part + o);
      o += (size_t)p.fwd.splits * t * q.n;
    }
    e = launch_gemm(L, s);
  }
  for (int i = 0; i < n_proj && e == hipSuccess && p.fwd.splits > 1; ++i)
    e = launch_split_reduce(part + part_off[i], p.fwd.splits, t, projs[i].n, projs[i].bias, projs[i].residual, true,
                            projs[i].y, out_f32, s);
  return e == hipSuccess ? MSQ_OK : hip_error(e, fn);
}

size_t lora_group_bwd_workspace_size(int64_t t, int64_t k, const msq_lora_proj_grad* projs, int n_proj, int32_t r) {
  int64_t ns[GEMM_MAX_SEGS];
  msq_lora_cfg cfg;
  memset(&cfg, 0, sizeof(cfg));
  cfg.r = r;
  cfg.alpha = 1.0f;
  if (group_bwd_check("lora_group_bwd_workspace_size", t, k, projs, n_proj, cfg, ns) != MSQ_OK) return 0;
  return group_bwd_plan(t, k, ns, n_proj, r).bytes;
}

int lora_bwd_group(const void* x, int64_t t, int64_t k, const msq_lora_proj_grad* projs, int n_proj,
                   msq_lora_cfg cfg, void* dx, int dx_accumulate, int dAB_accumulate, void* workspace,
                   size_t workspace_bytes, msq_stream_t stream) {
  const char* fn = "lora_bwd_group";
  int64_t ns[GEMM_MAX_SEGS];
  int rc = group_bwd_check(fn, t, k, projs, n_proj, cfg, ns);
  if (rc) return rc;
  if (!workspace || (t > 0 && (!x || !dx))) return set_error(MSQ_E_INVAL, "%s: null pointer", fn);
  if ((dx_accumulate != 0 && dx_accumulate != 1) || (dAB_accumulate != 0 && dAB_accumulate != 1))
    return set_error(MSQ_E_INVAL, "%s: accumulate flags must be 0 or 1", fn);
  if (!aligned(x, 16) || !aligned(dx, 16) || !aligned(workspace, 256))
    return set_error(MSQ_E_INVAL, "%s: misaligned pointer (x, dx: 16 bytes; workspace 256)", fn);
  const GroupBwdPlan p = group_bwd_plan(t, k, ns, n_proj, cfg.r);
  if (workspace_bytes < p.bytes) return set_error(MSQ_E_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, p.bytes);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int r = cfg.r;
  const bool act_f32 = cfg.flags & MSQ_ACT_F32, out_f32 = cfg.flags & MSQ_OUT_F32;
  const float lscale = r > 0 ? cfg.alpha / (float)r : 0.0f;
  hipError_t e = hipSuccess;
  const float* u[GEMM_MAX_SEGS];
  float* du[GEMM_MAX_SEGS];
  Dropout d[GEMM_MAX_SEGS];
  for (int i = 0; i < n_proj; ++i) {
    d[i] = make_dropout(projs[i].key, cfg.p_drop);
    du[i] = (float*)(ws + p.off_du[i]);
    u[i] = projs[i].u;
  }
  if (t > 0) {
    uint16_t* act = (uint16_t*)(ws + p.off_act);
    const int steps = (int)(p.red / 64);
    // u of the projections whose forward u was not passed in: one pass over x for all
    LoraProduct up[GEMM_MAX_SEGS];
    int nu = 0;
    for (int i = 0; i < n_proj && r > 0; ++i)
      if (!u[i]) {
        float* ut = (float*)(ws + p.off_u[i]);
        up[nu++] = {projs[i].A, d[i], 1.0f, (float*)(ws + p.off_sk[i]), ut, 0};
        u[i] = ut;
      }
    if (nu > 0) {
      const PackInput xin{x, k, 0, nu};
      e = launch_pack(&xin, 1, act_f32, t, 0, r, up, nullptr, 0, s);
      if (e == hipSuccess) e = launch_product_reduce(up, nu, t, r, s);
    }
    // every dy_i in one launch, into k-steps step0_i .. of the shared operand, with the
    // partials of du_i = s dy_i B_i; one launch then sums every du
    LoraProduct dp[GEMM_MAX_SEGS];
    PackInput dyin[GEMM_MAX_SEGS];
    int step0 = 0;
    for (int i = 0; i < n_proj; ++i) {
      const msq_lora_proj_grad& q = projs[i];
      dp[i] = {q.B, no_dropout(), lscale, (float*)(ws + p.off_sk[i]), du[i], 0};
      dyin[i] = {q.dy, q.n, step0, r > 0 ? 1 : 0};
      step0 += (int)(q.n / 64);
    }
    if (e == hipSuccess) e = launch_pack(dyin, n_proj, act_f32, t, 1, r, dp, act, steps, s);
    if (e == hipSuccess) e = launch_product_reduce(dp, r > 0 ? n_proj : 0, t, r, s);
    float* part = (float*)(ws + p.off_part);
    if (e == hipSuccess) {
      GemmLaunch L;
      L.mode = 1;
      L.act = act;
      L.M = t;
      L.K = k;
      L.plan = p.bwd;
      L.r = r;
      L.lscale = 1.0f;
      L.out_f32 = out_f32;
      L.nseg = n_proj;
      for (int i = 0; i < n_proj; ++i) {
        const msq_lora_proj_grad& q = projs[i];
        GemmSegment& S = L.seg[i];
        S.codes = q.codes;
        S.absmax = q.absmax;
        S.wbf = q.w;
        S.N = q.n;
        S.lu = du[i];
        S.lw = q.A;
        S.drop = d[i];
      }
      L.seg[0].addend = dx_accumulate && p.bwd.splits == 1 ? dx : nullptr;
      L.seg[0].out = p.bwd.splits == 1 ? dx : (void*)part;
      e = launch_gemm(L, s);
    }
    if (e == hipSuccess && p.bwd.splits > 1)
      e = launch_split_reduce(part, p.bwd.splits, t, k, nullptr, dx_accumulate ? dx : nullptr, false, dx, out_f32, s);
  }
  // every dA_i and dB_i in one launch (zero, or unchanged when accumulating, at t == 0)
  if (e == hipSuccess && r > 0) {
    ColgradTask tasks[COLGRAD_MAX_TASKS];
    for (int i = 0; i < n_proj; ++i) {
      const msq_lora_proj_grad& q = projs[i];
      tasks[2 * i] = {t > 0 ? x : nullptr, du[i], q.dA, k, 1.0f, 0, d[i]};
      tasks[2 * i + 1] = {t > 0 ? q.dy : nullptr, u[i], q.dB, q.n, lscale, 1, no_dropout()};
    }
    e = launch_colgrad(tasks, 2 * n_proj, act_f32, t, r, dAB_accumulate, s);
  }
  return e == hipSuccess ? MSQ_OK : hip_error(e, fn);
}

int bf16_lora_fwd(const void* x, int64_t t, int64_t k, int64_t n, const uint16_t* w,
                  const uint16_t* bias, const void* residual, const float* A, const float* B,
                  msq_lora_cfg cfg, msq_rng_key key, void* y, float* u_out, void* workspace,
                  size_t workspace_bytes, msq_stream_t stream) {
  if (!w) return set_error(MSQ_E_INVAL, "bf16_lora_fwd: null pointer (w)");
  return lora_fwd("bf16_lora_fwd", x, t, k, n, Base{nullptr, nullptr, w}, bias, residual, A, B, cfg, key, y,
                  u_out, workspace, workspace_bytes, stream);
}

int bf16_lora_bwd(const void* dy, const void* x, int64_t t, int64_t k, int64_t n, const uint16_t* w,
                  const float* A, const float* B, msq_lora_cfg cfg, msq_rng_key key, const float* u,
                  void* dx, int dx_accumulate, float* dA, float* dB, int dAB_accumulate,
                  void* workspace, size_t workspace_bytes, msq_stream_t stream) {
  if (!w) return set_error(MSQ_E_INVAL, "bf16_lora_bwd: null pointer (w)");
  return lora_bwd("bf16_lora_bwd", dy, x, t, k, n, Base{nullptr, nullptr, w}, A, B, cfg, key, u, dx,
                  dx_accumulate, dA, dB, dAB_accumulate, workspace, workspace_bytes, stream);
}

int msq_swiglu_fwd(const float* g, const float* u, int64_t n, float* a, msq_stream_t stream) {
  if (n < 0 || n > (int64_t(1) << 40)) return set_error(MSQ_E_SHAPE, "msq_swiglu_fwd: n = %lld outside [0, 2^40]", (long long)n);
  if (n == 0) return MSQ_OK;
  if (!g || !u || !a) return set_error(MSQ_E_INVAL, "msq_swiglu_fwd: null pointer");
  if (!aligned(g, 16) || !aligned(u, 16) || !aligned(a, 16))
    return set_error(MSQ_E_INVAL, "msq_swiglu_fwd: misaligned pointer (16 bytes)");
  const hipError_t e = launch_swiglu_fwd(g, u, n, a, (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "msq_swiglu_fwd launch");
}

int msq_swiglu_bwd(const float* da, const float* g, const float* u, int64_t n, float* dg, float* du,
                   msq_stream_t stream) {
  if (n < 0 || n > (int64_t(1) << 40)) return set_error(MSQ_E_SHAPE, "msq_swiglu_bwd: n = %lld outside [0, 2^40]", (long long)n);
  if (n == 0) return MSQ_OK;
  if (!da || !g || !u || !dg || !du) return set_error(MSQ_E_INVAL, "msq_swiglu_bwd: null pointer");
  if (!aligned(da, 16) || !aligned(g, 16) || !aligned(u, 16) || !aligned(dg, 16) || !aligned(du, 16))
    return set_error(MSQ_E_INVAL, "msq_swiglu_bwd: misaligned pointer (16 bytes)");
  const hipError_t e = launch_swiglu_bwd(da, g, u, n, dg, du, (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "msq_swiglu_bwd launch");
}

static int rope_entry(const char* fn, bool backward, const float* x, const float* cs, const float* sn, int64_t t,
                      int32_t heads, int32_t d, float* y, msq_stream_t stream) {
  if (t < 0 || heads < 1 || d < 2 || d % 2 || (double)t * heads * d > (double)(int64_t(1) << 40))
    return set_error(MSQ_E_SHAPE, "%s: t = %lld, heads = %d, d = %d (need t >= 0, heads >= 1, even d >= 2, t*heads*d <= 2^40)",
                     fn, (long long)t, heads, d);
  if (t == 0) return MSQ_OK;
  if (!x || !cs || !sn || !y) return set_error(MSQ_E_INVAL, "%s: null pointer", fn);
  if (!aligned(x, 16) || !aligned(cs, 16) || !aligned(sn, 16) || !aligned(y, 16))
    return set_error(MSQ_E_INVAL, "%s: misaligned pointer (16 bytes)", fn);
  const hipError_t e = launch_rope(backward, x, cs, sn, t, heads, d, y, (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, fn);
}

int msq_rope_fwd(const float* x, const float* cos_t, const float* sin_t, int64_t t, int32_t heads, int32_t d,
                 float* y, msq_stream_t stream) {
  return rope_entry("msq_rope_fwd", false, x, cos_t, sin_t, t, heads, d, y, stream);
}

int msq_rope_bwd(const float* dy, const float* cos_t, const float* sin_t, int64_t t, int32_t heads, int32_t d,
                 float* dx, msq_stream_t stream) {
  return rope_entry("msq_rope_bwd", true, dy, cos_t, sin_t, t, heads, d, dx, stream);
}

static int rmsnorm_entry(const char* fn, bool backward, const float* dy, const float* h, const float* r,
                         const float* w, int64_t t, int64_t d, float* out, float* hdot, msq_stream_t stream) {
  if (t < 0 || d < 4 || d % 4 || (double)t * d > (double)(int64_t(1) << 40))
    return set_error(MSQ_E_SHAPE, "%s: t = %lld, d = %lld (need t >= 0, d >= 4, d %% 4 == 0, t*d <= 2^40)", fn,
                     (long long)t, (long long)d);
  if (t == 0) return MSQ_OK;
  if (!h || !r || !w || !out || (backward && (!dy || !hdot))) return set_error(MSQ_E_INVAL, "%s: null pointer", fn);
  if (!aligned(h, 16) || !aligned(r, 4) || !aligned(w, 16) || !aligned(out, 16) || !aligned(dy, 16) ||
      !aligned(hdot, 16))
    return set_error(MSQ_E_INVAL, "%s: misaligned pointer (16 bytes; r 4)", fn);
  const hipError_t e = launch_rmsnorm_apply(backward, dy, h, r, w, t, d, out, hdot, (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, fn);
}

int msq_rmsnorm_apply_fwd(const float* h, const float* r, const float* w, int64_t t, int64_t d, float* y,
                          msq_stream_t stream) {
  return rmsnorm_entry("msq_rmsnorm_apply_fwd", false, nullptr, h, r, w, t, d, y, nullptr, stream);
}

int msq_rmsnorm_apply_bwd(const float* dy, const float* h, const float* r, const float* w, int64_t t, int64_t d,
                          float* dh, float* hdot, msq_stream_t stream) {
  return rmsnorm_entry("msq_rmsnorm_apply_bwd", true, dy, h, r, w, t, d, dh, hdot, stream);
}

// The device-side address of p (device memory, or pinned host memory mapped for the
// device), or null when p is neither.
static const void* device_side(const void* p) {
  hipPointerAttribute_t a;
  memset(&a, 0, sizeof(a));
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice) return p;
  if (a.type == hipMemoryTypeHost && a.devicePointer) {
    // devicePointer and hostPointer describe the same place; keep p's offset from it
    const char* hp = (const char*)a.hostPointer;
    const ptrdiff_t off = hp ? (const char*)p - hp : 0;
    return (const char*)a.devicePointer + off;
  }
  return nullptr;
}

int msq_kernel_copy(const void* src, void* dst, size_t bytes, msq_stream_t stream) {
  const char* fn = "msq_kernel_copy";
  if (bytes == 0) return MSQ_OK;
  if (!src || !dst) return set_error(MSQ_E_INVAL, "%s: null pointer", fn);
  if (bytes % 16 || !aligned(src, 16) || !aligned(dst, 16))
    return set_error(MSQ_E_INVAL, "%s: pointers must be 16-byte aligned and bytes (%zu) a multiple of 16", fn, bytes);
  const char* s0 = (const char*)src;
  const char* d0 = (const char*)dst;
  if (s0 < d0 + bytes && d0 < s0 + bytes) return set_error(MSQ_E_INVAL, "%s: src and dst overlap", fn);
  const void* sd = device_side(src);
  const void* se = device_side(s0 + bytes - 1);
  const void* dd = device_side(dst);
  const void* de = device_side(d0 + bytes - 1);
  if (!sd || !se || (const char*)se - (const char*)sd != (ptrdiff_t)(bytes - 1))
    return set_error(MSQ_E_INVAL, "%s: src (%p, %zu bytes) is not device or pinned host memory over its range", fn,
                     src, bytes);
  if (!dd || !de || (const char*)de - (const char*)dd != (ptrdiff_t)(bytes - 1))
    return set_error(MSQ_E_INVAL, "%s: dst (%p, %zu bytes) is not device or pinned host memory over its range", fn,
                     dst, bytes);
  const hipError_t e = launch_kernel_copy(sd, (void*)dd, (int64_t)bytes, (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "msq_kernel_copy launch");
}

int64_t msq_adamw_partials(const msq_adamw_tensor* tensors, int n_tensors) {
  if (n_tensors < 0 || (n_tensors > 0 && !tensors)) return -1;
  std::vector<int64_t> n((size_t)n_tensors);
  for (int i = 0; i < n_tensors; ++i) {
    if (tensors[i].n < 0) return -1;
    n[i] = tensors[i].n;
  }
  return adamw_workgroups(n.data(), n_tensors);
}

int msq_adamw_step(const msq_adamw_tensor* tensors, int n_tensors, msq_adamw_cfg cfg, int64_t step, float* gsq,
                   msq_stream_t stream) {
  const char* fn = "msq_adamw_step";
  if (n_tensors < 0 || (n_tensors > 0 && !tensors)) return set_error(MSQ_E_INVAL, "%s: %d tensors", fn, n_tensors);
  if (step < 1) return set_error(MSQ_E_INVAL, "%s: step %lld < 1", fn, (long long)step);
  if (!(cfg.lr >= 0.0) || !(cfg.beta1 >= 0.0 && cfg.beta1 < 1.0) || !(cfg.beta2 >= 0.0 && cfg.beta2 < 1.0) ||
      !(cfg.eps > 0.0) || !(cfg.weight_decay >= 0.0))
    return set_error(MSQ_E_INVAL, "%s: lr %g, betas (%g, %g), eps %g, weight_decay %g out of range", fn, cfg.lr,
                     cfg.beta1, cfg.beta2, cfg.eps, cfg.weight_decay);
  std::vector<float*> p, m, v;
  std::vector<const float*> g;
  std::vector<int64_t> n;
  for (int i = 0; i < n_tensors; ++i) {
    const msq_adamw_tensor& t = tensors[i];
    if (t.n < 0) return set_error(MSQ_E_INVAL, "%s: tensor %d has n = %lld", fn, i, (long long)t.n);
    if (t.n == 0) continue;
    if (!t.p || !t.g || !t.m || !t.v) return set_error(MSQ_E_INVAL, "%s: tensor %d: null pointer", fn, i);
    if (!aligned(t.p, 16) || !aligned(t.g, 16) || !aligned(t.m, 16) || !aligned(t.v, 16))
      return set_error(MSQ_E_INVAL, "%s: tensor %d: misaligned pointer (16 bytes)", fn, i);
    p.push_back(t.p);
    g.push_back(t.g);
    m.push_back(t.m);
    v.push_back(t.v);
    n.push_back(t.n);
  }
  // the partials of empty tensors are none, so the kept ones land where msq_adamw_partials counts them
  const double lr = cfg.lr, b1 = cfg.beta1, b2 = cfg.beta2;
  AdamwHyper h;
  h.decay = (float)(1.0 - lr * cfg.weight_decay);
  h.b1c = (float)(1.0 - b1);
  h.b2 = (float)b2;
  h.b2c = (float)(1.0 - b2);
  h.bc2s = (float)std::sqrt(1.0 - std::pow(b2, (double)step));
  h.eps = (float)cfg.eps;
  h.step = (float)(lr / (1.0 - std::pow(b1, (double)step)));
  if (p.empty()) return MSQ_OK;
  const hipError_t e = launch_adamw(p.data(), g.data(), m.data(), v.data(), n.data(), (int)p.size(), h, gsq,
                                    (hipStream_t)stream);
  return e == hipSuccess ? MSQ_OK : hip_error(e, "msq_adamw_step launch");
}

}  // extern "C"
