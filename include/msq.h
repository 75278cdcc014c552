/*
 * msq.h -- C ABI of the MI355X (gfx950) streamed NF4 + LoRA training hot path.
 *
 * The operations follow the problem the source pages state: a frozen, 4-bit
 * (NF4) base is read block by block while only LoRA adapters are trained; the
 * backward reloads each block, recomputes its forward with the same dropout
 * masks and differentiates only the adapters and the block input ("Poros"
 * research post, the paragraphs on streamed residency, RNG state capture and
 * the training step; package README, "How it works").
 *
 * Conventions shared by every entry point
 *   - All pointers are device pointers unless a comment says "host".
 *   - bf16 tensors are passed as uint16_t bit patterns; all matrices are dense
 *     row-major with no padding between rows.
 *   - msq_stream_t is a hipStream_t (NULL = the legacy null stream).  Every
 *     compute call is asynchronous on the stream it is given and never
 *     synchronises the host.
 *   - The caller owns all device memory (inputs, outputs, workspaces, the
 *     window arena); the library allocates no device memory.  The one exception
 *     is nf4_lora_fwd_noalloc's scratch, a static array of the library's device
 *     code, which the runtime provides when the code is loaded on a GPU.
 *   - Every function returns 0 on success or a negative MSQ_E_* code.  All
 *     arguments are validated on the host before any HIP call, so an invalid
 *     call launches nothing and leaves outputs untouched.  msq_last_error()
 *     returns a thread-local description of the most recent failure.
 *   - Results are deterministic: tiling and reduction order depend only on the
 *     shapes and on r, never on pointers, alignment, timing or free memory, and
 *     no kernel uses floating-point atomics.  Identical calls on identical bytes
 *     give identical bytes, wherever the operands live (this is what makes a
 *     streamed run bit-identical to a resident one).
 */
#ifndef MSQ_H
#define MSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSQ_ABI_VERSION 15

typedef void* msq_stream_t; /* hipStream_t */

enum {
  MSQ_OK = 0,
  MSQ_E_INVAL = -1,     /* null pointer, negative size, misaligned pointer, bad flag */
  MSQ_E_SHAPE = -2,     /* k % 64 != 0, n % 64 != 0, r outside [0, 64], t*k too large */
  MSQ_E_DROPOUT = -3,   /* p_drop outside [0, 1), or alpha not finite */
  MSQ_E_WORKSPACE = -4, /* workspace smaller than nf4_lora_workspace_size() */
  MSQ_E_WINDOW = -5,    /* arena cannot hold n_slots windows; message names the
                           largest window_blocks that fits */
  MSQ_E_ORDER = -6,     /* window protocol violated (acquire before prefetch,
                           prefetch with no free slot, release of a slot not held) */
  MSQ_E_HIP = -7        /* a HIP runtime call failed; msq_last_error() has its text */
};

/* ABI version of the loaded library (MSQ_ABI_VERSION). */
int msq_abi_version(void);
/* Static description of an error code. */
const char* msq_strerror(int code);
/* Thread-local text of the most recent error raised on this thread ("" if none). */
const char* msq_last_error(void);

/* Host-only: the 16 NF4 levels (ascending, fp32) the kernels use.  out: host,
 * 16 floats.  The levels are computed by the library itself from the NormalFloat
 * construction (8 positive and 7 negative normal quantiles plus an exact zero,
 * normalised to [-1, 1]).  Never touches the GPU. */
int msq_nf4_codebook(float* out);

/* ------------------------------------------------------------------------- */
/* NF4 quantization of the frozen base.
 * The pages name the base format (NF4 via bitsandbytes: "Limitations", "What
 * 0.00e+00 means"; A100 results, "Configuration") but not its parameters; this
 * ABI fixes them: blocks of 64 consecutive elements of the row-major matrix,
 * one fp32 absmax per block, code = nearest level of w/absmax decided exactly
 * (ties to the lower code; an all-zero block stores absmax 0 and code 7),
 * two codes per byte with the even element in the high nibble.
 *
 *   w      [n, k] bf16, finite values (non-finite input gives unspecified codes)
 *   codes  [n, k/2] uint8  (output), 16-byte aligned
 *   absmax [n, k/64] fp32  (output), 4-byte aligned
 * Requires n >= 0, k % 64 == 0, w 16-byte aligned.  n == 0 is a no-op (pointers
 * may then be NULL). */
int nf4_quantize(const uint16_t* w, int64_t n, int64_t k, uint8_t* codes, float* absmax,
                 msq_stream_t stream);

/* Dequantization to bf16: w[i] = bf16_rne(fp32(level[code_i] * absmax_block)).
 * Same layouts and requirements as nf4_quantize; w is the output. */
int nf4_dequantize(const uint8_t* codes, const float* absmax, int64_t n, int64_t k, uint16_t* w,
                   msq_stream_t stream);

/* ------------------------------------------------------------------------- */
/* Dropout key.  The mask of one projection's LoRA input element (t, kk), with
 * e = t*k + kk, is word (e & 3) of Philox4x32-10 (Salmon et al., SC'11) at
 *   counter (e >> 2, (layer << 4) | proj, step, micro), key (seed lo32, seed hi32);
 * the element is kept iff word >= floor(p_drop * 2^32), and kept elements are
 * scaled by fp32(1 / fp32(1 - p_drop)).  Replaces the pages' RNG snapshot and
 * restore ("Poros" research post, RNG state capture): the same key replays the
 * same mask in the recompute.  proj: q 0, k 1, v 2, o 3, gate 4, up 5, down 6. */
typedef struct {
  uint64_t seed;
  uint32_t step;
  uint32_t micro;
  uint32_t layer;
  uint32_t proj; /* < 16 */
} msq_rng_key;

/* LoRA adapter configuration: scaling s = alpha / r; r == 0 means base only
 * (A, B, u are ignored and may be NULL).
 * flags selects the activation dtypes:
 *   MSQ_ACT_F32  x (forward and backward) and dy (backward) are fp32 instead of
 *                bf16.  The base-weight contraction still runs on bf16 MFMA: the
 *                library rounds the activation to bf16 (RNE) for that product only;
 *                the rank-r LoRA products keep fp32 accuracy.
 *   MSQ_OUT_F32  y (forward) and dx (backward) are written (and, when
 *                accumulating, read) as fp32 instead of bf16.
 *   MSQ_U_ONLY   forward only: compute u = drop(x) A^T and skip y (y may be NULL).
 *                For the recompute of a projection whose output the backward never
 *                reads (the last projection of a block): its backward needs only its
 *                input and u. */
#define MSQ_ACT_F32 1u
#define MSQ_OUT_F32 2u
#define MSQ_U_ONLY 4u
/*   MSQ_U_GIVEN  forward only (single calls and groups): u_out holds u = drop(x) A^T from an
 *                earlier call with the same x, A and key, and the call uses it instead of
 *                forming it (u_out is read, not written).  For the recompute of a block whose
 *                first forward kept its u: the recompute's y is the same as the first one's
 *                without the rank-r product.  Needs r > 0 and u_out (every projection's, for
 *                a group); not with MSQ_U_ONLY (MSQ_E_INVAL). */
#define MSQ_U_GIVEN 32u
/* Path of a single call (nf4_lora_fwd/bwd, bf16_lora_fwd/bwd; groups always take the
 * tiled path and reject MSQ_PATH_SMALL):
 *   tiled:  512-token x 128-column tiles with the reduction split across workgroups
 *           (a packing pass, the rank-r product reduction, the GEMM, the split sum);
 *   small:  64 x 64 tiles, each over the whole reduction (one launch per forward; the
 *           backward's input gradient with du in one launch, then the column gradients).
 * Neither flag: the small-tile path when r <= 32 with r % 4 == 0, t <= 1024 and k, n <= 1024
 * (shapes at which the tiled launches are latency-bound), else the tiled path.
 * MSQ_PATH_SMALL needs r <= 32 with r % 4 == 0 (MSQ_E_SHAPE otherwise).  The two paths agree within fp32 rounding order
 * (the oracle's parity bar holds for both); each is bitwise reproducible on its own. */
#define MSQ_PATH_TILED 8u
#define MSQ_PATH_SMALL 16u
typedef struct {
  int32_t r;      /* 0 .. 64 */
  float alpha;
  float p_drop;   /* dropout probability on the LoRA input, in [0, 1) */
  uint32_t flags; /* MSQ_ACT_F32 | MSQ_OUT_F32 | MSQ_U_ONLY | MSQ_U_GIVEN | MSQ_PATH_*, other bits 0 */
} msq_lora_cfg;

/* Bytes of scratch device memory one nf4_lora_fwd or nf4_lora_bwd call with
 * these shapes needs (split reduction partials, u/du staging).  Depends only on
 * the shapes.  Returns 0 for invalid shapes. */
size_t nf4_lora_workspace_size(int64_t t, int64_t k, int64_t n, int32_t r);

/* Fused forward of one NF4 frozen linear with a LoRA adapter:
 *   u = drop(x) A^T                   (fp32, written to u_out when non-NULL)
 *   y = x W^T + bias + (alpha/r) u B^T
 * where W is the dequantized NF4 matrix [n, k] (dequantized in-tile, never
 * materialised).  x and y are bf16 unless cfg.flags says fp32 (see msq_lora_cfg).
 *   x      [t, k], 16-byte aligned                  t >= 0, k % 64 == 0
 *   codes  [n, k/2] uint8, absmax [n, k/64] fp32     n % 64 == 0
 *   bias   [n] bf16 or NULL
 *   residual [t, n] in y's type, 16-byte aligned, or NULL.  When set, the output is
 *          residual + (the y above), the residual connection of a decoder block fused
 *          into this output pass (a pointwise fusion of the kind the pages allow for
 *          kernels around the engine, "Poros" README, Roadmap, "The Poros kernel"): y
 *          is formed and rounded to y's type as without it, and the one addition is
 *          the same rounded operation as a separate residual add.  May equal y.
 *   A      [r, k] fp32, B [n, r] fp32  (16-byte aligned)
 *   y      [t, n] output (16-byte aligned)
 *   u_out  [t, r] fp32 output or NULL
 *   workspace: device scratch of at least nf4_lora_workspace_size(t, k, n, r)
 *   bytes, 256-byte aligned; contents on entry are ignored.
 * t == 0 is a no-op (x, y may then be NULL).  t * k must stay below 2^34 (dropout
 * counter range) and t at most 65535. */
int nf4_lora_fwd(const void* x, int64_t t, int64_t k, int64_t n, const uint8_t* codes,
                 const float* absmax, const uint16_t* bias, const void* residual, const float* A,
                 const float* B, msq_lora_cfg cfg, msq_rng_key key, void* y, float* u_out,
                 void* workspace, size_t workspace_bytes, msq_stream_t stream);

/* Fused backward of the same layer (no gradient for W, absmax or bias: frozen).
 *   du = s dy B                       (s = alpha / r)
 *   dB = s dy^T u
 *   dA = du^T drop(x)                 (mask replayed from key)
 *   dx = dy W + sigma * keep (.) (du A)
 *   dy [t, n], x [t, k] (the forward's input): bf16, or fp32 with MSQ_ACT_F32
 *   u  [t, r] fp32 from the forward (or recompute), or NULL to recompute it here
 *   dx [t, k] output (bf16, or fp32 with MSQ_OUT_F32); dx_accumulate = 1 adds into
 *      the existing dx (the sum is formed in fp32 and rounded once), 0 overwrites
 *   dA [r, k] fp32, dB [n, r] fp32 outputs; dAB_accumulate = 1 adds into them
 *   dA/dB may be NULL only when r == 0.  With t == 0, dy, x and dx may be NULL and dA,
 *   dB are set to zero (or left unchanged when accumulating).
 * Shapes, alignment and workspace as for nf4_lora_fwd. */
int nf4_lora_bwd(const void* dy, const void* x, int64_t t, int64_t k, int64_t n,
                 const uint8_t* codes, const float* absmax, const float* A, const float* B,
                 msq_lora_cfg cfg, msq_rng_key key, const float* u, void* dx,
                 int dx_accumulate, float* dA, float* dB, int dAB_accumulate, void* workspace,
                 size_t workspace_bytes, msq_stream_t stream);

/* nf4_lora_fwd for callers that cannot allocate device memory at the call: code under
 * HIP stream capture, tight serving loops, harnesses that forbid hipMalloc.  Arguments,
 * outputs, dropout keys and results are nf4_lora_fwd's (the same kernels), except that
 * there is no workspace argument: the scratch lives in a static device array of the
 * library, MSQ_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, held from the first call on that
 * GPU until the process ends.  The call allocates and frees nothing.
 *   - A shape whose nf4_lora_workspace_size() exceeds MSQ_NOALLOC_SCRATCH_BYTES returns
 *     MSQ_E_WORKSPACE before any HIP call (at 512 tokens, r = 16, every projection of the
 *     Qwen2.5 0.5B .. 72B shapes fits: the largest needs 96.6 MiB).
 *   - The array is found on the stream's device (the current device for the NULL stream);
 *     its address is looked up once per device.
 *   - Every call on one GPU shares that GPU's array and nothing in it has to start at zero.
 *     Calls that may run at the same time on one GPU (different streams, or threads) race
 *     on it and give undefined results: serialise them on one stream. */
#define MSQ_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int nf4_lora_fwd_noalloc(const void* x, int64_t t, int64_t k, int64_t n, const uint8_t* codes,
                         const float* absmax, const uint16_t* bias, const void* residual, const float* A,
                         const float* B, msq_lora_cfg cfg, msq_rng_key key, void* y, float* u_out,
                         msq_stream_t stream);

/* The same layer over a frozen base kept in bf16 instead of NF4: the pages' bf16
 * streaming variant, which streams the base blockwise like NF4 at 4x the bytes and is
 * held to the same bitwise parity ("Current limitations", "bf16 LoRA").
 *   w  [n, k] bf16, row-major, 16-byte aligned (replaces codes and absmax)
 * Every other argument, the workspace (nf4_lora_workspace_size), the outputs, the
 * dropout keys and the error behaviour are those of nf4_lora_fwd / nf4_lora_bwd. */
int bf16_lora_fwd(const void* x, int64_t t, int64_t k, int64_t n, const uint16_t* w,
                  const uint16_t* bias, const void* residual, const float* A, const float* B,
                  msq_lora_cfg cfg, msq_rng_key key, void* y, float* u_out, void* workspace,
                  size_t workspace_bytes, msq_stream_t stream);
int bf16_lora_bwd(const void* dy, const void* x, int64_t t, int64_t k, int64_t n, const uint16_t* w,
                  const float* A, const float* B, msq_lora_cfg cfg, msq_rng_key key, const float* u,
                  void* dx, int dx_accumulate, float* dA, float* dB, int dAB_accumulate,
                  void* workspace, size_t workspace_bytes, msq_stream_t stream);

/* Grouped forward: up to 3 projections of the same input x [t, k] (a decoder block's
 * q/k/v, or gate/up) in one pass.  x is packed for the MFMA once, each projection's
 * rank-r product is formed with its own key and A, and one GEMM launch covers the column
 * tiles of all of them with one split plan, so the narrow projections no longer leave
 * most of the chip idle.  Each projection's outputs are those of nf4_lora_fwd (or
 * bf16_lora_fwd) with the same arguments, up to the fp32 summation order of the split
 * reduction, which the group's plan fixes.
 *   projs   n_proj (1..3) descriptors: n, the base (codes + absmax, or w; one format per
 *           group), bias, residual, A, B, the projection's rng key, y and u_out (or NULL),
 *           with the alignment and shapes of nf4_lora_fwd
 *   cfg     r, alpha, p_drop and the activation / output flags shared by the group
 *           (MSQ_U_ONLY is rejected)
 *   workspace  >= lora_group_workspace_size(t, k, projs, n_proj, r) bytes (0 for invalid
 *           descriptors), 256-byte aligned. */
typedef struct {
  int64_t n;
  const uint8_t* codes;
  const float* absmax;
  const uint16_t* w;
  const uint16_t* bias;
  const void* residual;
  const float* A;
  const float* B;
  msq_rng_key key;
  void* y;
  float* u_out;
} msq_lora_proj;

size_t lora_group_workspace_size(int64_t t, int64_t k, const msq_lora_proj* projs, int n_proj, int32_t r);
int lora_fwd_group(const void* x, int64_t t, int64_t k, const msq_lora_proj* projs, int n_proj,
                   msq_lora_cfg cfg, void* workspace, size_t workspace_bytes, msq_stream_t stream);

/* Grouped backward of up to 3 projections of the same input x [t, k] (q/k/v, or
 * gate/up): the gradients of nf4_lora_bwd (or bf16_lora_bwd) for each projection, with
 * their input gradients summed into one dx,
 *   dx = sum_i ( dy_i W_i + sigma * keep_i (.) (du_i A_i) ),   du_i = s dy_i B_i,
 * which is the backward of the block's use of x in the pages' training step ("Poros"
 * research post, the training-step paragraph: gradients reach only the adapters and the
 * activations).  The sum over i is one reduction over the projections' concatenated W rows
 * (a single GEMM launch with one split plan, each projection's LoRA term added with its
 * own key and keep mask), so a narrow k/v backward no longer runs as a launch of its own;
 * dx therefore equals the sum of the single calls' dx up to fp32 summation order.  dA_i
 * and dB_i are those of the single call with the same arguments.
 *   projs   n_proj (1..3) descriptors: n (% 64 == 0), the base (codes + absmax, or w; one
 *           format per group), A, B, the projection's rng key, dy [t, n] (x's type), u
 *           [t, r] fp32 from the forward or NULL to recompute, and the outputs dA [r, k],
 *           dB [n, r] fp32 (NULL only when r == 0); alignment as in nf4_lora_bwd
 *   dx      [t, k] output (bf16, or fp32 with MSQ_OUT_F32); dx_accumulate = 1 adds the sum
 *           into the existing dx (one rounding), 0 overwrites
 *   dAB_accumulate = 1 adds into every dA_i, dB_i
 *   cfg     r, alpha, p_drop and the activation / output flags shared by the group
 *           (MSQ_U_ONLY is rejected)
 *   workspace  >= lora_group_bwd_workspace_size(t, k, projs, n_proj, r) bytes (0 for
 *           invalid descriptors), 256-byte aligned.
 * t == 0: dA_i, dB_i are set to zero (or left unchanged when accumulating); x, dx and dy
 * may be NULL.  t * (sum of n) must stay below 2^34. */
typedef struct {
  int64_t n;
  const uint8_t* codes;
  const float* absmax;
  const uint16_t* w;
  const float* A;
  const float* B;
  msq_rng_key key;
  const void* dy;
  const float* u;
  float* dA;
  float* dB;
} msq_lora_proj_grad;

size_t lora_group_bwd_workspace_size(int64_t t, int64_t k, const msq_lora_proj_grad* projs, int n_proj,
                                     int32_t r);
int lora_bwd_group(const void* x, int64_t t, int64_t k, const msq_lora_proj_grad* projs, int n_proj,
                   msq_lora_cfg cfg, void* dx, int dx_accumulate, int dAB_accumulate, void* workspace,
                   size_t workspace_bytes, msq_stream_t stream);

/* ------------------------------------------------------------------------- */
/* Pointwise block glue of a Qwen2.5-style decoder block, fp32.
 * The pages allow fusing kernels around the engine only where the fused chain is
 * pointwise and yields the same per-element values as the unfused one, naming the
 * SwiGLU multiply, residual adds and rotary embedding with precomputed tables
 * ("Poros" README, Roadmap, "The Poros kernel"); reductions (RMSNorm's mean, softmax)
 * stay unfused.  Each entry evaluates the unfused chain's operations in the same order
 * with the same fp32 roundings (products rounded where the unfused chain stores them;
 * the one multiply-add it fuses, in the SiLU derivative, fused here too), so its result
 * is that chain's element for element.  All tensors are contiguous device fp32, 16-byte
 * aligned; outputs may not alias inputs.  n == 0 (t == 0) is a no-op; n (t*heads*d)
 * above 2^40 is MSQ_E_SHAPE, a null or misaligned pointer MSQ_E_INVAL.
 *
 * msq_swiglu_fwd:  a = silu(g) * u,  silu(g) = g / (1 + exp(-g)), n elements.
 * msq_swiglu_bwd:  du = da * silu(g);  dg = ((da * u) * s) * (1 + g * (1 - s)),
 *                  s = 1 / (1 + exp(-g)), with 1 + g * (1 - s) one fused multiply-add
 *                  -- the product rule followed by the SiLU derivative, as the two
 *                  unfused steps compute them.  The one exception to the no-alias rule:
 *                  dg may be g and du may be u (in place; each element's three inputs
 *                  are read before its two outputs are written), so a backward that
 *                  no longer needs g and u can take its gradients without new memory.
 *                  Partial overlaps remain invalid. */
int msq_swiglu_fwd(const float* g, const float* u, int64_t n, float* a, msq_stream_t stream);
int msq_swiglu_bwd(const float* da, const float* g, const float* u, int64_t n, float* dg,
                   float* du, msq_stream_t stream);

/* Rotary position embedding, rotate-half pairing (element i with i + d/2):
 *   x, y   [t, heads, d] (d even; heads, d >= 1), cos_t, sin_t [t, d] tables
 *   forward   y_i = x_i cos_i + (-x_{i+d/2}) sin_i,  y_{i+d/2} = x_{i+d/2} cos_{i+d/2} + x_i sin_{i+d/2}
 *   backward  dx_i = dy_i cos_i + dy_{i+d/2} sin_{i+d/2},
 *             dx_{i+d/2} = dy_{i+d/2} cos_{i+d/2} + (-(dy_i sin_i))
 * (msq_rope_bwd takes dy in x and writes dx in y). */
int msq_rope_fwd(const float* x, const float* cos_t, const float* sin_t, int64_t t, int32_t heads,
                 int32_t d, float* y, msq_stream_t stream);
int msq_rope_bwd(const float* dy, const float* cos_t, const float* sin_t, int64_t t, int32_t heads,
                 int32_t d, float* dx, msq_stream_t stream);

/* RMSNorm's pointwise tail.  r[t] = rsqrt(mean_c h[t][c]^2 + eps) is formed by the
 * caller: it holds a reduction, which stays unfused.
 *   h, y, dy, dh, hdot [t, d] (d % 4 == 0, d >= 4), r [t] (4-byte aligned), w [d] weights
 *   forward   y = (h * r) * w
 *   backward  g = dy * w;  dh = g * r;  hdot = g * h
 * dh is the norm input's gradient through the scaling (its other part runs through r);
 * the caller sums hdot over each row to get dr, the gradient of r.  The weights are
 * frozen: no gradient for w. */
int msq_rmsnorm_apply_fwd(const float* h, const float* r, const float* w, int64_t t, int64_t d,
                          float* y, msq_stream_t stream);
int msq_rmsnorm_apply_bwd(const float* dy, const float* h, const float* r, const float* w, int64_t t,
                          int64_t d, float* dh, float* hdot, msq_stream_t stream);

/* ------------------------------------------------------------------------- */
/* The optimizer step over the adapters ("Poros" research post, training-step paragraph:
 * one optimizer step after the backward, the same step a resident run takes; only the
 * adapters' optimizer state lives on the device).  The pages do not name the optimizer;
 * this is AdamW with decoupled weight decay, for step t >= 1 and every element:
 *   p <- p * (1 - lr * weight_decay)
 *   m <- m + (1 - beta1) * (g - m)
 *   v <- beta2 * v + (1 - beta2) * g^2
 *   p <- p - (lr / (1 - beta1^t)) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * in fp32, the scalar factors formed in double precision on the host.
 *
 * tensors[i]: n elements of fp32 parameters p, their gradient g and the two moments m, v,
 * each contiguous device memory, 16-byte aligned, no two of the four overlapping (and no
 * tensor overlapping another).  The caller owns all of them; p, m and v are updated in
 * place, g is only read.  Moments start at zero before step 1.
 * gsq (optional, NULL to skip): receives msq_adamw_partials(tensors, n) floats, partial
 * sums of g^2 over fixed ranges of elements in tensor order, each summed in a fixed order
 * -- their sum is the squared 2-norm of all the gradients, the same bits on every run.
 * Errors: n_tensors < 0, n < 0, step < 1, lr < 0, beta outside [0, 1), eps <= 0 or
 * weight_decay < 0 -> MSQ_E_INVAL; a null or misaligned pointer of a non-empty tensor
 * -> MSQ_E_INVAL.  Runs asynchronously on `stream`. */
typedef struct msq_adamw_cfg {
  double lr, beta1, beta2, eps, weight_decay; /* double: 1 - beta2 keeps its digits */
} msq_adamw_cfg;
typedef struct msq_adamw_tensor {
  float* p;
  const float* g;
  float* m;
  float* v;
  int64_t n;
} msq_adamw_tensor;
int64_t msq_adamw_partials(const msq_adamw_tensor* tensors, int n_tensors);
int msq_adamw_step(const msq_adamw_tensor* tensors, int n_tensors, msq_adamw_cfg cfg, int64_t step, float* gsq,
                   msq_stream_t stream);

/* Copy `bytes` from src to dst by a kernel on `stream` (in stream order): each side is
 * device memory or pinned host memory (msq_host_alloc, hipHostMalloc), which the kernel
 * reads or writes across the link with its own loads and stores -- no DMA engine, so the
 * copy is not queued behind the window's engine copies ("Poros" research post,
 * training-step paragraph: the block boundaries the forward keeps for the backward may be
 * parked in host memory this way).  src and dst: 16-byte aligned, not overlapping;
 * bytes a multiple of 16 (0 is a no-op).  A pointer that is neither device nor pinned
 * host memory, a null or misaligned pointer, or a bad size -> MSQ_E_INVAL.  The caller
 * owns both buffers and keeps them alive until the copy has run. */
int msq_kernel_copy(const void* src, void* dst, size_t bytes, msq_stream_t stream);

/* ------------------------------------------------------------------------- */
/* Pinned host memory for the frozen base ("Poros" research post: the base lives in
 * host memory between its trips through the window, and host RAM is the other cost of
 * streaming; memory paragraph).  msq_host_alloc pins `bytes` with hipHostMalloc, at
 * that size (no rounding up to a power of two, as a caching allocator may do), and
 * returns a host pointer aligned to at least 256 bytes; msq_host_free releases it (NULL
 * is a no-op).  bytes == 0 or above 2^46, or a NULL out, is MSQ_E_INVAL; a failed
 * allocation is MSQ_E_HIP. */
int msq_host_alloc(size_t bytes, void** out);
int msq_host_free(void* p);

/* ------------------------------------------------------------------------- */
/* Streamed quantizing load.
 * The pages' default loader stages one tensor at a time, quantizes it and evicts it
 * before the next, keeping the load-time device peak far below a standard load, with
 * output byte-identical to the standard load ("Poros" research post, streamed-loader
 * paragraph).  nf4_stream_load turns bf16 host tensors into NF4 codes + absmax in host
 * memory, one row chunk at a time: chunk c is copied into pinned bounce buffer c % 2
 * (host_threads threads), sent to device slot c % 2, quantized by the nf4_quantize
 * kernel and copied back into the job's destinations, the host copy of the next chunk
 * overlapping the device work.  A chunk holds up to chunk_rows * max_cols elements
 * (max_cols = the widest job): more rows for narrower tensors, whole rows always, so
 * the output is nf4_quantize's on the whole tensor, byte for byte.
 *   jobs        n_jobs tensors: src host bf16 [rows][cols] (any host memory, e.g. a
 *               memory-mapped file), cols % 64 == 0; codes [rows][cols/2] and absmax
 *               [rows][cols/64] host destinations (pinned for asynchronous copies)
 *   dev_staging device memory, 256-byte aligned, >= nf4_stream_load_device_bytes
 *   host_bounce pinned host memory, 256-byte aligned, >= nf4_stream_load_host_bytes
 * The call returns when every destination byte is written (it synchronizes `stream`).
 * Errors: MSQ_E_SHAPE for cols % 64, MSQ_E_WORKSPACE for short staging, MSQ_E_INVAL for
 * null or misaligned pointers and bad counts, MSQ_E_HIP for a failed HIP call. */
typedef struct {
  const void* src;
  int64_t rows, cols;
  uint8_t* codes;
  float* absmax;
} msq_quant_job;

size_t nf4_stream_load_device_bytes(int64_t max_cols, int64_t chunk_rows);
size_t nf4_stream_load_host_bytes(int64_t max_cols, int64_t chunk_rows);
int nf4_stream_load(const msq_quant_job* jobs, int n_jobs, int64_t chunk_rows, void* dev_staging,
                    size_t dev_bytes, void* host_bounce, size_t host_bytes, int host_threads,
                    msq_stream_t stream);

/* ------------------------------------------------------------------------- */
/* Host-to-device block-prefetch window.
 * The pages: the forward streams frozen blocks through a small GPU window with
 * asynchronous prefetch on side streams, the backward reloads each block in
 * reverse, and eviction is a pointer release because the base is read-only
 * ("Poros" research post, the training-step paragraph; "Limitations",
 * "Pretraining is out of scope"; README, "How it works").
 *
 * A window groups window_blocks consecutive layers; the caller's device arena is
 * split into n_slots slots of one window each (n_slots >= 2: one computing while
 * the next loads; more slots let the copies run further ahead).  With
 * window_blocks = 1 and n_slots = 2B the same arena as B-block windows double
 * buffered becomes a ring of single-layer slots, released and refilled layer by
 * layer.  Layer blobs live in pinned host memory (msq_host_alloc, hipHostMalloc or
 * registered memory; checked at creation) and are copied with hipMemcpyAsync, layer l
 * on copy_streams[l % n_copy_streams].  Position q of a slot (the q-th layer of the
 * window it holds) has a fixed byte range, as large as the largest layer at position q
 * of any window (sizes rounded up to 256 bytes), so the ranges of different positions
 * never overlap and a copy needs to wait only for the layer it overwrites.  The window
 * object owns only events and bookkeeping; it is not thread-safe.
 *
 *   host_blobs  host array of n_layers pointers to pinned host memory
 *   blob_bytes  host array of n_layers sizes
 *   dev_arena   caller-owned device memory, 256-byte aligned, arena_bytes long;
 *               needs at least block_stream_arena_bytes(...) bytes, else
 *               MSQ_E_WINDOW (the message names the largest window that fits).
 *   copy_streams host array of 1 .. MSQ_MAX_COPY_STREAMS streams (keep them at the
 *               default priority).  Two streams let one layer's copy run while the next
 *               waits for its position to be released.
 * A blob that is not pinned host memory over its whole range is MSQ_E_INVAL (a HIP
 * runtime that cannot tell, for instance with no GPU, is MSQ_E_HIP); every other
 * argument is checked before that, without HIP calls.
 * The arrays are copied; the blobs and the arena must outlive the window. */
#define MSQ_MAX_COPY_STREAMS 4
typedef struct msq_window msq_window;

typedef struct {
  uint64_t bytes_copied;    /* host-to-device bytes issued */
  uint64_t windows_copied;  /* window loads that issued copies */
  uint64_t windows_reused;  /* prefetches satisfied by a slot that still held the window */
  double copy_ms;           /* summed durations of the layer copies (events around each
                               copy, after its waits) */
  uint64_t copies_timed;    /* layer copies included in copy_ms */
  double busy_ms;           /* time at least one copy stream was copying: the union of the
                               copies' spans (equals copy_ms with one copy stream) */
} msq_window_stats;

size_t block_stream_arena_bytes(const size_t* blob_bytes, int n_layers, int window_blocks,
                                int n_slots);
int block_stream_create(msq_window** out, const void* const* host_blobs, const size_t* blob_bytes,
                        int n_layers, int window_blocks, int n_slots, void* dev_arena,
                        size_t arena_bytes, const msq_stream_t* copy_streams, int n_copy_streams);
/* Start loading the window that begins at first_layer (a multiple of
 * window_blocks) into a free slot (the least recently released one): the copy
 * stream first waits until the compute stream released that slot, then copies,
 * then marks it ready.  If a free slot still holds this window's bytes, no copy is
 * issued.  No free slot: MSQ_E_ORDER. */
int block_stream_prefetch(msq_window* w, int first_layer);
/* Make `compute` wait until `layer` (of a prefetched window) has arrived, and return
 * the layer's device address.  Window not prefetched: MSQ_E_ORDER. */
int block_stream_acquire(msq_window* w, int layer, msq_stream_t compute, const void** dev_blob);
/* Mark the window beginning at first_layer as no longer read by work queued so
 * far on `compute` (its layers not yet released, in ascending order); its slot may then
 * be refilled.  Not held: MSQ_E_ORDER. */
int block_stream_release(msq_window* w, int first_layer, msq_stream_t compute);
/* Release one layer of a held window as soon as the work queued so far on `compute` no
 * longer reads it.  Once every layer of the window is released the slot may be refilled;
 * the next window's layers are then copied in the order these layers were released, each
 * copy waiting only for the layer it overwrites, and block_stream_acquire waits only for
 * the acquired layer's own copy.  Window not held: MSQ_E_ORDER; released twice:
 * MSQ_E_ORDER. */
int block_stream_release_layer(msq_window* w, int layer, msq_stream_t compute);
/* Statistics since creation.  Waits for the issued copies to finish so that their
 * durations are included (call it outside timed regions).  The other window calls
 * never wait: a copy's duration is read from its events once they have completed. */
int block_stream_stats(msq_window* w, msq_window_stats* out);
/* Waits for the window's outstanding copies, then frees its events. */
int block_stream_destroy(msq_window* w);

/* ------------------------------------------------------------------------- */
/* Kernel timing (measurement support).  When enabled, every kernel launch of the
 * library carries a start and a stop HIP event recorded by the dispatch on the launch
 * stream.  msq_timing_collect waits for the recorded events and aggregates, per label
 * "<kernel> <shape>" (the dense GEMMs: "<t>x<n>x<k>"; the memory-bound LoRA-side
 * kernels: their token and column counts), the launch count, total milliseconds, total
 * algorithmic flops (2*t*k*n per GEMM launch) and total algorithmic bytes.  Host-side
 * bookkeeping only. */
typedef struct {
  char name[48];
  uint64_t launches;
  double total_ms;
  double total_flops;  /* algorithmic flops (dense MFMA kernels) */
  double total_bytes;  /* algorithmic HBM bytes: every input read once, every output written once */
} msq_kernel_timing;

/* on: 0 off, 1 every launch, 2 only the launches with algorithmic flops (the dense MFMA
 * GEMMs), which keeps the per-launch host bookkeeping off the many small kernels. */
int msq_timing_enable(int on);
/* Fills up to max entries; *n_out = number of kernel names seen.  Resets. */
int msq_timing_collect(msq_kernel_timing* out, int max, int* n_out);
/* Creates timing events ahead of use until at least `events` are pooled (two per timed
 * launch), so that a timed region creates none: creating an event costs host time that
 * would otherwise slow the launches being timed.  events < 0 -> MSQ_E_INVAL; a HIP
 * failure -> MSQ_E_HIP. */
int msq_timing_reserve(int events);

#ifdef __cplusplus
}
#endif

#endif /* MSQ_H */
