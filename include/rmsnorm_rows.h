/*
 * rmsnorm_rows.h -- C ABI of the MI355X (gfx950) row-normalization library.
 *
 * Operations
 * ----------
 * RMSNorm of a row x of length H with weight w:
 *     y_i = (w_i + b) * x_i * rsqrt( (1/H) * sum_j x_j^2 + eps ),   b in {0, 1}
 * as computed by the _qk_norm_kernel listing in the "QK Norm" section of
 * "CuTeDSL at Perplexity" (Perplexity blog): sum of squares accumulated in
 * float32, eps added to the mean inside the rsqrt, (w + WEIGHT_BIAS) times the
 * normalized row, one cast back to the storage type.  The page's "Inference at
 * Perplexity" section names the weight bias (plain w, or 1 + w) as a knob of
 * RMS norm; here it is the RN_FLAG_WEIGHT_PLUS_ONE flag and is specialized at
 * compile time.  With it, (1 + w) t is evaluated as the float32 fused
 * multiply-add w t + t (one rounding of the exact product).
 *
 * rmsnorm_fwd adds an optional residual stream in front of the norm (fused
 * residual add): h = round_res(x + residual) is written to residual_out and the
 * norm is taken over that rounded h.  It can also quantize y to OCP fp8 E4M3FN
 * with one dynamic scale per row: scale = amax / 448, amax = max_i |y_i|,
 * code_i = round_nearest_even(y_i / scale) saturated to +-448, or with the
 * block-scaled schemes of RN_SCALE_* below (fp8 per 128 elements; MX per 32,
 * fp8 or fp4 E2M1; NVFP4 per 16).  Neither the residual add nor the quantized
 * outputs' formulas are on the pages; both follow the plain reading stated
 * for each entry point below.  rmsnorm_fwd_call takes the same call as one
 * record, for callers that repeat a decode call on fixed buffers.
 *
 * qknorm_fwd applies the same RMSNorm to every (token, head) row of Q and K
 * over head_dim, with one weight vector per tensor shared by all heads, as in
 * the "QK Norm" section's kernel (heads of Q first, then heads of K, per token).
 *
 * rmsnorm_fwd_partials is the same fused add + norm with x given as a sum of
 * up to 8 partial tensors (summed exactly in the kernel, rounded once).
 *
 * silu_mul_fwd is the SwiGLU activation over rows of a merged gate/up
 * projection, with the same output types as rmsnorm_fwd.
 *
 * rn_launch_empty and rn_launch_copy are measurement references (bare launch
 * latency; streaming-copy bandwidth) launched through the same path.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are caller-owned DEVICE memory on the current HIP
 *    device, row-major and contiguous unless a stride argument says otherwise,
 *    and 16-byte aligned.  The library never allocates, frees or synchronizes;
 *    work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  The only global state is a per-device cache of the compute
 *    unit count, filled on first use (thread-safe).  Entry points are
 *    re-entrant.
 *  - Arguments are checked on the host before any HIP call, so every error in
 *    the table below is reported synchronously and without a GPU:
 *        RN_ERR_INVALID_ARG  missing pointer, bad size, bad eps, unknown flag
 *                            bits, inconsistent optional arguments;
 *        RN_ERR_UNSUPPORTED  a dtype combination or size this build does not
 *                            provide (e.g. H not a multiple of the 16-byte vector);
 *        RN_ERR_MISALIGNED   a pointer or row stride that is not 16-byte aligned;
 *        RN_ERR_HIP          a HIP runtime call failed (device query or launch).
 *    A fault inside a kernel surfaces asynchronously, at the caller's next
 *    synchronization.  rn_last_error() returns a message for the last non-OK
 *    status on the calling thread.
 *  - rows == 0 (or tokens == 0) is a valid no-op: RN_OK, nothing launched,
 *    pointers may then be NULL.
 */
#ifndef RMSNORM_ROWS_H
#define RMSNORM_ROWS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RN_ABI_VERSION 4

typedef enum rn_status {
  RN_OK = 0,
  RN_ERR_INVALID_ARG = 1,
  RN_ERR_UNSUPPORTED = 2,
  RN_ERR_MISALIGNED = 3,
  RN_ERR_HIP = 4
} rn_status;

/* Element types. */
#define RN_DTYPE_BF16 0u       /* bfloat16 */
#define RN_DTYPE_F32 1u        /* IEEE binary32 */
#define RN_DTYPE_FP8_E4M3FN 2u /* OCP fp8 E4M3FN, outputs only, with scales (see RN_SCALE_*) */
#define RN_DTYPE_FP4_E2M1 3u   /* OCP MX fp4 E2M1, outputs only, two codes per byte (element 2k
                                  in the low nibble), with MX or NVFP4 scales */

/* Scale granularity of a quantized output (flags bits 9-10), after the
 * block-scaled schemes of the "Blackwell support" section (MXFP8, MXFP4, NVFP4, FP8
 * block-wise scaling), with the formats of the OCP FP8 and MX specifications:
 *   RN_SCALE_ROW       fp8: one float32 scale amax/448 per row, amax = max|y| of the row
 *   RN_SCALE_GROUP128  fp8: one float32 scale amax/448 per 128 consecutive elements
 *                      (hidden % 128 == 0); an all-zero group has scale 0
 *   RN_SCALE_MX32      fp8 or fp4: one E8M0 byte per 32 consecutive elements (hidden % 32
 *                      == 0) holding e + 127 with e = clamp(floor(log2 amax) - emax, -127,
 *                      127), emax = 8 (fp8) or 2 (fp4); codes encode y * 2^-e with
 *                      saturation; an all-zero block has e = -127
 *   RN_SCALE_NV16      fp4 only (NVFP4, named with its absolute maximum over 16 elements in
 *                      the same section): one OCP E4M3FN byte per 16 consecutive elements
 *                      (hidden % 16 == 0) and a float32 tensor scale s_t > 0 supplied by the
 *                      caller (tensor_scale, device memory).  Reading: block scale code
 *                      s_b = e4m3fn(amax / (6 s_t)) -- float32 division by fl32(6 s_t),
 *                      then nearest-even, saturating at 448 -- and element codes
 *                      e2m1(y * rcp(fl32(value(s_b) * s_t))), rcp the hardware reciprocal
 *                      (within an ulp); a block scale of 0 gives zero codes.
 *                      Dequantize as value(code) * value(s_b) * s_t.
 * Codes round to nearest, ties to even, and saturate at the format's largest value. */
#define RN_SCALE_ROW 0u
#define RN_SCALE_GROUP128 1u
#define RN_SCALE_MX32 2u
#define RN_SCALE_NV16 3u

/* flags: bits 0-1 dtype of x, bits 2-3 dtype of residual and residual_out,
 * bits 4-5 dtype of weight, bits 6-7 dtype of out, bit 8 weight form (1 + w),
 * bits 9-10 scale granularity of a quantized out (RN_SCALE_*).
 * qknorm_fwd uses bits 0-1 for q/k (in and out), bits 4-5 for the weights and
 * bit 8; its other bits must be zero. */
#define RN_FLAGS_X_SHIFT 0
#define RN_FLAGS_RES_SHIFT 2
#define RN_FLAGS_W_SHIFT 4
#define RN_FLAGS_OUT_SHIFT 6
#define RN_FLAG_WEIGHT_PLUS_ONE (1u << 8)
#define RN_FLAGS_SCALE_SHIFT 9
#define RN_FLAGS_KNOWN_MASK 0x7FFu
#define RN_MAKE_FLAGS(x_dt, res_dt, w_dt, out_dt, plus_one)                                   \
  (((uint32_t)(x_dt) << RN_FLAGS_X_SHIFT) | ((uint32_t)(res_dt) << RN_FLAGS_RES_SHIFT) |     \
   ((uint32_t)(w_dt) << RN_FLAGS_W_SHIFT) | ((uint32_t)(out_dt) << RN_FLAGS_OUT_SHIFT) |     \
   ((plus_one) ? RN_FLAG_WEIGHT_PLUS_ONE : 0u))

/* Kernel families reported by the query functions. */
#define RN_KERNEL_ROWS 0  /* one workgroup of waves_per_row wave64s per row */
#define RN_KERNEL_HEADS 1 /* lanes_per_row lanes per (token, head) row, several rows per wave */

/* Launch configuration chosen by the host-side selector (or given explicitly). */
typedef struct rn_launch_config {
  int32_t kernel;        /* RN_KERNEL_ROWS or RN_KERNEL_HEADS */
  int32_t vec;           /* elements per lane vector: 16 bytes of x (8 bf16 or 4 f32) */
  int32_t waves_per_row; /* RN_KERNEL_ROWS: wave64s sharing one row (1..16); 1 = no LDS, no barrier */
  int32_t vecs_per_lane; /* RN_KERNEL_ROWS: vectors each lane holds (1, 2, 4 or 8) */
  int32_t lanes_per_row; /* RN_KERNEL_HEADS: lanes per head (head_dim / vec); ROWS: 64 * waves_per_row */
  int32_t rows_per_lane; /* RN_KERNEL_HEADS: heads each lane group normalizes (1, 2 or 4); ROWS: 1 */
  int32_t block_threads; /* workgroup size */
  int32_t reserved;      /* zero */
  int64_t grid;          /* workgroups launched; ROWS: at most rows, each workgroup strides over rows */
} rn_launch_config;

/*
 * Fused residual add + RMSNorm over rows.
 *
 *   x            [rows, hidden] of dtype flags.x                       (read)
 *   residual     [rows, hidden] of dtype flags.res, or NULL for no residual add (read)
 *   weight       [hidden] of dtype flags.w                             (read)
 *   out          [rows, hidden] of dtype flags.out: fp8 one byte per element, fp4 half a
 *                byte (hidden / 2 bytes per row)                      (write)
 *   residual_out [rows, hidden] of dtype flags.res; must be NULL iff residual is NULL (write)
 *   out_scale    quantized output only (else NULL): float32 [rows] (RN_SCALE_ROW),
 *                float32 [rows, hidden/128] (RN_SCALE_GROUP128), uint8 E8M0
 *                [rows, hidden/32] (RN_SCALE_MX32) or uint8 E4M3FN [rows, hidden/16]
 *                (RN_SCALE_NV16)                                       (write)
 *   rows         >= 0;  hidden >= 1, a multiple of the lane vector (8 for bf16 x,
 *                4 for f32 x) and at most 32768 (bf16 x) / 16384 (f32 x): the
 *                whole row is held in registers, 4096 lane vectors at most
 *   eps          finite, >= 0, used as given (a float32)
 *   flags        RN_MAKE_FLAGS(...) | (scale << RN_FLAGS_SCALE_SHIFT); x is bf16 or f32;
 *                the residual dtype is the x dtype or f32; weight bf16 or f32; out bf16,
 *                f32, fp8 (row, per-128 or MX scales) or fp4 (MX or NVFP4 scales).
 *                RN_SCALE_NV16 needs rmsnorm_fwd_ex's tensor_scale: rmsnorm_fwd
 *                rejects it with RN_ERR_INVALID_ARG.
 *
 * Residual reading (not on the pages): h = x + residual is rounded once to the
 * residual dtype, written to residual_out, and normalized; out == RMSNorm(h).
 * fp8 reading: amax and every y_i are float32 values computed from the same
 * products, scale = amax / 448 is an IEEE float32 division, an all-zero row has
 * scale 0 and all-zero codes.
 * Aliasing: out may equal x (in place) when both have the same element width
 * (else RN_ERR_INVALID_ARG: a narrower or wider out row would overlap other
 * rows of x still being read), and residual_out may equal residual; any other
 * overlap is undefined, and out == residual_out is rejected.
 * Range: the sum of squares accumulates in float32, as in the page's
 * listing.  So the tolerances hold while h^2 stays a float32 value
 * (|h| below about 1.8e19), and while the mean square does not underflow
 * where eps is 0.  Rows outside that range give zeros or infinities.
 */
rn_status rmsnorm_fwd(const void* x, const void* residual, const void* weight, void* out,
                      void* residual_out, void* out_scale, int64_t rows, int64_t hidden, float eps,
                      uint32_t flags, void* stream);

/* As rmsnorm_fwd; for a quantized output, out_amax (may be NULL) also receives
 * the float32 amax from which each scale was computed (one per row, group or
 * block, laid out like the scales).  out_amax must be NULL for other outputs.
 * tensor_scale: RN_SCALE_NV16 only (else NULL), a device pointer to one
 * float32, the per-tensor scale s_t, read by the kernel (4-byte aligned; it
 * should be positive and finite: other values give unspecified codes). */
rn_status rmsnorm_fwd_ex(const void* x, const void* residual, const void* weight, void* out,
                         void* residual_out, void* out_scale, float* out_amax, const float* tensor_scale,
                         int64_t rows, int64_t hidden, float eps, uint32_t flags, void* stream);

/*
 * One rmsnorm_fwd_ex call described by a record, for the decode path of
 * "Prefill & decode specialization" (a call whose cost should stay near that
 * of a bare launch): a caller that issues the same call many times (a serving
 * loop outside graph capture) fills the record once and passes its address,
 * one argument to marshal per call instead of thirteen.  Each field means
 * what the rmsnorm_fwd_ex argument of the same name means, with the same
 * checks and errors; the library reads the record during the call only and
 * keeps no pointer to it.  call == NULL gives RN_ERR_INVALID_ARG.
 */
typedef struct rn_rmsnorm_call {
  const void* x;
  const void* residual;
  const void* weight;
  void* out;
  void* residual_out;
  void* out_scale;
  float* out_amax;
  const float* tensor_scale;
  int64_t rows;
  int64_t hidden;
  float eps;
  uint32_t flags;
  void* stream;
} rn_rmsnorm_call;

rn_status rmsnorm_fwd_call(const rn_rmsnorm_call* call);

/* As rmsnorm_fwd_ex, with an explicit launch configuration instead of the
 * selector's (for tuning and for testing every kernel variant).  The launch
 * shape is the set of knobs the "Prefill & decode specialization" section of
 * "CuTeDSL at Perplexity" varies (vector width, warps per block, one row per
 * block or per warp); this entry point fixes them by hand.  cfg->kernel
 * must be RN_KERNEL_ROWS; waves_per_row in 1..16, vecs_per_lane in {1,2,4,8},
 * 64 * waves_per_row * vecs_per_lane * vec >= hidden, 1 <= grid <= rows;
 * block_threads, lanes_per_row and rows_per_lane are derived and ignored. */
rn_status rmsnorm_fwd_config(const void* x, const void* residual, const void* weight, void* out,
                             void* residual_out, void* out_scale, float* out_amax,
                             const float* tensor_scale, int64_t rows, int64_t hidden, float eps,
                             uint32_t flags, const rn_launch_config* cfg, void* stream);

/*
 * Fused sum of partial inputs + residual add + RMSNorm over rows.
 *
 * x is not given whole but as num_partials tensors whose elementwise sum it
 * is: the per-rank partial outputs of a row-parallel (tensor-parallel)
 * projection, which an all-reduce or reduce-scatter sums in front of the
 * norm, or the attention and MLP branch outputs of a parallel residual
 * block.  The "CuTeDSL at Perplexity" page fuses a local summation kernel
 * with the all-reduce that follows it into one decode launch (MoE
 * dispatch/combine, single-node tensor-parallel part) and names the fusion
 * of inter-device communication with normalization as what comes next
 * (Conclusion).  This entry point is that fusion's arithmetic on one GPU:
 * the partials are device pointers (local buffers, or peer buffers the
 * caller has mapped); the library does no communication itself.
 *
 *   partials      HOST array of num_partials device pointers, each [rows, hidden] of
 *                 dtype flags.x, 16-byte aligned, none NULL (when rows > 0)      (read)
 *   num_partials  1..8
 *   residual, weight, out, residual_out, out_scale, out_amax, tensor_scale, rows, eps,
 *   flags: as rmsnorm_fwd_ex (every output type and scale granularity);
 *   hidden        as rmsnorm_fwd, and at most 2048 lane vectors (16384 bf16 / 8192 f32
 *                 elements) when num_partials > 1
 *
 * Reading (not on the pages): x is the exact sum of the partials.  With a
 * residual, h = round_res(p_0 + ... + p_{n-1} + residual) is the exact sum of
 * all the terms rounded once (to nearest even) to the residual dtype and
 * written to residual_out; without one, h is the exact sum rounded once to
 * float32.  The norm and the output are those of rmsnorm_fwd over h, so the
 * result does not depend on the order of the partials.  The kernel sums with
 * error-free float32 additions (TwoSum) whose rounding errors it keeps in a
 * double, then rounds once through round-to-odd; this is the exact sum
 * whenever the largest running sum is below 2^74 times the last significant
 * bit of the smallest nonzero term -- for bf16 terms, any terms within 2^63
 * of one another in magnitude, for float32 terms within 2^47 -- and the
 * running sums stay below float32's largest value.  Outside that range the
 * sum can be off in its last bit.
 * num_partials == 1 is rmsnorm_fwd_ex on x = partials[0].
 * Aliasing: out may equal one of the partials (in place) when out has the
 * partials' element width (else RN_ERR_INVALID_ARG); residual_out may equal
 * residual; residual_out equal to a partial or to out is rejected; any other
 * overlap is undefined.
 */
rn_status rmsnorm_fwd_partials(const void* const* partials, int32_t num_partials, const void* residual,
                               const void* weight, void* out, void* residual_out, void* out_scale,
                               float* out_amax, const float* tensor_scale, int64_t rows, int64_t hidden, float eps,
                               uint32_t flags, void* stream);

/* As rmsnorm_fwd_partials with an explicit launch configuration (the rules of
 * rmsnorm_fwd_config, whose launch shape follows "Prefill & decode
 * specialization"; vecs_per_lane at most 2 when num_partials > 1). */
rn_status rmsnorm_fwd_partials_config(const void* const* partials, int32_t num_partials, const void* residual,
                                      const void* weight, void* out, void* residual_out, void* out_scale,
                                      float* out_amax, const float* tensor_scale, int64_t rows, int64_t hidden,
                                      float eps, uint32_t flags, const rn_launch_config* cfg, void* stream);

/*
 * Per-head RMSNorm of Q and K ("CuTeDSL at Perplexity", section "QK Norm").
 *
 *   q          [tokens, num_q_heads, head_dim], token stride q_token_stride elements
 *   k          [tokens, num_k_heads, head_dim] or NULL when num_k_heads == 0
 *   q_weight   [head_dim], k_weight [head_dim] (k_weight NULL iff k is NULL)
 *   q_out      same layout (token stride) as q; may equal q (in place, the page's form)
 *   k_out      same layout as k; may equal k; NULL iff k is NULL
 *   tokens     >= 0; num_q_heads >= 1; num_k_heads >= 0;
 *              tokens * (num_q_heads + num_k_heads) < 2^31
 *   head_dim   64, 128 or 256
 *   *_token_stride  elements between consecutive tokens; 0 means contiguous
 *              (heads * head_dim); otherwise >= heads * head_dim and 16-byte aligned
 *   flags      bits 0-1: dtype of q, k and outputs (bf16 or f32); bits 4-5:
 *              weight dtype (bf16 or f32); bit 8: weight form (1 + w)
 */
rn_status qknorm_fwd(const void* q, const void* k, const void* q_weight, const void* k_weight,
                     void* q_out, void* k_out, int64_t tokens, int32_t num_q_heads,
                     int32_t num_k_heads, int32_t head_dim, int64_t q_token_stride,
                     int64_t k_token_stride, float eps, uint32_t flags, void* stream);

/* As qknorm_fwd, with an explicit launch configuration (for tuning and for
 * testing every variant).  The "QK Norm" section sizes its kernel by head_dim
 * (threads per head, heads per block); "Prefill & decode specialization"
 * describes the same kind of shape choice for the row norms.  Here
 * cfg->kernel must be RN_KERNEL_HEADS, rows_per_lane
 * 1, 2 or 4, block_threads 64, 128 or 256; the grid is derived from those and
 * cfg's other fields are ignored. */
rn_status qknorm_fwd_config(const void* q, const void* k, const void* q_weight, const void* k_weight,
                            void* q_out, void* k_out, int64_t tokens, int32_t num_q_heads,
                            int32_t num_k_heads, int32_t head_dim, int64_t q_token_stride,
                            int64_t k_token_stride, float eps, uint32_t flags,
                            const rn_launch_config* cfg, void* stream);

/*
 * SiLU-and-mul (SwiGLU) over rows: out[r, i] = silu(x[r, i]) * x[r, d + i],
 * silu(g) = g / (1 + exp(-g)), in float32.  The gated activation of the MLP:
 * the "Tile-Level Activation Overlap for Efficient LLM Inference" summary
 * describes the SwiGLU step as the combination of the gate and up projections,
 * and "CuTeDSL at Perplexity" ("Inference at Perplexity") lists activation
 * kernels in the same library.  Reading: each row of x is a merged gate/up
 * projection, gate in its first half and up in its second half.
 *
 *   x          [rows, 2 d] of dtype flags.x (bf16 or f32)           (read)
 *   out        [rows, d] of dtype flags.out (bf16, f32, fp8; fp4: d / 2 bytes per row) (write)
 *   out_scale  quantized output only, laid out as for rmsnorm_fwd    (write)
 *   out_amax   quantized output only, may be NULL                    (write)
 *   tensor_scale  RN_SCALE_NV16 only (else NULL): device float32 s_t, as for rmsnorm_fwd_ex
 *   rows >= 0; d >= 1, a multiple of the 16-byte vector of x and at most 32768 (bf16) /
 *   16384 (f32); flags: bits 0-1 x dtype, bits 6-7 out dtype, bits 9-10 scale granularity
 *   (as for rmsnorm_fwd); other bits must be zero.  out may not overlap x.
 *
 * Range: the results hold the outputs' tolerances while |gate * up| is below
 * float32's largest value (about 3.4e38).  Past it, outputs of a negative gate
 * become -inf or NaN even where silu(gate) * up is finite, because the product
 * gate * up is formed first.  Below gate = -87.3 the factor 1 / (1 + exp(-gate))
 * (bf16 / fp8 / fp4 outputs) or exp(-|gate|) (f32 outputs) is a float32
 * subnormal and carries fewer bits, and for bf16 / fp8 / fp4 outputs it is
 * zero below gate = -103; this shows only where the result is still a normal
 * number (|up| above about 1e35).  Activations are many orders of magnitude
 * inside these limits.
 */
rn_status silu_mul_fwd(const void* x, void* out, void* out_scale, float* out_amax, const float* tensor_scale,
                       int64_t rows, int64_t d, uint32_t flags, void* stream);

/* As silu_mul_fwd with an explicit launch configuration (as rmsnorm_fwd_config;
 * the launch shapes of "Prefill & decode specialization" applied to the
 * activation rows). */
rn_status silu_mul_fwd_config(const void* x, void* out, void* out_scale, float* out_amax,
                              const float* tensor_scale, int64_t rows, int64_t d, uint32_t flags,
                              const rn_launch_config* cfg, void* stream);

/* Host-only: the launch configuration silu_mul_fwd would use: the selector of
 * rmsnorm_query_config (below) applied to the activation rows, with its own
 * measured table. */
rn_status silu_mul_query_config(int64_t rows, int64_t d, uint32_t flags, int32_t num_cus,
                                rn_launch_config* cfg);

/* Host-only: the launch configuration rmsnorm_fwd would use for these sizes on
 * a device with num_cus compute units (num_cus <= 0: query the current device);
 * has_residual says whether the call passes a residual (its dtype bits are then
 * read from flags).  This is the selector of "Prefill & decode specialization"
 * ("CuTeDSL at Perplexity"): the widest vector per lane first, then the warps
 * per row, a decode shape with one warp per row when the rows are few, and a
 * cap on warps per block that the page benchmarks; the compute-unit count
 * plays the part of the SM count that, per "Blackwell support", the host-side
 * launcher knows and sizes the grid by. */
rn_status rmsnorm_query_config(int64_t rows, int64_t hidden, uint32_t flags, int32_t has_residual,
                               int32_t num_cus, rn_launch_config* cfg);

/* The launch configuration rmsnorm_fwd_partials would use (host only when
 * num_cus > 0): the selector of rmsnorm_query_config ("Prefill & decode
 * specialization"; the compute-unit count as in "Blackwell support") for the
 * partial-input kernels, with its own measured table. */
rn_status rmsnorm_partials_query_config(int64_t rows, int64_t hidden, int32_t num_partials, uint32_t flags,
                                        int32_t has_residual, int32_t num_cus, rn_launch_config* cfg);

/* Host-only: the launch configuration qknorm_fwd would use: lanes per head
 * from head_dim as in the "QK Norm" section's kernel, heads per lane group and
 * the grid from the token count against the compute units, following the
 * shape selection of "Prefill & decode specialization" (the host knows the
 * compute-unit count, as the SM count in "Blackwell support"). */
rn_status qknorm_query_config(int64_t tokens, int32_t num_q_heads, int32_t num_k_heads,
                              int32_t head_dim, uint32_t flags, int32_t num_cus,
                              rn_launch_config* cfg);

/* Enqueues one wave64 of a kernel that does nothing, through the same launch
 * path as the entry points above: the reference for bare kernel-launch latency
 * when decode-sized calls are timed. */
rn_status rn_launch_empty(void* stream);

/* Enqueues a plain streaming copy of `bytes` bytes from src to dst (device
 * memory, 16-byte aligned, not overlapping; bytes a multiple of 16): one
 * nontemporal 16-byte load and store per lane, 8 KiB per workgroup.  The
 * practical bandwidth ceiling for a stream that reads and writes the same
 * number of bytes, measured through the same launch path as the entry points
 * above.  bytes == 0 is a no-op. */
rn_status rn_launch_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Static description of a status code. */
const char* rn_status_string(rn_status status);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* rn_last_error(void);

/* RN_ABI_VERSION of the built library. */
int32_t rn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_ROWS_H */
