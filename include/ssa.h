/*
 * ssa.h -- C ABI of the MI355X (gfx950) spatial self-attention block.
 *
 * The operation (tensortonic problem "Spatial Self-Attention", diffusion
 * L03: the formula, the prose under it and the parameter table):
 *
 *     Z   = tokens(GN(x))                     GN: num_groups groups, eps 1e-5,
 *                                                 affine norm_weight/norm_bias
 *     Q   = Z Wq^T + bq,  K = Z Wk^T + bk,  V = Z Wv^T + bv
 *     O_j = softmax(Q_j K_j^T / sqrt(d)) V_j  head j = channels j*d..(j+1)*d-1,
 *                                             d = C / num_heads, softmax over keys
 *     out = x + image([O_1 .. O_n] Wo^T + bo)
 *
 * tokens() maps pixel (i, j) of each sample to token row i*W + j; image() is
 * its inverse.  Weights are (C, C) stored (out, in) row-major, "as in a linear
 * layer"; biases and the GroupNorm affine are (C,).
 *
 * Conventions for every entry point below
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers to contiguous row-major memory of
 *   the element type `dtype` (x, out and all ten parameters share it):
 *     x, out                          (B, C, H, W)   NCHW
 *     norm_weight, norm_bias          (C,)
 *     q_weight, k_weight, v_weight,
 *     out_weight                      (C, C)         (out, in)
 *     q_bias, k_bias, v_bias, out_bias (C,)
 *   Every pointer must be 16-byte aligned.
 * - Biases are nullable: a NULL q_bias, k_bias, v_bias or out_bias is a
 *   projection without a bias (the HNDL attention operator's qkv_bias /
 *   out_bias flags: "a projection built without a bias has no bias
 *   parameter").  Every other data pointer is required.
 * - The caller owns every buffer, including `workspace`.  The library
 *   allocates no device memory and keeps no state between calls; calls on
 *   different streams with different workspaces may run concurrently.
 * - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *   asynchronously; completion is observed through the stream.
 * - Arguments are validated on the host before anything is enqueued.  On any
 *   error nothing is launched and nothing is written.
 * - B == 0, H == 0 or W == 0 is an empty input: SSA_OK, nothing launched, and
 *   the data pointers may be NULL.
 * - Supported: fp32 and bf16 (fp32 accumulation) with 1 <= d <= 128.  A
 *   head size above 128 returns SSA_E_UNSUPPORTED, and so does a call with
 *   3*B*H*W*C >= 2^31 (the Q|K|V projection's output must stay below 2^31
 *   elements; every tensor then fits 32-bit offsets).  bf16 heads narrower
 *   than a multiple of 32 are zero-padded to the next one (dp below), which
 *   leaves every score and output unchanged.
 *
 * Workspace (bytes from ssa_workspace_size; regions from
 * ssa_get_workspace_layout, each 256-byte aligned):
 *   gn_partial  float4 (count, mean, M2, 0) per (b, g, split)
 *   gn_stats    float2 (mean, rstd) per (b, g)
 *   gn_coef     float2 (a, s) per (b, c): GN(x)[b,c,t] = a*x[b,c,t] + s
 *   q, k        (B, n, T, dp)  dtype, token-major per head; dp = d for fp32,
 *                              d rounded up to a multiple of 32 for bf16, the
 *                              columns d .. dp-1 zero; bf16 q holds
 *                              Q * log2(e) / sqrt(d) (the score scale; with
 *                              query/key normalisation Q * log2(e))
 *   vt          (B, n, dp, Tp) dtype, V transposed, Tp = T rounded up to 64;
 *                              fp32: token t in column t; bf16: token t in
 *                              column t with bits 2 and 3 swapped (the order of
 *                              the attention kernel's MFMA operand); columns of
 *                              tokens >= T and rows d .. dp-1 are never written
 *   o           (B, T, C)      dtype, heads concatenated along channels
 *   rope        (T, d/2) float2 (cos, sin) of the rotary angles (bf16 with
 *                              d in {16, 32, 64, 128} and the projection's main
 *                              path: C % 64 == 0, T % 4 == 0); else empty
 *   qk32        (2, B, n, T, d) fp32 Q and K before the optional steps (bf16
 *                              problems without the rope region); else empty
 *   attn_part   fp32 partial attention results (O, running max, row sums) of
 *                              the query tiles whose keys are split over several
 *                              work-groups (bf16, d in 33..64, T >= 1024 with T
 *                              % 128 == 0, when the 256-query tiles leave a
 *                              partial last round of at most half the compute
 *                              units); else empty
 * After ssa_forward these hold the block's intermediates for inspection.
 */
#ifndef SSA_H_
#define SSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSA_OK = 0,
  SSA_E_NULL = 1,         /* a required pointer is NULL (biases may be NULL)   */
  SSA_E_SHAPE = 2,        /* a size is negative, or C < 1                       */
  SSA_E_CONSTRAINT = 3,   /* num_groups or num_heads < 1 or does not divide C   */
  SSA_E_DTYPE = 4,        /* unknown dtype code                                 */
  SSA_E_UNSUPPORTED = 5,  /* head size or total size outside the supported set  */
  SSA_E_WORKSPACE = 6,    /* workspace_bytes < ssa_workspace_size(...)          */
  SSA_E_ALIAS = 7,        /* out overlaps an input or the workspace, or the
                             workspace overlaps an input                        */
  SSA_E_ALIGN = 8,        /* a pointer is not 16-byte aligned                   */
  SSA_E_HIP = 9,          /* a HIP launch failed (e.g. no gfx950 code object)   */
  SSA_E_STAGE = 10,       /* unknown stage code                                 */
  SSA_E_SCRATCH = 11      /* ssa_forward_noalloc: workspace above its maximum   */
} ssa_status;

typedef enum { SSA_F32 = 0, SSA_BF16 = 1 } ssa_dtype;

/* The kernels of the block.  ssa_forward runs stages 0, 1, 2, 3 in this
 * order, or 0, 4, 3 where ssa_uses_fused_stage() returns 1 (then q, k and vt
 * of the workspace are not written). */
typedef enum {
  SSA_STAGE_GN_STATS = 0,   /* GroupNorm statistics -> gn_stats, gn_coef        */
  SSA_STAGE_QKV = 1,        /* normalise + Q/K/V projections -> q, k, vt        */
  SSA_STAGE_ATTENTION = 2,  /* per-head softmax(QK^T/sqrt(d))V -> o             */
  SSA_STAGE_OUT_PROJ = 3,   /* o Wo^T + bo + x, back to NCHW -> out             */
  SSA_STAGE_QKV_ATTENTION = 4 /* stages 1 and 2 in one kernel -> o (the same
                                 bits); reads gn_coef, writes only o          */
} ssa_stage;

typedef struct {
  size_t total;        /* bytes, same as ssa_workspace_size                   */
  size_t gn_partial;   /* byte offsets of each region from workspace start    */
  size_t gn_stats;
  size_t gn_coef;
  size_t q;
  size_t k;
  size_t vt;
  size_t o;
  size_t rope;         /* 0 bytes long when absent (offset of the next region) */
  size_t qk32;
  size_t attn_part;
  int64_t gn_splits;   /* splits per (b, g) segment in gn_partial             */
  int64_t t_pad;       /* Tp: row pitch of vt in elements                     */
  int64_t d_pad;       /* dp: row pitch of q and k, rows per head of vt       */
} ssa_workspace_layout;

/* Bytes of workspace ssa_forward needs for this problem, or 0 when the
 * arguments would be rejected (see ssa_status) or the input is empty. */
size_t ssa_workspace_size(int64_t B, int64_t C, int64_t H, int64_t W,
                          int64_t num_groups, int64_t num_heads, int dtype);

/* Fills *layout with the workspace regions for this problem.
 * Returns SSA_E_NULL when layout is NULL, else the status ssa_forward would
 * return for these sizes before looking at pointers. */
ssa_status ssa_get_workspace_layout(int64_t B, int64_t C, int64_t H, int64_t W,
                                    int64_t num_groups, int64_t num_heads, int dtype,
                                    ssa_workspace_layout* layout);

/* The whole block: enqueues the four stages on `stream`.
 * Parameter order follows the problem's parameter table. */
ssa_status ssa_forward(const void* x, void* out,
                       const void* norm_weight, const void* norm_bias,
                       const void* q_weight, const void* k_weight,
                       const void* v_weight, const void* out_weight,
                       const void* q_bias, const void* k_bias,
                       const void* v_bias, const void* out_bias,
                       int64_t B, int64_t C, int64_t H, int64_t W,
                       int64_t num_groups, int64_t num_heads, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* One stage of the block, with the same arguments and validation as
 * ssa_forward.  Running stages 0, 1, 2, 3 (or, where the fused stage is
 * available, 0, 4, 3) in order on one stream with one workspace is exactly
 * ssa_forward; both orders give the same output bit for bit.  A stage reads
 * what the earlier stages left in the workspace; running it out of order
 * computes from whatever the workspace holds (no error is detectable).
 * Stage 4 returns SSA_E_UNSUPPORTED for sizes ssa_uses_fused_stage() rejects.
 * Used to time and inspect each kernel separately. */
ssa_status ssa_forward_stage(int stage,
                             const void* x, void* out,
                             const void* norm_weight, const void* norm_bias,
                             const void* q_weight, const void* k_weight,
                             const void* v_weight, const void* out_weight,
                             const void* q_bias, const void* k_bias,
                             const void* v_bias, const void* out_bias,
                             int64_t B, int64_t C, int64_t H, int64_t W,
                             int64_t num_groups, int64_t num_heads, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Optional steps of ssa_forward_ex, each off when its field is NULL / 0.
 * Order: projections, query/key normalisation, rotary embedding, scaled
 * scores plus the relative-position bias, softmax, P V.
 *
 *  rel_pos_table  ((2H-1)*(2W-1), num_heads), dtype of x: learned 2-D
 *                 relative-position bias added to the scaled logits (HNDL
 *                 attention operator, "Relative position bias"): for query q
 *                 and key k at rows q/W, k/W and columns q%W, k%W,
 *                 bias[head, q, k] = table[(dy)*(2W-1) + dx, head] with
 *                 dy = row(q)-row(k)+H-1, dx = col(q)-col(k)+W-1.
 *  q_norm_gamma,  (num_heads, d) each, dtype of x, both or neither
 *  k_norm_gamma   (SSA_E_CONSTRAINT otherwise): per-head query/key
 *                 normalisation (vit-pytorch simple_vit_with_qk_norm.py,
 *                 RMSNorm): x / max(||x||_2, 1e-12) * sqrt(d) * gamma[head];
 *                 the scores are then not divided by sqrt(d).
 *  rope           nonzero: rotary embeddings over the token index t (HNDL
 *                 attention operator, "Rotary embeddings"): rotate-half over
 *                 the full head, theta_i = 10000^(-2i/d) and angle t*theta_i
 *                 in float32; needs an even d (SSA_E_UNSUPPORTED otherwise).
 * The library reads these tensors during the call's kernels and keeps no
 * reference; they must not overlap out or the workspace (SSA_E_ALIAS). */
typedef struct {
  const void* rel_pos_table;
  const void* q_norm_gamma;
  const void* k_norm_gamma;
  int32_t rope;
} ssa_options;

/* ssa_forward with optional steps (options may be NULL: the plain block).
 * Same workspace, validation and stream semantics as ssa_forward. */
ssa_status ssa_forward_ex(const void* x, void* out,
                          const void* norm_weight, const void* norm_bias,
                          const void* q_weight, const void* k_weight,
                          const void* v_weight, const void* out_weight,
                          const void* q_bias, const void* k_bias,
                          const void* v_bias, const void* out_bias,
                          int64_t B, int64_t C, int64_t H, int64_t W,
                          int64_t num_groups, int64_t num_heads, int dtype,
                          const ssa_options* options,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ssa_forward_stage with optional steps (options may be NULL): one stage of
 * ssa_forward_ex.  Running stages 0, 1, 2, 3 in order on one stream with one
 * workspace and the same options is exactly ssa_forward_ex (which never runs
 * the fused stage 4 while an optional step is on; stage 4 with an optional
 * step on returns SSA_E_UNSUPPORTED).  Used to time and inspect the kernels of
 * the optional steps. */
ssa_status ssa_forward_stage_ex(int stage,
                                const void* x, void* out,
                                const void* norm_weight, const void* norm_bias,
                                const void* q_weight, const void* k_weight,
                                const void* v_weight, const void* out_weight,
                                const void* q_bias, const void* k_bias,
                                const void* v_bias, const void* out_bias,
                                int64_t B, int64_t C, int64_t H, int64_t W,
                                int64_t num_groups, int64_t num_heads, int dtype,
                                const ssa_options* options,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ssa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same block, validation and stream semantics, with the workspace taken from
 * a static array of the library (ssa_noalloc_max_workspace() bytes, 128 MiB,
 * on each GPU the library runs on, held until the process ends) instead of a
 * caller buffer.  It calls no allocating routine.  A problem whose
 * ssa_workspace_size exceeds the maximum returns SSA_E_SCRATCH before
 * anything is launched.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (on different streams, or from different
 * threads) race and may corrupt each other's output; calls ordered on one
 * stream do not.  The array keeps the last call's intermediates (no kernel
 * relies on its previous contents). */
ssa_status ssa_forward_noalloc(const void* x, void* out,
                               const void* norm_weight, const void* norm_bias,
                               const void* q_weight, const void* k_weight,
                               const void* v_weight, const void* out_weight,
                               const void* q_bias, const void* k_bias,
                               const void* v_bias, const void* out_bias,
                               int64_t B, int64_t C, int64_t H, int64_t W,
                               int64_t num_groups, int64_t num_heads, int dtype,
                               void* stream);

/* Bytes of the static scratch of ssa_forward_noalloc (its largest workspace). */
size_t ssa_noalloc_max_workspace(void);

/* 1 when ssa_forward (and ssa_forward_ex with no optional step on) runs the
 * fused stage SSA_STAGE_QKV_ATTENTION for this problem, else 0 (also for
 * arguments ssa_forward would reject).  The fused kernel keeps one head's
 * Q, K and V in the LDS of one compute unit: bf16, head size 128, 192 < H*W
 * <= 256 with H*W a multiple of 4, and at least one (sample, head) pair per
 * compute unit of the current device (tensortonic "Spatial Self-Attention":
 * the projections and the per-head attention of its formula). */
int ssa_uses_fused_stage(int64_t B, int64_t C, int64_t H, int64_t W,
                         int64_t num_groups, int64_t num_heads, int dtype);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* ssa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SSA_H_ */
