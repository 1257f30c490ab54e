/*
 * joint_attn.h - C ABI of the MI355X (gfx950) joint text+image attention
 * forward library, libjoint_attn.so.
 *
 * The operation is the joint attention of a DiT block: text tokens, noisy
 * target-image latent tokens and optional reference-image tokens form ONE
 * sequence and every query attends to every key of it, with no mask
 * ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA Blackwell
 * GPUs", section "FLUX 3 inference with TensorRT LLM VisualGen").  Q and K
 * carry rotary position embeddings applied where they are produced (same
 * page, section "GEMM kernel optimization"), here fused into the attention's
 * Q/K load; the FP8 path quantizes Q, K and V to FP8 (same page, section
 * "Quantized and sparse attention", qk_dtype / v_dtype fp8).
 *
 *   O[b,i,h,:] = sum_j softmax_j( <R_i q[b,i,h], R_j k[b,j,h]> * scale ) v[b,j,h,:]
 *
 * with R_t the rotation of token t (a 2x2 rotation of every adjacent pair
 * (2p, 2p+1) of the head vector by the angle whose cos/sin the RoPE table
 * holds) and scale = 1/sqrt(D) unless given.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device.
 *     The caller allocates and owns every buffer, workspaces included; the
 *     library allocates no device or host memory and keeps no per-call
 *     state.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work: they return after the launch, inputs must stay unchanged
 *     and outputs unread until the stream reaches the call.  Calls are
 *     thread-safe.
 *   - Validation happens on the host before anything is enqueued; on any
 *     error nothing is launched and no output is written.  Faults inside a
 *     kernel are asynchronous and surface at the caller's next
 *     synchronisation of the stream.
 *   - bf16 is bfloat16 (1-8-7, round to nearest even); e4m3 is the OCP 8-bit
 *     floating point E4M3 format (bias 7, no infinities, max 448).
 */
#ifndef JOINT_ATTN_H
#define JOINT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  JA_OK = 0,
  JA_ERR_INVALID_ARG = 1,  /* null pointer, size < 1, bad stride or alignment */
  JA_ERR_UNSUPPORTED = 2,  /* head_dim not 64 or 128, grid too large          */
  JA_ERR_HIP = 3           /* the HIP runtime refused the launch               */
} ja_status;

/*
 * Shape and layout of one attention call.
 *   batch, seq_len, heads >= 1; head_dim in {64, 128}.
 *   Q/K/V/O are addressed as x[b*x_sb + s*x_ss + h*x_sh + d] (strides in
 *   ELEMENTS, the D stride is 1).  A contiguous [B, S, H, D] tensor has
 *   x_ss = H*D, x_sh = D, x_sb = S*H*D; [B, H, S, D] works too.  Strides must
 *   be multiples of 8 and base pointers 16-byte aligned (16-byte vector
 *   loads).  softmax_scale = 0 selects 1/sqrt(head_dim).
 *
 *   q_norm, k_norm, norm_eps: optional query/key RMS normalization (the
 *   pages fuse "query/key normalization" with RoPE into the QKV epilogue,
 *   section "GEMM kernel optimization").  q_norm / k_norm are device fp32
 *   weights [head_dim] (16-byte aligned), shared by all heads; NULL = that
 *   tensor is not normalized.  Each (batch, token, head) vector x becomes
 *     y_d = fl(fl(x_d * r) * g_d),  r = 1 / sqrt(ss / head_dim + eps)
 *   in fp32 (IEEE square root and division), before RoPE and with no rounding
 *   of its own; ss, the sum of squares, is taken chunk by chunk (8 elements,
 *   fma in element order) and then pairwise over chunk c and c ^ k for
 *   k = 2, 4, ..., head_dim/16, then k = 1.  norm_eps = 0 selects 1e-6.  The
 *   normalization happens wherever RoPE is applied: the Q load of the bf16
 *   forwards, joint_attn_prep_kv_bf16 (K), joint_attn_quant_rope_fp8 (Q, K)
 *   and joint_attn_fp8_repair_plan (K).  Zero-initialize the struct to get
 *   no normalization.
 */
typedef struct {
  int32_t batch, seq_len, heads, head_dim;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  float softmax_scale;
  const float *q_norm, *k_norm;
  float norm_eps;
} ja_params;

/*
 * joint_attn_rope_table_2d - cos/sin of every rotation angle of 2D-axial
 * RoPE (the position encoding of the image latent grid; the pages fuse RoPE
 * into the QKV epilogue, section "GEMM kernel optimization").
 *   pos    device int32 [seq_len][2]: (row, col) grid position of each token
 *          (text tokens conventionally at (0, 0)); any int32 values.
 *   table  device float [seq_len][head_dim/2][2]: written with
 *          (cos a, sin a) of pair p's angle a, computed in fp64 and rounded
 *          once to fp32.  Pair p < head_dim/4 rotates by the row with
 *          frequency w_p; pair p >= head_dim/4 by the column with w_(p-D/4);
 *          w_k = theta^(-4k/head_dim) (the 1-D RoPE of dimension D/2 on each
 *          axis).
 *   theta  > 0 (10000 in the FLUX-style DiT).
 * The table depends only on positions, head_dim and theta: build it once per
 * forward pass and pass it to every layer's attention call.
 */
ja_status joint_attn_rope_table_2d(const int32_t *pos, int32_t seq_len,
                                   int32_t head_dim, float theta, float *table,
                                   void *stream);

/*
 * joint_attn_prep_kv_bf16 - K/V preparation of the BF16 forward: RoPE fused
 * into the single load of K (same page, section "GEMM kernel optimization",
 * where RoPE is fused into the epilogue that produces K), V transposed.
 *   k, v     device bf16, layout per ja_params (its K and V strides).
 *   rope     as for joint_attn_fwd_bf16 (NULL = no rotation).  K is rotated
 *            in fp32, pair (x, y) -> (fma(x, c, -fl(y s)), fma(x, s, fl(y c))),
 *            and rounded to bf16.
 *   kv       device buffer (16-byte aligned) of kv_bytes >=
 *            joint_attn_prep_kv_bf16_bytes(p), written with
 *              Kr [batch*heads][S_pad][head_dim]  rotated K,
 *              Vt [batch*heads][head_dim][S_pad]  V transposed, the keys of
 *                   every 16-key group in the order p -> 4*(p/8) + (p%8 < 4 ?
 *                   p%8 : p%8 + 4) (the P operand order of the forward),
 *            S_pad = seq_len rounded up to 64, zeros past seq_len.
 * The buffer depends only on K, V and the table: when several calls share
 * them, prepare once.
 */
size_t joint_attn_prep_kv_bf16_bytes(const ja_params *p);
ja_status joint_attn_prep_kv_bf16(const ja_params *p, const void *k, const void *v,
                                  const float *rope, void *kv, size_t kv_bytes, void *stream);

/*
 * joint_attn_fwd_bf16 - BF16 joint attention on K/V prepared by
 * joint_attn_prep_kv_bf16 (with the same p and rope), with RoPE fused into
 * the load of Q.
 *   q        device bf16, layout per ja_params.
 *   kv, kv_bytes  the prepared K/V buffer.
 *   rope     the table the K/V were prepared with (NULL = no rotation); Q is
 *            rotated as K was and rounded to bf16 before Q K^T.
 *   o        device bf16, layout per ja_params (o_* strides); must not alias
 *            q or kv.
 *   lse      device float [batch][heads][seq_len], nullable: natural-log
 *            log-sum-exp of each query row's scaled scores.
 *   workspace, workspace_bytes
 *            optional device scratch (16-byte aligned) of at least
 *            joint_attn_fwd_bf16_workspace_bytes(p) bytes.  With it, the
 *            work items of a last, mostly idle round of workgroups are split
 *            over key ranges and merged exactly (same softmax rescaling as
 *            between key tiles), which shortens that round; NULL or too
 *            small = no split.  The scratch must not be used by another call
 *            that runs concurrently; its contents on return are undefined.
 * Softmax statistics and both products accumulate in fp32; P is rounded to
 * bf16 for the P.V product.
 */
ja_status joint_attn_fwd_bf16(const ja_params *p, const void *q, const void *kv,
                              size_t kv_bytes, const float *rope, void *o, float *lse,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * joint_attn_fwd_bf16_workspace_bytes - bytes of the optional workspace of
 * joint_attn_fwd_bf16 (and joint_attn_fwd_bf16_block_sparse) for this shape
 * on the current device (0: no split helps, or p is invalid).  Host-only;
 * launches nothing.
 */
size_t joint_attn_fwd_bf16_workspace_bytes(const ja_params *p);

/* Block granularity of joint_attn_fwd_bf16_block_sparse's mask. */
#define JA_SPARSE_QUERY_BLOCK 128
#define JA_SPARSE_KEY_BLOCK 64

/*
 * joint_attn_fwd_bf16_block_sparse - joint_attn_fwd_bf16 restricted to the
 * blocks of a given block mask: the kernel half of the pages' block-sparse
 * attention (section "Quantized and sparse attention": Sol-Attention runs on
 * a general block-sparse attention kernel; how it chooses the blocks is not
 * on the pages, so the mask is an input).
 *   block_mask  device uint8 [batch][heads][nqb][nkb], contiguous, with
 *               nqb = ceil(seq_len / JA_SPARSE_QUERY_BLOCK) and
 *               nkb = ceil(seq_len / JA_SPARSE_KEY_BLOCK); nonzero = keep.
 *               Query i attends key j iff
 *               block_mask[b][h][i / JA_SPARSE_QUERY_BLOCK][j / JA_SPARSE_KEY_BLOCK]
 *               is nonzero, and its softmax runs over those keys only.  A
 *               query row that keeps no key gets O = 0 and LSE = -inf.
 *   Every other argument, the arithmetic and the workspace (same size,
 *   joint_attn_fwd_bf16_workspace_bytes) are those of joint_attn_fwd_bf16;
 *   an all-nonzero mask gives the same result as joint_attn_fwd_bf16.
 *   seq_len up to 1048576 (JA_ERR_UNSUPPORTED above).  Work and time scale
 *   with the key blocks kept by any of the three consecutive query blocks
 *   that one workgroup covers.
 */
ja_status joint_attn_fwd_bf16_block_sparse(const ja_params *p, const void *q, const void *kv,
                                           size_t kv_bytes, const float *rope,
                                           const uint8_t *block_mask, void *o, float *lse,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream);

/*
 * joint_attn_quant_rope_fp8 - RoPE on Q and K, then per-token FP8
 * quantization of Q, K and V (the pages' fp8 qk_dtype / v_dtype).
 *   q, k, v     device bf16, layout per ja_params (its Q, K, V strides).
 *   rope        as for joint_attn_fwd_bf16 (NULL = no rotation).
 *   q8, k8, v8  device e4m3 (1 byte each), written contiguous
 *               [batch][seq_len][heads][head_dim].
 *   sq, sk, sv  device float [batch][heads][seq_len]: one scale per (b, token,
 *               head).  For each head vector x (after RoPE, computed in fp32
 *               as (fma(x, c, -fl(y s)), fma(x, s, fl(y c)))): amax = max|x|;
 *               Q and K: scale = the smallest power of two s with
 *               amax <= 448 s, at least 2^-126 (an E8M0 exponent);
 *               V: scale = amax/448; all three: 1 if amax = 0;
 *               code = e4m3_rne(clamp(fl(x/scale), -448, 448)).
 */
ja_status joint_attn_quant_rope_fp8(const ja_params *p, const void *q,
                                    const void *k, const void *v,
                                    const float *rope, void *q8, void *k8,
                                    void *v8, float *sq, float *sk, float *sv,
                                    void *stream);

/*
 * Repair of the FP8 path (the pages' VC-Attention FP8 with vc_repair_budget:
 * the fraction of tokens with the highest quantization error gets a residual
 * correction; section "Quantized and sparse attention").  Reading: per
 * (batch, head), token t's error is e = max_d |k - k^| + max_d |v - v^| in
 * fp32 (k the rotated key that was quantized, k^ = fl(value(code) * scale));
 * the n_rep tokens with the largest e (ties to the lower index) are repaired:
 * their key and value enter attention at bf16-path precision.
 *
 * joint_attn_fp8_repair_plan - selects the repaired tokens and gathers them.
 *   p           shape and the K/V strides of k and v (Q and O strides unused).
 *   k, v, rope  as for joint_attn_quant_rope_fp8.
 *   k8, v8, sk, sv   that call's outputs.
 *   n_rep       0 <= n_rep <= seq_len (ceil(budget * seq_len) for a budget).
 *   idx         device int32 [batch][heads][n_rep]: written with the repaired
 *               token indices, ascending (may be NULL when n_rep = 0).
 *   kr, vr      device bf16 [batch][heads][n_pad][head_dim], n_pad = n_rep
 *               rounded up to a multiple of 32: the rotated keys (rotation
 *               and bf16 rounding as in joint_attn_fwd_bf16) and the values of
 *               the repaired tokens; rows n_rep .. n_pad-1 are zero.
 *   kbias       device float [batch][heads][seq_len]: 0, or -inf for a
 *               repaired token.
 * seq_len is limited to 39936 (the selection keeps a row's errors in LDS);
 * larger: JA_ERR_UNSUPPORTED.
 */
ja_status joint_attn_fp8_repair_plan(const ja_params *p, const void *k, const void *v,
                                     const float *rope, const void *k8, const void *v8,
                                     const float *sk, const float *sv, int32_t n_rep,
                                     int32_t *idx, void *kr, void *vr, float *kbias,
                                     void *stream);

/* The repair set passed to joint_attn_fwd_fp8 (n_rep = 0: none). */
typedef struct {
  int32_t n_rep;
  const float *kbias;   /* [batch][heads][seq_len], 16-byte aligned */
  const void *kr, *vr;  /* [batch][heads][n_pad][head_dim] bf16 */
} ja_fp8_repair;

/*
 * joint_attn_prep_kv_fp8_bytes - bytes of the prepared K/V buffer of the FP8
 * forward for this shape (0 if p is invalid).  Host-only.
 */
size_t joint_attn_prep_kv_fp8_bytes(const ja_params *p);

/*
 * joint_attn_prep_kv_fp8 - K/V preparation of the FP8 forward: the e4m3 keys
 * and values of each (batch, head) laid out as the forward's LDS tiles, with
 * the per-key values of its softmax.  One pass over K and V.
 *   p           shape and softmax_scale (the forward must use the same); the
 *               Q, K, V and O strides are unused.
 *   k8, v8, sk, sv   joint_attn_quant_rope_fp8's outputs: e4m3 codes
 *               contiguous [batch][seq_len][heads][head_dim], 16-byte aligned;
 *               fp32 scales [batch][heads][seq_len].  sk must hold positive
 *               normal powers of two (the quantizer's K scales), sv positive
 *               finite values; a key that breaks this turns every row of its
 *               (batch, head) into NaN in the forward.
 *   repair      nullable; with n_rep > 0 its kbias (0, or -inf for a
 *               repaired key, from joint_attn_fp8_repair_plan) removes the
 *               repaired keys from the FP8 tiles.
 *   kv8, kv8_bytes   device output of at least
 *               joint_attn_prep_kv_fp8_bytes(p) bytes, 16-byte aligned:
 *               K [B*H][S_pad][D], then V^T [B*H][D][S_pad] (keys of each
 *               64-key tile in the order in which the forward's P' operand
 *               holds them), then [B*H][S_pad/64] blocks of 256 words per
 *               tile: log2(sv)/c (+ kbias; -inf past the end), 1/sv (0 past
 *               the end), the E8M0 exponent of sk (127 past the end), c; with
 *               S_pad = seq_len rounded up to 64, c the softmax scale times
 *               log2(e), rows past the end zero.
 * Same size limits as joint_attn_fwd_fp8.
 */
ja_status joint_attn_prep_kv_fp8(const ja_params *p, const void *k8, const void *v8,
                                 const float *sk, const float *sv, const ja_fp8_repair *repair,
                                 void *kv8, size_t kv8_bytes, void *stream);

/*
 * joint_attn_fwd_fp8 - joint attention on FP8 inputs produced by
 * joint_attn_quant_rope_fp8 (RoPE already applied), with K and V prepared
 * by joint_attn_prep_kv_fp8.
 *   q8          device e4m3, contiguous [batch][seq_len][heads][head_dim]
 *               (the Q, K and V strides of p are ignored), 16-byte aligned.
 *   sq          device float [batch][heads][seq_len]: Q's dequantization
 *               scales, positive normal powers of two (the quantizer's);
 *               their exponents are the E8M0 block scales of the Q K^T MFMA.
 *               A workgroup that meets another value writes NaN into its O
 *               rows and LSE entries (its 384-row query block).
 *   kv8, kv8_bytes   the prepared K/V buffer.  If it was prepared for another
 *               softmax scale, every row comes back NaN.
 *   repair      nullable: with n_rep > 0, the repaired tokens from
 *               joint_attn_fp8_repair_plan (kr, vr; kbias went to the
 *               preparation), attended from their bf16 values in the same
 *               softmax.
 *   o           device bf16, layout per ja_params (o_* strides).
 *   lse         device float [batch][heads][seq_len], nullable.
 *   workspace, workspace_bytes
 *               optional scratch of joint_attn_fwd_fp8_workspace_bytes(p)
 *               bytes, as for joint_attn_fwd_bf16.
 * Q K^T and P.V run on FP8 MFMA, Q K^T with the Q and K scales as E8M0
 * block scales.  V's per-key scale is folded into the probabilities before
 * they are rounded to e4m3 for P.V: each score accumulator starts at
 * log2(sv[key]) / c (c the softmax scale in the exp2 domain), so that
 * P' = exp2(c acc - ref) = P * sv[key], with the reference ref kept 5 below
 * the running row max (P' < 2^8).  Softmax statistics and accumulation are
 * fp32; the output is bf16.  The size of one (batch, head)'s prepared K or V
 * (S_pad * head_dim bytes) must stay below 2^31: JA_ERR_UNSUPPORTED.
 */
ja_status joint_attn_fwd_fp8(const ja_params *p, const void *q8, const float *sq,
                             const void *kv8, size_t kv8_bytes, const ja_fp8_repair *repair,
                             void *o, float *lse, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * joint_attn_fwd_fp8_workspace_bytes - bytes of the optional workspace of
 * joint_attn_fwd_fp8 for this shape on the current device (0: no split
 * helps, or p is invalid).  Host-only; launches nothing.
 */
size_t joint_attn_fwd_fp8_workspace_bytes(const ja_params *p);

/* Human-readable name of a status code (static string, never NULL). */
const char *joint_attn_status_string(ja_status s);

/* Message of the last HIP error seen by this thread's library calls
 * (static per-thread buffer; "" if none). */
const char *joint_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JOINT_ATTN_H */
