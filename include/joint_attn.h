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
 * with R_t the 2D-axial rotation of token t (every adjacent pair (2p, 2p+1)
 * of the head vector turned by an angle of its grid row, p < D/4, or column,
 * p >= D/4) and scale = 1/sqrt(D) unless given.
 *
 * Entry points, from one call per operation to the pieces it is made of:
 *   joint_attn_fwd_bf16               Q, K, V (bf16) and positions -> O
 *   joint_attn_fwd_bf16_block_sparse  the same on the blocks of a block mask
 *   joint_attn_quant_rope_fp8         Q, K, V (bf16) -> e4m3 codes + fp32 scales
 *   joint_attn_fwd_fp8                e4m3 Q, K, V with their scales -> O
 *   joint_attn_fwd_fp8_block_sparse   the same on the blocks of a block mask
 *   joint_attn_fp8_repair_count / _repair_plan   repair of the FP8 path
 *   joint_attn_rope_table_2d, joint_attn_prep_kv_bf16, joint_attn_prep_kv_fp8,
 *   joint_attn_fwd_*_prepared         the two phases of the forwards, for
 *                                     callers that reuse a table or K/V
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
 *   - A call that needs scratch memory takes a workspace (device, 16-byte
 *     aligned) and has a joint_attn_*_workspace_bytes(p) query for its size
 *     (host-only, launches nothing; 0 if p is invalid).  A smaller workspace
 *     than the query's gives JA_ERR_INVALID_ARG.  Its contents on return are
 *     undefined, and two calls that run concurrently must not share one.
 *   - Validation happens on the host before anything is enqueued; on any
 *     error nothing is launched and no output is written, and
 *     joint_attn_last_error() says what was wrong.  Faults inside a kernel
 *     are asynchronous and surface at the caller's next synchronisation of
 *     the stream.
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
  JA_ERR_INVALID_ARG = 1,  /* null pointer, size < 1, bad stride, alignment or buffer size */
  JA_ERR_UNSUPPORTED = 2,  /* head_dim not 64 or 128, shape past a size limit          */
  JA_ERR_HIP = 3           /* the HIP runtime refused the launch                       */
} ja_status;

/* ja_params.flags */
#define JA_FLAG_NO_SPLIT 1u  /* never split the last round of workgroups (see below) */

/*
 * Shape and layout of one attention call.
 *   batch, seq_len, heads >= 1; head_dim in {64, 128}.
 *   Q/K/V/O are addressed as x[b*x_sb + s*x_ss + h*x_sh + d] (strides in
 *   ELEMENTS, the D stride is 1).  A contiguous [B, S, H, D] tensor has
 *   x_ss = H*D, x_sh = D, x_sb = S*H*D; [B, H, S, D] works too.  Strides must
 *   be multiples of 8 and base pointers 16-byte aligned (16-byte vector
 *   loads).  Calls on e4m3 codes take them contiguous [B, S, H, D] and ignore
 *   the Q/K/V strides.  softmax_scale = 0 selects 1/sqrt(head_dim).
 *
 *   pos, rope_theta, rope_table, rope_table_bytes: 2D-axial RoPE of Q and K.
 *   pos is device int32 [seq_len][2], the (row, col) grid position of each
 *   token (text tokens conventionally at (0, 0)); rope_theta is the base of
 *   the frequencies (0 selects 10000).  rope_table may hold the cos/sin
 *   table of those positions built by joint_attn_rope_table_2d (same
 *   seq_len, head_dim and theta), rope_table_bytes its size (at least
 *   seq_len * head_dim * 8); with it no call rebuilds the table and pos is
 *   not read.  RoPE is applied iff pos or rope_table is non-NULL.  Calls
 *   that rotate build the table themselves (in their workspace, or in the
 *   prepared K/V buffer) when only pos is given.
 *
 *   q_norm, k_norm, norm_eps: optional query/key RMS normalization (the
 *   pages fuse "query/key normalization" with RoPE into the QKV epilogue,
 *   section "GEMM kernel optimization").  q_norm / k_norm are device fp32
 *   weights [head_dim] (16-byte aligned), shared by all heads; NULL = that
 *   tensor is not normalized.  Each (batch, token, head) vector x becomes
 *     y_d = x_d / sqrt(mean(x^2) + eps) * g_d
 *   before RoPE and with no rounding of its own, evaluated in fp64 like the
 *   rotation (see below).  norm_eps = 0 selects 1e-6 (the fp32 value).  The
 *   normalization happens wherever RoPE is applied.
 *
 *   Precision of the Q/K prologue: normalization and rotation are evaluated
 *   in fp64 from the fp64 cos/sin table, and the result is rounded ONCE to
 *   the operand format (bf16 to nearest even; e4m3 after the scale), as if
 *   the exact value were rounded.
 *
 *   flags: JA_FLAG_NO_SPLIT, or 0.
 *
 * Zero-initialize the struct to get no RoPE, no normalization, no flags.
 */
typedef struct {
  int32_t batch, seq_len, heads, head_dim;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  float softmax_scale;
  const int32_t *pos;
  float rope_theta;
  const double *rope_table;
  size_t rope_table_bytes;
  const float *q_norm, *k_norm;
  float norm_eps;
  uint32_t flags;
} ja_params;

/* ======================================================================
 * BF16 path
 * ====================================================================== */

/*
 * joint_attn_fwd_bf16 - BF16 joint attention of Q, K, V with RoPE (and the
 * optional Q/K RMS normalization) fused into the loads of Q and K.
 *   q, k, v    device bf16, layout per ja_params.
 *   o          device bf16, layout per ja_params (o_* strides); must not
 *              alias q, k, v or the workspace.
 *   lse        device float [batch][heads][seq_len], nullable: natural-log
 *              log-sum-exp of each query row's scaled scores.
 *   workspace, workspace_bytes   at least
 *              joint_attn_fwd_bf16_workspace_bytes(p) bytes: the prepared
 *              K/V of joint_attn_prep_kv_bf16 (RoPE and coordinate tables
 *              included when only pos is given) and the partial results of
 *              the split below.
 * Q and K are normalized and rotated in fp64 and rounded once to bf16 before
 * Q K^T.  Softmax
 * statistics and both products accumulate in fp32; P is rounded to bf16 for
 * the P.V product and the normaliser sums that bf16 P.  Work items of a last,
 * mostly idle round of workgroups are split over key ranges and merged
 * exactly (the softmax rescaling used between key tiles), unless
 * JA_FLAG_NO_SPLIT.  The result is bitwise reproducible for a given shape
 * and device.
 */
size_t joint_attn_fwd_bf16_workspace_bytes(const ja_params *p);
ja_status joint_attn_fwd_bf16(const ja_params *p, const void *q, const void *k, const void *v,
                              void *o, float *lse, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Block granularity of the block-sparse forwards' masks. */
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
 *   Every other argument and the arithmetic are those of joint_attn_fwd_bf16
 *   (same workspace size); an all-nonzero mask gives the same result as
 *   joint_attn_fwd_bf16 with JA_FLAG_NO_SPLIT.  seq_len up to 1048576
 *   (JA_ERR_UNSUPPORTED above).  Time scales with the kept blocks.
 */
ja_status joint_attn_fwd_bf16_block_sparse(const ja_params *p, const void *q, const void *k,
                                           const void *v, const uint8_t *block_mask, void *o,
                                           float *lse, void *workspace, size_t workspace_bytes,
                                           void *stream);

/*
 * joint_attn_rope_table_2d - cos/sin of every rotation angle of 2D-axial
 * RoPE (the position encoding of the image latent grid; the pages fuse RoPE
 * into the QKV epilogue, section "GEMM kernel optimization").
 *   pos    device int32 [seq_len][2]: (row, col) grid position of each token;
 *          any int32 values.
 *   table  device double [seq_len][head_dim/2][2] (seq_len * head_dim * 8
 *          bytes, 16-byte aligned): written with (cos a, sin a) of pair p's
 *          angle a in fp64.  Pair
 *          p < head_dim/4 rotates by the row with frequency w_p; pair
 *          p >= head_dim/4 by the column with w_(p-D/4); w_k =
 *          theta^(-4k/head_dim) (the 1-D RoPE of dimension D/2 on each axis).
 *   theta  > 0 (10000 in the FLUX-style DiT).
 * The table depends only on positions, head_dim and theta: build it once per
 * forward pass and pass it to every layer's calls as ja_params.rope_table.
 */
ja_status joint_attn_rope_table_2d(const int32_t *pos, int32_t seq_len, int32_t head_dim,
                                   float theta, double *table, void *stream);

/*
 * joint_attn_prep_kv_bf16 - first phase of joint_attn_fwd_bf16: RoPE (and
 * the optional K normalization) fused into the single load of K (same page,
 * section "GEMM kernel optimization", where RoPE is fused into the epilogue
 * that produces K), V transposed.
 *   k, v     device bf16, layout per ja_params (its K and V strides).
 *   kv       device buffer (16-byte aligned) of kv_bytes >=
 *            joint_attn_prep_kv_bf16_bytes(p), written with
 *              Kr [batch*heads][S_pad][head_dim]  rotated K (bf16),
 *              Vt [batch*heads][S_pad/32][head_dim][32]  V transposed in
 *                   tiles of 32 keys (per tile one row of 32 keys for each
 *                   head-dimension column), the keys of every 16-key group
 *                   in the order p -> 4*(p/8) + (p%8 < 4 ? p%8 : p%8 + 4)
 *                   (the P operand order of the forward),
 *              and, when p gives pos without rope_table, the RoPE table of
 *              pos (fp64 [seq_len][head_dim/2][2]), then the coordinate
 *              table (fp64 [1024][head_dim/4][2]: cos and sin of c * w_k
 *              for every grid coordinate c < 1024), each starting on a
 *              256-byte boundary; the forward rotates Q from the coordinate
 *              table where a token's coordinates lie in it (the same values
 *              bit for bit),
 *            S_pad = seq_len rounded up to 64, zeros past seq_len.
 * The buffer depends only on K, V and the positions: when several calls
 * share them, prepare once.
 */
size_t joint_attn_prep_kv_bf16_bytes(const ja_params *p);
ja_status joint_attn_prep_kv_bf16(const ja_params *p, const void *k, const void *v, void *kv,
                                  size_t kv_bytes, void *stream);

/*
 * joint_attn_fwd_bf16_prepared - second phase of joint_attn_fwd_bf16: the
 * attention of q on K/V prepared by joint_attn_prep_kv_bf16 with the same
 * p (Q is rotated with the table p names, or the one in kv).
 *   kv, kv_bytes   the prepared buffer.
 *   workspace, workspace_bytes   at least
 *            joint_attn_fwd_bf16_prepared_workspace_bytes(p) bytes (0 when
 *            no split is planned; NULL allowed then).
 * Other arguments as for joint_attn_fwd_bf16.
 */
size_t joint_attn_fwd_bf16_prepared_workspace_bytes(const ja_params *p);
ja_status joint_attn_fwd_bf16_prepared(const ja_params *p, const void *q, const void *kv,
                                       size_t kv_bytes, void *o, float *lse, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* joint_attn_fwd_bf16_block_sparse on K/V prepared by joint_attn_prep_kv_bf16
 * (workspace: joint_attn_fwd_bf16_prepared_workspace_bytes). */
ja_status joint_attn_fwd_bf16_block_sparse_prepared(const ja_params *p, const void *q,
                                                    const void *kv, size_t kv_bytes,
                                                    const uint8_t *block_mask, void *o,
                                                    float *lse, void *workspace,
                                                    size_t workspace_bytes, void *stream);

/*
 * joint_attn_fwd_bf16_prepared_noalloc - joint_attn_fwd_bf16_prepared for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments and
 * result, without the workspace.  Its scratch (the partial results of the
 * split of the last round) is a static device array of
 * JA_NOALLOC_SCRATCH_BYTES that every device the library runs on holds
 * until the process ends; a shape whose split needs more gets
 * JA_ERR_UNSUPPORTED (JA_FLAG_NO_SPLIT needs none).  All calls on one device
 * share that array, so two calls that overlap on one device race.  The call
 * allocates nothing.
 */
#define JA_NOALLOC_SCRATCH_BYTES ((size_t)72 << 20)
ja_status joint_attn_fwd_bf16_prepared_noalloc(const ja_params *p, const void *q,
                                               const void *kv, size_t kv_bytes, void *o,
                                               float *lse, void *stream);

/* ======================================================================
 * FP8 path
 * ====================================================================== */

/*
 * joint_attn_quant_rope_fp8 - RoPE on Q and K (after the optional Q/K RMS
 * normalization), then per-token FP8 quantization of Q, K and V (the pages'
 * fp8 qk_dtype / v_dtype, section "Quantized and sparse attention").
 *   q, k, v     device bf16, layout per ja_params (its Q, K, V strides).
 *   q8, k8, v8  device e4m3 (1 byte each), written contiguous
 *               [batch][seq_len][heads][head_dim], 16-byte aligned.
 *   sq, sk, sv  device float [batch][heads][seq_len]: one scale per (b, token,
 *               head).  For each head vector x (Q and K after the fp64
 *               prologue, as for the BF16 path): amax = max|x|;
 *               Q and K: scale = the smallest power of two s with
 *               amax <= 448 s, at least 2^-126 (an E8M0 exponent);
 *               V: scale = fl32(amax / 448); all three: 1 if amax = 0;
 *               code = e4m3_rne(clamp(x / scale, -448, 448)) with the
 *               quotient rounded once (from its exact value).
 *   workspace, workspace_bytes   joint_attn_quant_rope_fp8_workspace_bytes(p)
 *               bytes (the RoPE table, when only pos is given; else 0).
 */
size_t joint_attn_quant_rope_fp8_workspace_bytes(const ja_params *p);
ja_status joint_attn_quant_rope_fp8(const ja_params *p, const void *q, const void *k,
                                    const void *v, void *q8, void *k8, void *v8, float *sq,
                                    float *sk, float *sv, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * joint_attn_fwd_fp8 - joint attention on FP8 inputs produced by
 * joint_attn_quant_rope_fp8 (RoPE already applied: pos and rope_table are
 * not used).
 *   q8, k8, v8  device e4m3, contiguous [batch][seq_len][heads][head_dim],
 *               16-byte aligned.
 *   sq, sk, sv  device float [batch][heads][seq_len]: their dequantization
 *               scales.  sq and sk must be positive normal powers of two (the
 *               quantizer's): their exponents are the E8M0 block scales of
 *               the Q K^T MFMA.  sv must be positive and finite.  Rows that
 *               meet another value come back NaN (O and LSE): a bad sq value
 *               poisons the rows of its 128-query block, a bad sk or sv value
 *               every row of its (batch, head).
 *   o           device bf16, layout per ja_params (o_* strides).
 *   lse         device float [batch][heads][seq_len], nullable.
 *   workspace, workspace_bytes   joint_attn_fwd_fp8_workspace_bytes(p) bytes:
 *               the prepared K/V of joint_attn_prep_kv_fp8 and the split's
 *               partial results.
 * Q K^T and P.V run on FP8 MFMA, Q K^T with the Q and K scales as E8M0
 * block scales.  V's per-key scale is folded into the probabilities before
 * they are rounded to e4m3 for P.V: each score accumulator starts at
 * log2(sv[key]) / c (c the softmax scale in the exp2 domain), so that
 * P' = exp2(c acc - ref) = P * sv[key], with the reference ref kept 5 below
 * the running row max (P' < 2^8); the normaliser sums P' / sv[key] in fp32.
 * Softmax statistics and accumulation are fp32; the output is bf16.  The
 * size of one (batch, head)'s prepared K or V (S_pad * head_dim bytes) must
 * stay below 2^31: JA_ERR_UNSUPPORTED.
 */
size_t joint_attn_fwd_fp8_workspace_bytes(const ja_params *p);
ja_status joint_attn_fwd_fp8(const ja_params *p, const void *q8, const void *k8, const void *v8,
                             const float *sq, const float *sk, const float *sv, void *o,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * joint_attn_fwd_fp8_block_sparse - joint_attn_fwd_fp8 restricted to the
 * blocks of a given block mask (the pages' block-sparse attention on a
 * general block-sparse kernel, section "Quantized and sparse attention", here
 * on FP8 inputs).  block_mask as for joint_attn_fwd_bf16_block_sparse (128
 * queries x 64 keys, one mask column per 64-key FP8 tile); a query row that
 * keeps no key gets O = 0 and LSE = -inf.  Every other argument, the
 * arithmetic and the workspace size (joint_attn_fwd_fp8_workspace_bytes) are
 * those of joint_attn_fwd_fp8; an all-nonzero mask gives the same result as
 * joint_attn_fwd_fp8 with JA_FLAG_NO_SPLIT.  seq_len up to 1048576
 * (JA_ERR_UNSUPPORTED above).
 */
ja_status joint_attn_fwd_fp8_block_sparse(const ja_params *p, const void *q8, const void *k8,
                                          const void *v8, const float *sq, const float *sk,
                                          const float *sv, const uint8_t *block_mask, void *o,
                                          float *lse, void *workspace, size_t workspace_bytes,
                                          void *stream);

/*
 * Repair of the FP8 path (the pages' VC-Attention FP8 with vc_repair_budget,
 * section "Quantized and sparse attention": a small budget of the tokens
 * whose quantization error is largest get their residual added back).
 * Reading: per (batch, head), token t's error is
 * e = fl32(max_d |k - k^| + max_d |v - v^|), the terms in fp64 (k the
 * rotated key that was quantized, k^ = value(code) * scale); the n_rep
 * tokens with the largest e (ties to the lower index) are repaired: their
 * key and value enter attention at bf16-path precision.
 *
 * joint_attn_fp8_repair_count - tokens repaired per (batch, head) for a
 * budget: ceil(budget * seq_len), evaluated in fp64; -1 if the budget is not
 * in [0, 1] or seq_len < 1.
 */
int32_t joint_attn_fp8_repair_count(double budget, int32_t seq_len);

/*
 * joint_attn_fp8_repair_plan - selects the repaired tokens and gathers them.
 *   p           shape, positions, K norm and the K/V strides of k and v (Q
 *               and O strides unused).
 *   k, v        as for joint_attn_quant_rope_fp8.
 *   k8, v8, sk, sv   that call's outputs.
 *   n_rep       0 <= n_rep <= seq_len (joint_attn_fp8_repair_count).
 *   idx         device int32 [batch][heads][n_rep]: written with the repaired
 *               token indices, ascending (may be NULL when n_rep = 0).
 *   kr, vr      device bf16 [batch][heads][n_pad][head_dim], n_pad = n_rep
 *               rounded up to a multiple of 32: the rotated keys (rotation
 *               and bf16 rounding as in joint_attn_fwd_bf16) and the values of
 *               the repaired tokens; rows n_rep .. n_pad-1 are zero.
 *   kbias       device float [batch][heads][seq_len]: 0, or -inf for a
 *               repaired token.
 *   workspace, workspace_bytes   joint_attn_fp8_repair_plan_workspace_bytes(p)
 *               bytes (the RoPE table, when only pos is given; else 0).
 * seq_len is limited to 39936 (the selection keeps a row's errors in LDS);
 * larger: JA_ERR_UNSUPPORTED.
 */
size_t joint_attn_fp8_repair_plan_workspace_bytes(const ja_params *p);
ja_status joint_attn_fp8_repair_plan(const ja_params *p, const void *k, const void *v,
                                     const void *k8, const void *v8, const float *sk,
                                     const float *sv, int32_t n_rep, int32_t *idx, void *kr,
                                     void *vr, float *kbias, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* The repair set passed to the FP8 preparation and forward (n_rep = 0: none). */
typedef struct {
  int32_t n_rep;
  const float *kbias;   /* [batch][heads][seq_len], 4-byte aligned */
  const void *kr, *vr;  /* [batch][heads][n_pad][head_dim] bf16, 16-byte aligned */
} ja_fp8_repair;

/*
 * joint_attn_prep_kv_fp8 - first phase of joint_attn_fwd_fp8: the e4m3 keys
 * and values of each (batch, head) laid out as the forward's LDS tiles, with
 * the per-key values of its softmax.  One pass over K and V.
 *   p           shape and softmax_scale (the forward must use the same); the
 *               Q, K, V and O strides are unused.
 *   k8, v8, sk, sv   as for joint_attn_fwd_fp8.  A key whose sk is not a
 *               positive normal power of two, or whose sv is not positive
 *               and finite, turns every row of its (batch, head) into NaN.
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
 */
size_t joint_attn_prep_kv_fp8_bytes(const ja_params *p);
ja_status joint_attn_prep_kv_fp8(const ja_params *p, const void *k8, const void *v8,
                                 const float *sk, const float *sv, const ja_fp8_repair *repair,
                                 void *kv8, size_t kv8_bytes, void *stream);

/*
 * joint_attn_fwd_fp8_prepared - second phase of joint_attn_fwd_fp8: the
 * attention of q8 on K/V prepared by joint_attn_prep_kv_fp8 with the same p.
 *   q8, sq      as for joint_attn_fwd_fp8.
 *   kv8, kv8_bytes   the prepared buffer.  If it was prepared for another
 *               softmax scale, every row comes back NaN.
 *   repair      nullable: with n_rep > 0, the repaired tokens from
 *               joint_attn_fp8_repair_plan (kr, vr; kbias went to the
 *               preparation), attended from their bf16 values in the same
 *               softmax.
 *   workspace, workspace_bytes   at least
 *               joint_attn_fwd_fp8_prepared_workspace_bytes(p) bytes (0 when
 *               no split is planned; NULL allowed then).
 * Other arguments and the arithmetic as for joint_attn_fwd_fp8.
 */
size_t joint_attn_fwd_fp8_prepared_workspace_bytes(const ja_params *p);
ja_status joint_attn_fwd_fp8_prepared(const ja_params *p, const void *q8, const float *sq,
                                      const void *kv8, size_t kv8_bytes,
                                      const ja_fp8_repair *repair, void *o, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* joint_attn_fwd_fp8_block_sparse on K/V prepared by joint_attn_prep_kv_fp8
 * (without repair; workspace: joint_attn_fwd_fp8_prepared_workspace_bytes). */
ja_status joint_attn_fwd_fp8_block_sparse_prepared(const ja_params *p, const void *q8,
                                                   const float *sq, const void *kv8,
                                                   size_t kv8_bytes, const uint8_t *block_mask,
                                                   void *o, float *lse, void *workspace,
                                                   size_t workspace_bytes, void *stream);

/* ======================================================================
 * Status
 * ====================================================================== */

/* Human-readable name of a status code (static string, never NULL). */
const char *joint_attn_status_string(ja_status s);

/* What the last failing library call of this thread found wrong: the
 * argument it rejected, or the HIP error (static per-thread buffer; "" if
 * none). */
const char *joint_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JOINT_ATTN_H */
