/*
 * rrp.h -- C-ABI of the MI355X (gfx950) library for the RoPE-aligned Q/K
 * rotation and dynamic INT4 KV4 quantisation path.
 *
 * The method: "When Local Variance Optimality Is Not Enough: RoPE-Aligned Q/K
 * Rotations for Dynamic 4-Bit Quantisation" (abstract and technical summary,
 * sections "methodology", "optimisation objective", "estimator strategies",
 * "contributions").  After RoPE, every Q and K row of a head is turned by a
 * head-shared plane rotation inside each RoPE frequency pair (angle phi_k),
 * then by a block Walsh-Hadamard transform of support b; each K row is then
 * quantised to INT4 with a dynamic per-group absmax scale and written into a
 * packed KV4 cache.  Q is rotated but not quantised (only K is quantised after
 * the transform, estimator-strategies section).
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE memory unless marked "host".  The caller owns every
 *     buffer; nothing passed in is retained after the call returns.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the null stream).  The host returns as soon as the work is
 *     enqueued; the caller synchronises before reading outputs.
 *   - Arguments are validated on the host before anything is enqueued.  On an
 *     error the function returns a non-zero rrp_status and enqueues nothing.
 *     RRP_ERR_HIP reports a failed kernel launch; work enqueued before the
 *     failing launch may have run.
 *   - The library allocates no memory.  Calibration and diagnostics keep their
 *     per-block partial sums in a caller-owned device workspace whose size the
 *     matching *_workspace_size query gives for the same shape and token count;
 *     a NULL or smaller workspace is RRP_ERR_INVALID_ARG, one not 8-byte aligned
 *     RRP_ERR_MISALIGNED (both before anything is enqueued).  The workspace is
 *     used by the enqueued work only: it may be reused by work enqueued later
 *     on the same stream, and two calls in flight at once need two workspaces.
 *   - Tensors are dense, row-major, token-major: Q is [n_tokens][n_q_heads]
 *     [head_dim], K is [n_tokens][n_kv_heads][head_dim], in `dtype`.
 *   - Q, K and Q-output pointers must be 16-byte aligned (128-bit accesses).
 *   - Supported head_dim: 64 and 128.  Others return RRP_ERR_UNSUPPORTED.
 *   - Thread-safe: the library keeps no mutable global state.
 */
#ifndef RRP_H
#define RRP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rrp_status {
    RRP_OK = 0,
    RRP_ERR_INVALID_ARG = 1,  /* NULL required pointer, bad size, bad enum value      */
    RRP_ERR_MISALIGNED = 2,   /* a pointer violates its alignment requirement         */
    RRP_ERR_UNSUPPORTED = 3,  /* valid in principle but not built (e.g. head_dim 96)  */
    RRP_ERR_HIP = 4           /* a HIP runtime call failed                             */
} rrp_status;

typedef enum rrp_dtype { RRP_F32 = 0, RRP_BF16 = 1 } rrp_dtype;

/* Estimators of the shared angle ("estimator strategies" section):
 *   DEFAULT          pool the raw Q and K sums over heads and tokens, then centre
 *                    (each sample counts once, so Q weighs H_q / H_kv times K);
 *   K_ONLY           the covariance of the K samples alone;
 *   STREAM_BALANCED  equal weight to the Q and K raw (uncentred) moments, each
 *                    normalised by its own sample count, then centre. */
typedef enum rrp_estimator {
    RRP_EST_DEFAULT = 0,
    RRP_EST_K_ONLY = 1,
    RRP_EST_STREAM_BALANCED = 2
} rrp_estimator;

/* Which channels form RoPE frequency pair k (problem-statement section: RoPE
 * splits a head into fixed two-dimensional frequency pairs).
 *   HALF_SPLIT   (k, k + head_dim/2)   -- the Llama / Mistral convention
 *   INTERLEAVED  (2k, 2k + 1) */
typedef enum rrp_rope_layout { RRP_ROPE_HALF_SPLIT = 0, RRP_ROPE_INTERLEAVED = 1 } rrp_rope_layout;

/* Shape of one attention layer (host struct).  RoPE frequency of pair k is
 * fp32(rope_theta^(-2k/head_dim)) (rounded once from fp64); the angle at
 * position p is the single fp32 product fp32(p) * freq_k.
 *
 * angle_heads chooses the pair-angle parameterisation ("optimisation
 * objective" section: the paper evaluates one angle per frequency pair shared
 * by all heads of a layer):
 *   0 or 1      one set of head_dim/2 angles shared by every head;
 *   n_kv_heads  one set per key head; query head h uses the set of its key head
 *               h * n_kv_heads / n_q_heads (so the rotation still cancels in
 *               Q K^T).  Needs n_q_heads a multiple of n_kv_heads and at most 8
 *               key heads (RRP_ERR_UNSUPPORTED above).
 * Every other value is RRP_ERR_INVALID_ARG.  "Angle sets" below means 1 or
 * n_kv_heads accordingly; angle arrays are float[angle sets][head_dim/2]. */
typedef struct rrp_shape {
    int32_t n_q_heads;   /* >= 0 */
    int32_t n_kv_heads;  /* >= 1 */
    int32_t head_dim;    /* 64 or 128 */
    int32_t rope_layout; /* rrp_rope_layout */
    double rope_theta;   /* > 0 */
    int32_t angle_heads; /* 0 / 1 (shared) or n_kv_heads (one set per key head) */
    int32_t reserved;    /* set to 0 */
} rrp_shape;

/* rrp_rotate_quantize_qk -- the hot path ("methodology" and "contributions"
 * sections: RoPE, then the pair rotation, then the block Hadamard of support b;
 * dynamic tokenwise group-range INT4 quantisation of K into the KV4 cache).
 *
 * For each token t, each Q head and each K head:
 *   y = H_b / sqrt(b) . R_phi . RoPE_pos[t] (x)
 *   H_b: Sylvester Hadamard on contiguous blocks of b channels, natural order.
 * Q rows: y is written to q_out in `dtype` (bf16 round-to-nearest-even).
 * K rows: for each group of `group` consecutive channels of y,
 *   s32 = fp32(max|y| / 7); s_h = fp16(s32) (nearest-even, saturated at 65504);
 *   code = clamp(round_half_even(y / s_h), -7, 7) (all 0 when s_h == 0);
 *   byte i of the row = (code[2i] & 0xF) | (code[2i+1] & 0xF) << 4.
 *
 * shape         host; head counts, head_dim, RoPE theta and pair layout.
 * dtype         RRP_F32 or RRP_BF16, for q, k and q_out.
 * q             [n_tokens][n_q_heads][head_dim] or NULL (no Q rows processed).
 * k             [n_tokens][n_kv_heads][head_dim], required.
 * pos           int32[n_tokens] RoPE positions, each in [0, 2^24).
 * angles        float[angle sets][head_dim/2] pair angles phi_k (output of
 *               rrp_calibrate_angles) or NULL for no pair rotation.
 * support_b     1, 2, 4, ..., head_dim; 1 = no Hadamard (pairwise only).
 * group         quantisation group size: a power of two in [2, head_dim].
 * q_out         rotated Q, same layout as q; may equal q (in place); NULL = Q
 *               not written.  Requires q.
 * k_codes       uint8 [n_slots][n_kv_heads][head_dim/2], 4-byte aligned.
 * k_scales      uint16 (fp16 bits) [n_slots][n_kv_heads][head_dim/group], 2-byte aligned.
 * slot_mapping  int64[n_tokens]: cache slot of token t, or NULL for slot = t.
 *               Tokens whose slot lies outside [0, n_slots) write nothing
 *               (padding).  Two tokens with one slot: unspecified winner.
 * n_slots       cache capacity in slots; with slot_mapping == NULL it must be
 *               >= n_tokens.
 * q_rot_f32     optional fp32 copy of rotated Q, [n_tokens][n_q_heads][head_dim], 16-B aligned.
 * k_rot_f32     optional fp32 copy of rotated K, [n_tokens][n_kv_heads][head_dim], 16-B aligned.
 * k_scale_f32   optional fp32 group scales s32 indexed by TOKEN (not slot),
 *               [n_tokens][n_kv_heads][head_dim/group], 4-byte aligned.
 * stream        hipStream_t or NULL.
 * n_tokens == 0 is a no-op returning RRP_OK once the shape, support_b and
 * group are valid; the arrays are then not examined and may be NULL. */
int rrp_rotate_quantize_qk(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                           const int32_t* pos, int64_t n_tokens, const float* angles,
                           int32_t support_b, int32_t group, void* q_out, uint8_t* k_codes,
                           uint16_t* k_scales, const int64_t* slot_mapping, int64_t n_slots,
                           float* q_rot_f32, float* k_rot_f32, float* k_scale_f32, void* stream);

/* rrp_rotate_quantize_qkv -- rrp_rotate_quantize_qk plus the V half of the KV4
 * cache in the same launch (LLM rotation-quantisation notes, section 3.2.2: V
 * is multiplied online by the head-wise Hadamard so the value cache loses its
 * outliers; the Hadamard left on the attention output folds into the output
 * projection offline).
 *
 * Q and K rows exactly as rrp_rotate_quantize_qk.  V rows get no RoPE and no
 * pair rotation, and always the full-head transform:
 *   y = H_d / sqrt(head_dim) . v
 * then the K quantiser with the same `group` (same scale rule, codes and
 * nibble order), written at the same slot.
 *
 * v             [n_tokens][n_kv_heads][head_dim] in `dtype`, 16-byte aligned, required.
 * v_codes       uint8 [n_slots][n_kv_heads][head_dim/2] (alignment as k_codes), required.
 * v_scales      uint16 (fp16 bits) [n_slots][n_kv_heads][head_dim/group], required.
 * v_rot_f32     optional fp32 copy of transformed V, [n_tokens][n_kv_heads][head_dim], 16-B aligned.
 * v_scale_f32   optional fp32 V group scales indexed by token, like k_scale_f32.
 * Every other argument, and the error behaviour, as rrp_rotate_quantize_qk. */
int rrp_rotate_quantize_qkv(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                            const void* v, const int32_t* pos, int64_t n_tokens, const float* angles,
                            int32_t support_b, int32_t group, void* q_out, uint8_t* k_codes,
                            uint16_t* k_scales, uint8_t* v_codes, uint16_t* v_scales,
                            const int64_t* slot_mapping, int64_t n_slots, float* q_rot_f32,
                            float* k_rot_f32, float* k_scale_f32, float* v_rot_f32, float* v_scale_f32,
                            void* stream);

/* Workspace bytes (written to *bytes, host) of one rrp_calibrate_angles call
 * with this shape and token count; with_q != 0 when q is not NULL.  0 when
 * n_tokens == 0.  At most 4096 * head_dim/2 * 5 * 8 bytes (10.5 MB at head_dim
 * 128).  Errors: an invalid shape (as the entry point), n_tokens < 0 or
 * bytes == NULL. */
int rrp_calibrate_angles_workspace_size(const rrp_shape* shape, int64_t n_tokens, int32_t with_q, size_t* bytes);

/* rrp_calibrate_angles -- the calibration pass ("optimisation objective" and
 * "estimator strategies" sections: a closed-form shared angle per pair that
 * minimises the larger of the pair's two channel variances under a
 * pooled-covariance, position-averaged surrogate).
 *
 * Accumulates, for every pair k and stream S in {Q, K}, the fp64 sums
 * n, sum u, sum v, sum u^2, sum v^2, sum u*v of the post-RoPE pair (u, v) over
 * all tokens and all heads of S (per-head sets: all heads of the set's group)
 * into
 *   moments   double[angle sets][head_dim/2][2][6]  (stream 0 = Q, 1 = K)
 * which the caller zeroes before the first batch and may keep across batches
 * (it is the resumable calibration state).  Tokens are reduced in a fixed order:
 * repeated calls on the same inputs give bit-identical moments.
 * If angles_out != NULL the angles are then finalised from the accumulated
 * moments with `estimator`: centred covariance [[a, c], [c, b]] of the pair,
 *   phi_k = atan2(a - b, 2c) / 2, wrapped into (-pi/4, pi/4]
 * (0 for a degenerate pair or no samples), written as float[angle sets][head_dim/2].
 *
 * q may be NULL (Q stream not accumulated); then estimator must be K_ONLY.
 * n_tokens == 0 only finalises (if angles_out != NULL).
 * workspace     device, workspace_bytes >= rrp_calibrate_angles_workspace_size
 *               (shape, n_tokens, q != NULL); may be NULL when that size is 0. */
int rrp_calibrate_angles(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                         const int32_t* pos, int64_t n_tokens, int32_t estimator,
                         double* moments, float* angles_out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* rrp_calibrate_angles_noalloc -- rrp_calibrate_angles for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and results (the same
 * block partials, reduced in the same order), with the partials in a static
 * device array of the library instead of a caller workspace.  That array holds
 * 4096 * 64 * 5 doubles (10 MiB, the largest calibration workspace of any
 * accepted shape); each GPU the library runs on holds its own copy until the
 * process ends.  A call whose workspace size would exceed it returns
 * RRP_ERR_UNSUPPORTED (no accepted shape does).  The call allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (different streams, or different host threads without ordering)
 * race and give wrong moments; calls ordered on one stream are safe.  The
 * first call on a device looks up the array's device address (no allocation).
 * Arguments, outputs and errors as rrp_calibrate_angles, without the
 * workspace; RRP_ERR_HIP also reports a failed lookup of the stream's device or
 * of the array. */
int rrp_calibrate_angles_noalloc(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                                 const int32_t* pos, int64_t n_tokens, int32_t estimator, double* moments,
                                 float* angles_out, void* stream);

/* rrp_quant_error_stats -- the diagnostic pass ("contributions" and "results"
 * sections: K range and relative quantisation error along the block-Hadamard
 * support interpolation).  Transforms every K row as rrp_rotate_quantize_qk
 * does (same angles, support_b, group), quantises and dequantises it
 * (yhat = code * s_h) and writes
 *   stats_out  double[8] = { E = sum (yhat - y)^2, N = sum y^2,
 *                            sum of group max|y|, max of group max|y|,
 *                            sum of group (max y - min y), n_groups, n_rows, 0 }
 * (overwritten).  Relative error = sqrt(E / N); mean K range = [2] / [5].
 * Reduced in a fixed order (bit-reproducible).
 * workspace     device, workspace_bytes >= rrp_quant_error_stats_workspace_size
 *               (shape, n_tokens); may be NULL when that size is 0. */
int rrp_quant_error_stats(const rrp_shape* shape, int32_t dtype, const void* k, const int32_t* pos,
                          int64_t n_tokens, const float* angles, int32_t support_b, int32_t group,
                          double* stats_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes (host *bytes) of one rrp_quant_error_stats call: at most
 * 8192 * 5 * 8.  Errors as rrp_calibrate_angles_workspace_size. */
int rrp_quant_error_stats_workspace_size(const rrp_shape* shape, int64_t n_tokens, size_t* bytes);

/* rrp_quant_error_sweep -- the support interpolation in one call ("contributions"
 * and "results" sections: K range and relative quantisation error as the block
 * Hadamard support grows from 2 to head_dim).  Writes, for every support
 * b = 2^j, j = 0 .. log2(head_dim) (b = 1: no Hadamard), the statistics
 * rrp_quant_error_stats gives at that b (same angles and group):
 *   stats_out  double[log2(head_dim) + 1][8], row j = { E, N, sum of group max|y|,
 *              max of group max|y|, sum of group (max y - min y), n_groups,
 *              n_rows, b }  (overwritten).
 * K is read once (one launch).  Each row matches a separate
 * rrp_quant_error_stats call up to the order of fp64 rounding: the transform
 * of support 2^j is built from the one of support 2^(j-1) by one more
 * butterfly stage, kept without its 1 / sqrt(b) (applied to each group's
 * scale constants and to the sums instead), and N is taken once, from the
 * rotated row (every support's transform is orthogonal).
 * workspace     device, workspace_bytes >= rrp_quant_error_sweep_workspace_size
 *               (shape, n_tokens); may be NULL when that size is 0.
 * Errors as rrp_quant_error_stats. */
int rrp_quant_error_sweep(const rrp_shape* shape, int32_t dtype, const void* k, const int32_t* pos,
                          int64_t n_tokens, const float* angles, int32_t group, double* stats_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes (host *bytes) of one rrp_quant_error_sweep call: at most
 * 4096 * (log2(head_dim) + 1) * 5 * 8.  Errors as
 * rrp_calibrate_angles_workspace_size. */
int rrp_quant_error_sweep_workspace_size(const rrp_shape* shape, int64_t n_tokens, size_t* bytes);

/* rrp_decode_scores -- decode attention logits read straight from the KV4 cache
 * (LLM rotation-quantisation notes, section 3.2.1: the head-wise rotation
 * cancels inside Q K^T, so the rotated query against the rotated key is the
 * RoPE logit; the Qift page, introduction: decode reads the KV cache and is
 * memory-bound).  The consumer of what rrp_rotate_quantize_qk writes.
 *
 * For sequence b, query head h (key head h / (n_q_heads / n_kv_heads)) and key
 * j < min(seq_len[b], max_len) at cache slot seq_start[b] + j:
 *   scores[b][h][j] = sum_c q[b][h][c] * code(slot, kv, c) * s_h(slot, kv, c / group)
 * (the logit before any 1/sqrt(head_dim) factor; fp32 result, fp32 accumulation
 * of exact f16 products on the matrix cores).
 *
 * shape       host; n_q_heads a multiple of n_kv_heads, at most 16 query heads
 *             per key head, and 256 * n_kv_heads * head_dim/2 < 2^31 (a slot row
 *             band of 256 keys addressed by 32-bit offsets; else
 *             RRP_ERR_UNSUPPORTED); head_dim 64 or 128.
 * dtype       dtype of q: RRP_BF16 or RRP_F32.
 * q           [n_seqs][n_q_heads][head_dim] rotated queries (the q_out of
 *             rrp_rotate_quantize_qk for the decode tokens), 16-byte aligned.
 * k_codes     uint8 [n_slots][n_kv_heads][head_dim/2], aligned to head_dim/8 bytes.
 * k_scales    uint16 fp16 bits [n_slots][n_kv_heads][head_dim/group], aligned to
 *             min(2 * head_dim/group, 8) bytes.
 * group       the group size the cache was written with (power of two in [2, head_dim]).
 * seq_start   int64[n_seqs], 8-byte aligned: slot of key 0 of each sequence.
 * seq_len     int32[n_seqs]: keys per sequence (values above max_len are cut to max_len).
 * max_len     row length of `scores`, at most 2^31 - 513 (else RRP_ERR_UNSUPPORTED).
 * scores      fp32 [n_seqs][n_q_heads][max_len].  Only j < min(seq_len[b], max_len)
 *             is written; a key whose slot lies outside [0, n_slots) gets NaN.
 * n_slots     cache capacity in slots, >= 1.
 * n_seqs == 0 or max_len == 0 is a no-op returning RRP_OK.  Any number of
 * sequences is accepted: a batch larger than one grid holds is enqueued as
 * several launches over consecutive sequence ranges.  A sequence takes
 * ceil(max_len / 256) * n_kv_heads waves; where the one-dimensional grid is
 * used (n_kv_heads not a multiple of 4, or more than 65535 key chunks) and that
 * exceeds the 67108860 waves one grid holds, RRP_ERR_UNSUPPORTED. */
int rrp_decode_scores(const rrp_shape* shape, int32_t dtype, const void* q, int64_t n_seqs,
                      const uint8_t* k_codes, const uint16_t* k_scales, int32_t group, int64_t n_slots,
                      const int64_t* seq_start, const int32_t* seq_len, int32_t max_len, float* scores,
                      void* stream);

/* Host: static description of a status code. */
const char* rrp_status_string(int status);

/* Host: library version as major * 10000 + minor * 100 + patch. */
int rrp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RRP_H */
