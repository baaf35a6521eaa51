/*
 * rrp_oracle.h -- plain CPU oracle for the RoPE-aligned Q/K rotation + INT4 KV4 path.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the slow, obviously-correct
 * reference that the GPU path is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product library never links, includes or calls it, and it shares no code,
 * header, table or constant with the product library.
 *
 * Everything is evaluated in fp64 from the exact input values, except where
 * a definition itself fixes a narrower precision (the fp32 RoPE angle, the
 * fp32 group scale, the fp16 stored scale, the bf16 / fp32 Q output).
 *
 * Sources (cited by page title and section):
 *   [RAQK]  "When Local Variance Optimality Is Not Enough: RoPE-Aligned Q/K
 *           Rotations for Dynamic 4-Bit Quantisation" -- the abstract page and
 *           the two technical summaries (sections: problem statement,
 *           methodology, theoretical characterisation, optimisation
 *           objective, estimator strategies, contributions, results).
 *   [NOTES] "LLM旋转量化笔记" (LLM rotation-quantisation notes) -- section 1.2
 *           (symmetric quantiser), section 2.2 (norm preservation and the
 *           normalised Hadamard example), section 3.2.1 (online Q/K rotation
 *           after RoPE), section 3.3 (online FWHT over head_dim), section 6.1
 *           (Sylvester construction).
 */
#ifndef RRP_ORACLE_H
#define RRP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_ROPE_HALF_SPLIT = 0, ORC_ROPE_INTERLEAVED = 1 };
enum { ORC_EST_DEFAULT = 0, ORC_EST_K_ONLY = 1, ORC_EST_STREAM_BALANCED = 2 };
enum { ORC_STREAM_Q = 0, ORC_STREAM_K = 1 };

/* Number of fp64 accumulators per (pair, stream): n, Su, Sv, Suu, Svv, Suv. */
#define ORC_NMOM 6

/* ---- scalar building blocks (exported so the tests can pin each one) ---- */

/* inv_freq[k] = fp32(theta^(-2k/d)), k < d/2, evaluated in fp64 and rounded once. */
void orc_inv_freq(double theta, int head_dim, float* inv_freq);

/* RoPE angle of pair k at position pos: one fp32 multiply fp32(pos) * inv_freq[k]. */
float orc_rope_angle(int32_t pos, float inv_freq_k);

/* Channel indices of RoPE pair k: (lo, hi) = (k, k + d/2) or (2k, 2k + 1). */
void orc_pair_channels(int head_dim, int layout, int k, int* lo, int* hi);

/* out = RoPE_pos(x): each pair (x_lo, x_hi) rotated by its angle. */
void orc_rope_row(const double* x, int head_dim, int layout, const float* inv_freq,
                  int32_t pos, double* out);

/* out = R_phi(x): each pair rotated by angles[k] (same sense as RoPE). */
void orc_pair_rotate_row(const double* x, int head_dim, int layout, const float* angles,
                         double* out);

/* out = blockdiag(H_b / sqrt(b)) x, Sylvester Hadamard in natural order, written
 * from its entry formula H[i][m] = (-1)^popcount(i & m).  b == 1 is the identity. */
void orc_hadamard_blocks(const double* x, int n, int b, double* out);

/* Full row transform: Hadamard_b( R_phi( RoPE_pos(x) ) ).  angles may be NULL. */
void orc_transform_row(const double* x, int head_dim, int layout, const float* inv_freq,
                       int32_t pos, const float* angles, int b, double* out);

/* IEEE binary16 bits of x, round-to-nearest-even, saturated to +-65504. */
uint16_t orc_f16_bits(float x);
/* Value of binary16 bits. */
double orc_f16_value(uint16_t bits);
/* bfloat16 bits of x, round-to-nearest-even (x finite). */
uint16_t orc_bf16_bits(double x);

/* Symmetric absmax INT4 quantiser for one group of g values.
 * m = max|y|, s32 = fp32(m / 7), s_h = fp16(s32); q = clamp(rne(y / s_h), -7, 7),
 * all-zero codes when s_h == 0. */
void orc_quantize_group(const double* y, int g, int8_t* q, uint16_t* s_h_bits, float* s32);

/* byte i = (q[2i] & 0xF) | (q[2i+1] & 0xF) << 4. n even. */
void orc_pack_nibbles(const int8_t* q, int n, uint8_t* bytes);

/* ---- the three operations ---- */

/* angle_heads: 0 or 1 = one angle set shared by every head of the layer (the
 * parameterisation the paper evaluates); n_kv_heads = one set per key head,
 * query head h using the set of its key head h * Hkv / Hq.  Angle arrays are
 * [angle groups][d/2], moments [angle groups][d/2][2][6]. */
typedef struct orc_shape {
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t rope_layout;
    double rope_theta;
    int32_t angle_heads;
    int32_t reserved;
} orc_shape;

/* Rotate Q and K rows, quantise K rows into the KV4 cache.
 *   q: [T][Hq][d], k: [T][Hkv][d] in `dtype` (fp32 or bf16 bits), pos: int32[T].
 *   q_out (may be NULL): [T][Hq][d] in `dtype` (bf16 by RNE from fp64).
 *   k_codes: uint8[n_slots][Hkv][d/2], k_scales: uint16 (fp16 bits) [n_slots][Hkv][d/g];
 *   row t goes to slot slot_mapping[t] (slot = t when slot_mapping is NULL); slots outside
 *   [0, n_slots) are skipped.
 *   q_rot (may be NULL): fp64 [T][Hq][d]; k_rot (may be NULL): fp64 [T][Hkv][d];
 *   k_scale32 (may be NULL): fp32 [T][Hkv][d/g].
 * Returns 0, or -1 on an invalid argument. */
int orc_rotate_quantize_qk(const orc_shape* s, int dtype, const void* q, const void* k,
                           const int32_t* pos, int64_t n_tokens, const float* angles,
                           int support_b, int group, void* q_out, uint8_t* k_codes,
                           uint16_t* k_scales, const int64_t* slot_mapping, int64_t n_slots,
                           double* q_rot, double* k_rot, float* k_scale32);

/* Quantise V rows into the V half of the KV4 cache: y = H_d / sqrt(d) . v (full-head
 * Sylvester Hadamard, no RoPE, no pair rotation), then the K group quantiser and
 * packing.  v: [T][Hkv][d]; v_codes / v_scales / slot rules as for K;
 * v_rot (may be NULL): fp64 [T][Hkv][d]; v_scale32 (may be NULL): fp32 [T][Hkv][d/g]. */
int orc_quantize_v(const orc_shape* s, int dtype, const void* v, int64_t n_tokens, int group,
                   uint8_t* v_codes, uint16_t* v_scales, const int64_t* slot_mapping, int64_t n_slots,
                   double* v_rot, float* v_scale32);

/* Accumulate post-RoPE pair moments into moments[angle groups][P][2][6] (n, Su, Sv,
 * Suu, Svv, Suv); each head adds to its angle group; q may be NULL (Q stream
 * skipped). */
int orc_calibrate_moments(const orc_shape* s, int dtype, const void* q, const void* k,
                          const int32_t* pos, int64_t n_tokens, double* moments);

/* Closed-form minimax-variance angle per pair from accumulated moments.
 * phi64 / phi32 / abc ([P][3] centred a, b, c) may each be NULL. */
int orc_angles_from_moments(const double* moments, int n_pairs, int estimator,
                            double* phi64, float* phi32, double* abc);

/* stats[8] = {E = sum (yhat - y)^2, N = sum y^2, sum of group absmax, max group absmax,
 *             sum of group (max - min), n_groups, n_rows, 0}. */
int orc_quant_error_stats(const orc_shape* s, int dtype, const void* k, const int32_t* pos,
                          int64_t n_tokens, const float* angles, int support_b, int group,
                          double* stats);

/* Decode attention logits from the KV4 cache: scores[b][h][j] = sum_c q[b][h][c] *
 * code * s_h for key j < min(seq_len[b], max_len) at slot seq_start[b] + j, key head
 * h * Hkv / Hq (fp64).  q: [n_seqs][Hq][d] in `dtype`; scores: fp64 [n_seqs][Hq][max_len];
 * NaN for slots outside [0, n_slots); entries at j >= seq_len[b] are left untouched. */
int orc_decode_scores(const orc_shape* s, int dtype, const void* q, int64_t n_seqs,
                      const uint8_t* k_codes, const uint16_t* k_scales, int group, int64_t n_slots,
                      const int64_t* seq_start, const int32_t* seq_len, int max_len, double* scores);

/* Threads the token-parallel entry points may use (OpenMP), 1 without OpenMP. */
int orc_max_threads(void);
int orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
