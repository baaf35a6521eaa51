/*
 * rrp_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see rrp_oracle.h).
 *
 * Written from the definitions, one step at a time, in fp64.  No blocking,
 * fusion or fast transforms: the Hadamard is evaluated from its entry formula,
 * the quantiser from its scalar definition, the calibration sums one sample at
 * a time.  Parity of every function is pinned by the CPU test suite against
 * closed forms, library routines, brute force and the worked example printed
 * in the LLM rotation-quantisation notes (section 2.2).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC (see build.py).
 * -ffp-contract=off keeps every product a separately rounded operation, so the
 * fp32 RoPE angle is exactly one fp32 multiply.
 */
#include "rrp_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_MAX_DIM 1024

/* ------------------------------------------------------------------------ */
/* Number formats.                                                           */
/* ------------------------------------------------------------------------ */

/* Round |a| (finite, > 0) to the nearest multiple of 2^(E - mant_bits) where E is
 * its binade exponent, clamped below at emin (gradual underflow).  rint() rounds
 * half to even in the default rounding mode. */
static double round_to_format(double a, int mant_bits, int emin)
{
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) -> binade exponent e - 1 */
    int E = e - 1;
    if (E < emin) E = emin;
    double quantum = ldexp(1.0, E - mant_bits);
    return rint(a / quantum) * quantum;
}

uint16_t orc_f16_bits(float xf)
{
    double x = (double)xf;
    if (isnan(x)) return 0x7E00;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (a >= 65504.0) return (uint16_t)(sign | 0x7BFFu); /* saturate at the largest finite */
    if (a == 0.0) return sign;
    double r = round_to_format(a, 10, -14);
    if (r == 0.0) return sign;
    int e;
    frexp(r, &e);
    int E = e - 1;
    if (E < -14) { /* subnormal: r = mant * 2^-24 */
        return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
    }
    unsigned mant = (unsigned)((ldexp(r, -E) - 1.0) * 1024.0);
    return (uint16_t)(sign | (unsigned)(E + 15) << 10 | mant);
}

double orc_f16_value(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int ex = (bits >> 10) & 0x1F;
    int mant = bits & 0x3FF;
    double v;
    if (ex == 0)
        v = ldexp((double)mant, -24);
    else if (ex == 31)
        v = mant ? NAN : INFINITY;
    else
        v = ldexp(1.0 + mant / 1024.0, ex - 15);
    return sign ? -v : v;
}

uint16_t orc_bf16_bits(double x)
{
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (a == 0.0) return sign;
    double r = round_to_format(a, 7, -126);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float rf = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFFu));
}

static double load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    uint32_t u = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* The row transform.                                                        */
/* ------------------------------------------------------------------------ */

/* RoPE frequencies: theta^(-2k/d) for the k-th two-dimensional frequency pair
 * ([RAQK] problem statement: RoPE splits each head into fixed 2-D frequency
 * pairs with distinct frequencies). */
void orc_inv_freq(double theta, int head_dim, float* inv_freq)
{
    for (int k = 0; k < head_dim / 2; ++k)
        inv_freq[k] = (float)pow(theta, -2.0 * (double)k / (double)head_dim);
}

float orc_rope_angle(int32_t pos, float inv_freq_k)
{
    float p = (float)pos;
    return p * inv_freq_k;
}

void orc_pair_channels(int head_dim, int layout, int k, int* lo, int* hi)
{
    if (layout == ORC_ROPE_INTERLEAVED) {
        *lo = 2 * k;
        *hi = 2 * k + 1;
    } else {
        *lo = k;
        *hi = k + head_dim / 2;
    }
}

/* Rotate the pair (a, b) by an angle with cosine c and sine s. */
static void rotate2(double a, double b, double c, double s, double* oa, double* ob)
{
    *oa = a * c - b * s;
    *ob = b * c + a * s;
}

void orc_rope_row(const double* x, int head_dim, int layout, const float* inv_freq,
                  int32_t pos, double* out)
{
    for (int k = 0; k < head_dim / 2; ++k) {
        int lo, hi;
        orc_pair_channels(head_dim, layout, k, &lo, &hi);
        double alpha = (double)orc_rope_angle(pos, inv_freq[k]);
        double a, b;
        rotate2(x[lo], x[hi], cos(alpha), sin(alpha), &a, &b);
        out[lo] = a;
        out[hi] = b;
    }
}

/* Head-shared pair rotation by phi_k inside each RoPE pair ([RAQK] methodology:
 * the pairwise-only transform; it commutes with RoPE because both are plane
 * rotations of the same pair). */
void orc_pair_rotate_row(const double* x, int head_dim, int layout, const float* angles,
                         double* out)
{
    for (int k = 0; k < head_dim / 2; ++k) {
        int lo, hi;
        orc_pair_channels(head_dim, layout, k, &lo, &hi);
        double phi = (double)angles[k];
        double a, b;
        rotate2(x[lo], x[hi], cos(phi), sin(phi), &a, &b);
        out[lo] = a;
        out[hi] = b;
    }
}

static int parity_bit(unsigned v)
{
    return __builtin_popcount(v) & 1;
}

/* Block Hadamard of support b ([RAQK] contributions: the block-Hadamard support
 * interpolation from b = 2 to b = d_h; [NOTES] section 2.2: normalised by
 * 1/sqrt(K); section 6.1: Sylvester construction, first column all ones). */
void orc_hadamard_blocks(const double* x, int n, int b, double* out)
{
    double norm = 1.0 / sqrt((double)b);
    for (int blk = 0; blk < n; blk += b) {
        for (int i = 0; i < b; ++i) {
            double acc = 0.0;
            for (int m = 0; m < b; ++m) {
                double h = parity_bit((unsigned)(i & m)) ? -1.0 : 1.0;
                acc += h * x[blk + m];
            }
            out[blk + i] = acc * norm;
        }
    }
}

/* Online transform after RoPE: pair rotation, then the block Hadamard
 * ([RAQK] methodology: pairwise + Hadamard composition; [NOTES] section 3.2.1:
 * Q and K are rotated after RoPE, before the KV cache). */
void orc_transform_row(const double* x, int head_dim, int layout, const float* inv_freq,
                       int32_t pos, const float* angles, int b, double* out)
{
    double r[ORC_MAX_DIM], p[ORC_MAX_DIM];
    orc_rope_row(x, head_dim, layout, inv_freq, pos, r);
    if (angles)
        orc_pair_rotate_row(r, head_dim, layout, angles, p);
    else
        memcpy(p, r, sizeof(double) * (size_t)head_dim);
    orc_hadamard_blocks(p, head_dim, b, out);
}

/* ------------------------------------------------------------------------ */
/* Quantiser ([NOTES] section 1.2: q = clip(round(x / s), -qmax, qmax) with   */
/* s = absmax / qmax shared by the group; [RAQK] contributions: the dynamic   */
/* quantiser sets its step from the tokenwise group range).                   */
/* ------------------------------------------------------------------------ */

void orc_quantize_group(const double* y, int g, int8_t* q, uint16_t* s_h_bits, float* s32)
{
    double m = 0.0;
    for (int i = 0; i < g; ++i)
        if (fabs(y[i]) > m) m = fabs(y[i]);
    float s = (float)(m / 7.0);
    uint16_t sh = orc_f16_bits(s);
    double shv = orc_f16_value(sh);
    for (int i = 0; i < g; ++i) {
        if (shv == 0.0) {
            q[i] = 0;
            continue;
        }
        double r = rint(y[i] / shv);
        if (r > 7.0) r = 7.0;
        if (r < -7.0) r = -7.0;
        q[i] = (int8_t)r;
    }
    if (s_h_bits) *s_h_bits = sh;
    if (s32) *s32 = s;
}

void orc_pack_nibbles(const int8_t* q, int n, uint8_t* bytes)
{
    for (int i = 0; i < n / 2; ++i)
        bytes[i] = (uint8_t)(((unsigned)q[2 * i] & 0xFu) | (((unsigned)q[2 * i + 1] & 0xFu) << 4));
}

/* ------------------------------------------------------------------------ */
/* Operations.                                                               */
/* ------------------------------------------------------------------------ */

static int is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

static int check_shape(const orc_shape* s)
{
    if (!s) return -1;
    int d = s->head_dim;
    if (d < 2 || d > ORC_MAX_DIM || (d & 1)) return -1;
    if (s->n_q_heads < 0 || s->n_kv_heads <= 0) return -1;
    if (s->rope_layout != ORC_ROPE_HALF_SPLIT && s->rope_layout != ORC_ROPE_INTERLEAVED) return -1;
    if (!(s->rope_theta > 0.0)) return -1;
    if (s->angle_heads < 0 || (s->angle_heads > 1 && s->angle_heads != s->n_kv_heads)) return -1;
    if (s->angle_heads > 1 && s->n_q_heads % s->n_kv_heads) return -1;
    return 0;
}

/* Number of angle sets, and the set of query head h / key head kh (per-head
 * parameterisation: every query head shares its key head's set, so the
 * rotation still cancels in Q K^T). */
static int angle_groups(const orc_shape* s) { return s->angle_heads > 1 ? s->angle_heads : 1; }
static int q_angle_group(const orc_shape* s, int h)
{
    return s->n_q_heads > 0 ? (int)((int64_t)h * angle_groups(s) / s->n_q_heads) : 0;
}
static int k_angle_group(const orc_shape* s, int kh) { return (int)((int64_t)kh * angle_groups(s) / s->n_kv_heads); }
static const float* angle_set(const float* angles, int group, int head_dim)
{
    return angles ? angles + (int64_t)group * (head_dim / 2) : NULL;
}

int orc_rotate_quantize_qk(const orc_shape* s, int dtype, const void* q, const void* k,
                           const int32_t* pos, int64_t n_tokens, const float* angles,
                           int support_b, int group, void* q_out, uint8_t* k_codes,
                           uint16_t* k_scales, const int64_t* slot_mapping, int64_t n_slots,
                           double* q_rot, double* k_rot, float* k_scale32)
{
    if (check_shape(s) || n_tokens < 0 || !k || !pos || !k_codes || !k_scales) return -1;
    const int d = s->head_dim, hq = s->n_q_heads, hk = s->n_kv_heads;
    if (!is_pow2(support_b) || d % support_b) return -1;
    if (group < 2 || (group & 1) || d % group) return -1;
    if (hq > 0 && !q && (q_out || q_rot)) return -1;
    float inv_freq[ORC_MAX_DIM / 2];
    orc_inv_freq(s->rope_theta, d, inv_freq);
    const int ng = d / group;

#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tokens; ++t) {
        double x[ORC_MAX_DIM], y[ORC_MAX_DIM];
        int8_t codes[ORC_MAX_DIM];
        const int32_t p = pos[t];
        if (q) {
            for (int h = 0; h < hq; ++h) {
                const int64_t row = (t * hq + h) * (int64_t)d;
                for (int c = 0; c < d; ++c) x[c] = load_elem(q, dtype, row + c);
                orc_transform_row(x, d, s->rope_layout, inv_freq, p, angle_set(angles, q_angle_group(s, h), d),
                                  support_b, y);
                for (int c = 0; c < d; ++c) {
                    if (q_rot) q_rot[row + c] = y[c];
                    if (q_out) {
                        if (dtype == ORC_F32)
                            ((float*)q_out)[row + c] = (float)y[c];
                        else
                            ((uint16_t*)q_out)[row + c] = orc_bf16_bits(y[c]);
                    }
                }
            }
        }
        const int64_t slot = slot_mapping ? slot_mapping[t] : t;
        for (int h = 0; h < hk; ++h) {
            const int64_t row = (t * hk + h) * (int64_t)d;
            for (int c = 0; c < d; ++c) x[c] = load_elem(k, dtype, row + c);
            orc_transform_row(x, d, s->rope_layout, inv_freq, p, angle_set(angles, k_angle_group(s, h), d),
                              support_b, y);
            if (k_rot)
                for (int c = 0; c < d; ++c) k_rot[row + c] = y[c];
            for (int j = 0; j < ng; ++j) {
                uint16_t sh;
                float s32;
                orc_quantize_group(y + j * group, group, codes + j * group, &sh, &s32);
                if (k_scale32) k_scale32[(t * hk + h) * ng + j] = s32;
                if (slot >= 0 && slot < n_slots) k_scales[(slot * hk + h) * ng + j] = sh;
            }
            if (slot >= 0 && slot < n_slots)
                orc_pack_nibbles(codes, d, k_codes + (slot * hk + h) * (int64_t)(d / 2));
        }
    }
    return 0;
}

/* V side of the KV4 cache ([NOTES] section 3.2.2: V is multiplied online by the
 * head-wise Hadamard so the value cache loses its outliers; the Hadamard left on
 * the attention output folds into the output projection offline).  No RoPE and
 * no pair rotation: y = H_d / sqrt(d) . v, then the K quantiser and packing. */
int orc_quantize_v(const orc_shape* s, int dtype, const void* v, int64_t n_tokens, int group,
                   uint8_t* v_codes, uint16_t* v_scales, const int64_t* slot_mapping, int64_t n_slots,
                   double* v_rot, float* v_scale32)
{
    if (check_shape(s) || n_tokens < 0 || !v || !v_codes || !v_scales) return -1;
    const int d = s->head_dim, hk = s->n_kv_heads;
    if (group < 2 || (group & 1) || d % group) return -1;
    const int ng = d / group;

#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tokens; ++t) {
        double x[ORC_MAX_DIM], y[ORC_MAX_DIM];
        int8_t codes[ORC_MAX_DIM];
        const int64_t slot = slot_mapping ? slot_mapping[t] : t;
        const int in_cache = slot >= 0 && slot < n_slots;
        for (int h = 0; h < hk; ++h) {
            const int64_t row = (t * hk + h) * (int64_t)d;
            for (int c = 0; c < d; ++c) x[c] = load_elem(v, dtype, row + c);
            orc_hadamard_blocks(x, d, d, y);
            if (v_rot)
                for (int c = 0; c < d; ++c) v_rot[row + c] = y[c];
            for (int j = 0; j < ng; ++j) {
                uint16_t sh;
                float s32;
                orc_quantize_group(y + j * group, group, codes + j * group, &sh, &s32);
                if (v_scale32) v_scale32[(t * hk + h) * ng + j] = s32;
                if (in_cache) v_scales[(slot * hk + h) * ng + j] = sh;
            }
            if (in_cache) orc_pack_nibbles(codes, d, v_codes + (slot * hk + h) * (int64_t)(d / 2));
        }
    }
    return 0;
}

/* Calibration sums ([RAQK] estimator strategies: raw Q and K moment accumulators
 * pooled across heads before centring; optimisation objective: pooled-covariance,
 * position-averaged surrogate).  The samples are the post-RoPE pairs of every
 * calibration token and head; pooling over positions is the position average. */
int orc_calibrate_moments(const orc_shape* s, int dtype, const void* q, const void* k,
                          const int32_t* pos, int64_t n_tokens, double* moments)
{
    if (check_shape(s) || n_tokens < 0 || !k || !pos || !moments) return -1;
    const int d = s->head_dim, P = d / 2;
    float inv_freq[ORC_MAX_DIM / 2];
    orc_inv_freq(s->rope_theta, d, inv_freq);
    double x[ORC_MAX_DIM], r[ORC_MAX_DIM];
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int stream = 0; stream < 2; ++stream) {
            const void* src = stream == ORC_STREAM_Q ? q : k;
            const int nh = stream == ORC_STREAM_Q ? s->n_q_heads : s->n_kv_heads;
            if (!src) continue;
            for (int h = 0; h < nh; ++h) {
                const int64_t row = (t * nh + h) * (int64_t)d;
                for (int c = 0; c < d; ++c) x[c] = load_elem(src, dtype, row + c);
                orc_rope_row(x, d, s->rope_layout, inv_freq, pos[t], r);
                for (int kk = 0; kk < P; ++kk) {
                    int lo, hi;
                    orc_pair_channels(d, s->rope_layout, kk, &lo, &hi);
                    const double u = r[lo], v = r[hi];
                    const int grp = stream == ORC_STREAM_Q ? q_angle_group(s, h) : k_angle_group(s, h);
                    double* m = moments + (((int64_t)grp * P + kk) * 2 + stream) * ORC_NMOM;
                    m[0] += 1.0;
                    m[1] += u;
                    m[2] += v;
                    m[3] += u * u;
                    m[4] += v * v;
                    m[5] += u * v;
                }
            }
        }
    }
    return 0;
}

/* Closed-form angle ([RAQK] optimisation objective: the shared angle phi*_k that
 * minimises the larger of the two channel variances of the pair).  For a pair
 * with centred covariance [[a, c], [c, b]] rotated by phi,
 *   Var(u') = (a+b)/2 + (a-b)/2 cos 2phi - c sin 2phi,
 *   Var(v') = (a+b)/2 - (a-b)/2 cos 2phi + c sin 2phi,
 * so the larger one is >= (a+b)/2 with equality iff (a-b) cos 2phi = 2c sin 2phi,
 * i.e. 2phi = atan2(a-b, 2c) + n*pi.  The representative in (-pi/4, pi/4] is
 * returned; a degenerate pair (a == b, c == 0, or no samples) gets 0. */
int orc_angles_from_moments(const double* moments, int n_pairs, int estimator,
                            double* phi64, float* phi32, double* abc)
{
    if (!moments || n_pairs < 0) return -1;
    if (estimator < ORC_EST_DEFAULT || estimator > ORC_EST_STREAM_BALANCED) return -1;
    const double quarter_pi = atan(1.0);
    for (int kk = 0; kk < n_pairs; ++kk) {
        const double* mq = moments + ((int64_t)kk * 2 + ORC_STREAM_Q) * ORC_NMOM;
        const double* mk = moments + ((int64_t)kk * 2 + ORC_STREAM_K) * ORC_NMOM;
        double n = 0.0, E[5] = {0, 0, 0, 0, 0}; /* E[u], E[v], E[uu], E[vv], E[uv] */
        int use_q = estimator != ORC_EST_K_ONLY && mq[0] > 0.0;
        int use_k = mk[0] > 0.0;
        if (estimator == ORC_EST_STREAM_BALANCED && use_q && use_k) {
            n = mq[0] + mk[0];
            for (int j = 0; j < 5; ++j) E[j] = 0.5 * (mq[1 + j] / mq[0] + mk[1 + j] / mk[0]);
        } else {
            double S[5] = {0, 0, 0, 0, 0};
            if (use_q) {
                n += mq[0];
                for (int j = 0; j < 5; ++j) S[j] += mq[1 + j];
            }
            if (use_k) {
                n += mk[0];
                for (int j = 0; j < 5; ++j) S[j] += mk[1 + j];
            }
            if (n > 0.0)
                for (int j = 0; j < 5; ++j) E[j] = S[j] / n;
        }
        double phi = 0.0, a = 0.0, b = 0.0, c = 0.0;
        if (n > 0.0) {
            a = E[2] - E[0] * E[0];
            b = E[3] - E[1] * E[1];
            c = E[4] - E[0] * E[1];
            phi = 0.5 * atan2(a - b, 2.0 * c);
            if (phi > quarter_pi) phi -= 2.0 * quarter_pi;
            if (phi <= -quarter_pi) phi += 2.0 * quarter_pi;
        }
        if (phi64) phi64[kk] = phi;
        if (phi32) phi32[kk] = (float)phi;
        if (abc) {
            abc[3 * kk + 0] = a;
            abc[3 * kk + 1] = b;
            abc[3 * kk + 2] = c;
        }
    }
    return 0;
}

/* K-range and relative-error statistics of the support sweep ([RAQK]
 * contributions and results: K range and relative quantisation error versus the
 * block-Hadamard support b).  Dequantised value = code * stored fp16 scale. */
int orc_quant_error_stats(const orc_shape* s, int dtype, const void* k, const int32_t* pos,
                          int64_t n_tokens, const float* angles, int support_b, int group,
                          double* stats)
{
    if (check_shape(s) || n_tokens < 0 || !k || !pos || !stats) return -1;
    const int d = s->head_dim, hk = s->n_kv_heads;
    if (!is_pow2(support_b) || d % support_b) return -1;
    if (group < 2 || (group & 1) || d % group) return -1;
    float inv_freq[ORC_MAX_DIM / 2];
    orc_inv_freq(s->rope_theta, d, inv_freq);
    double E = 0, N = 0, sum_m = 0, max_m = 0, sum_range = 0, n_groups = 0, n_rows = 0;
    double x[ORC_MAX_DIM], y[ORC_MAX_DIM];
    int8_t codes[ORC_MAX_DIM];
    for (int64_t t = 0; t < n_tokens; ++t) {
        for (int h = 0; h < hk; ++h) {
            const int64_t row = (t * hk + h) * (int64_t)d;
            for (int c = 0; c < d; ++c) x[c] = load_elem(k, dtype, row + c);
            orc_transform_row(x, d, s->rope_layout, inv_freq, pos[t], angle_set(angles, k_angle_group(s, h), d),
                              support_b, y);
            for (int j = 0; j < d / group; ++j) {
                const double* yg = y + j * group;
                uint16_t sh;
                orc_quantize_group(yg, group, codes, &sh, NULL);
                const double shv = orc_f16_value(sh);
                double m = 0.0, lo = yg[0], hi = yg[0];
                for (int i = 0; i < group; ++i) {
                    const double yhat = (double)codes[i] * shv;
                    E += (yhat - yg[i]) * (yhat - yg[i]);
                    N += yg[i] * yg[i];
                    if (fabs(yg[i]) > m) m = fabs(yg[i]);
                    if (yg[i] < lo) lo = yg[i];
                    if (yg[i] > hi) hi = yg[i];
                }
                sum_m += m;
                if (m > max_m) max_m = m;
                sum_range += hi - lo;
                n_groups += 1.0;
            }
            n_rows += 1.0;
        }
    }
    stats[0] = E;
    stats[1] = N;
    stats[2] = sum_m;
    stats[3] = max_m;
    stats[4] = sum_range;
    stats[5] = n_groups;
    stats[6] = n_rows;
    stats[7] = 0.0;
    return 0;
}

/* Value of the two's-complement INT4 code held in nibble `which` (0 = low) of a byte. */
static int nibble_code(uint8_t byte, int which)
{
    const int n = which ? (byte >> 4) & 0xF : byte & 0xF;
    return n >= 8 ? n - 16 : n;
}

/* Decode attention logits read from the KV4 cache ([NOTES] section 3.2.1: the
 * head-wise rotation cancels inside Q K^T, so the rotated query against the
 * rotated, quantised key gives the attention logit; [QIFT] introduction: decode
 * reads the KV cache and is memory-bound).  For sequence b, query head h (key
 * head h * Hkv / Hq) and key j < seq_len[b] at slot seq_start[b] + j:
 *   score = sum_c q[b][h][c] * code(slot, kv, c) * s_h(slot, kv, c / g)
 * in fp64.  Keys whose slot lies outside [0, n_slots) give NaN; entries at
 * j >= seq_len[b] (or j >= max_len) are not written. */
int orc_decode_scores(const orc_shape* s, int dtype, const void* q, int64_t n_seqs,
                      const uint8_t* k_codes, const uint16_t* k_scales, int group, int64_t n_slots,
                      const int64_t* seq_start, const int32_t* seq_len, int max_len, double* scores)
{
    if (check_shape(s) || n_seqs < 0 || max_len < 0 || !q || !k_codes || !k_scales || !seq_start || !seq_len ||
        !scores)
        return -1;
    const int d = s->head_dim, hq = s->n_q_heads, hk = s->n_kv_heads;
    if (hq < 1 || hq % hk) return -1;
    if (group < 2 || (group & 1) || d % group) return -1;
    const int ng = d / group;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < n_seqs; ++b) {
        double qv[ORC_MAX_DIM];
        const int len = seq_len[b] < max_len ? seq_len[b] : max_len;
        for (int h = 0; h < hq; ++h) {
            const int kv = (int)((int64_t)h * hk / hq);
            for (int c = 0; c < d; ++c) qv[c] = load_elem(q, dtype, (b * hq + h) * (int64_t)d + c);
            double* out = scores + (b * hq + h) * (int64_t)max_len;
            for (int j = 0; j < len; ++j) {
                const int64_t slot = seq_start[b] + j;
                if (slot < 0 || slot >= n_slots) {
                    out[j] = NAN;
                    continue;
                }
                const uint8_t* row = k_codes + (slot * hk + kv) * (int64_t)(d / 2);
                const uint16_t* srow = k_scales + (slot * hk + kv) * (int64_t)ng;
                double acc = 0.0;
                for (int c = 0; c < d; ++c)
                    acc += qv[c] * (double)nibble_code(row[c / 2], c & 1) * orc_f16_value(srow[c / group]);
                out[j] = acc;
            }
        }
    }
    return 0;
}

/* Threads the token loops above may use (1 without OpenMP). */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads later calls use (n >= 1); returns the previous count. */
int orc_set_threads(int n)
{
    const int prev = orc_max_threads();
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}
