// rrp_calib.hip -- calibration pass: fp64 post-RoPE pair moments pooled over
// heads and tokens, then the closed-form minimax-variance angle per pair.
//
// One angle set shared by all heads (calib_moments_kernel): blocks [0, nbq)
// accumulate the Q stream, blocks [nbq, nbq + nbk) the K stream.  One set per
// key head: calib_sets_kernel below.  A row of head_dim channels is held by P/4
// lanes, each with four
// RoPE pairs (two 8-byte loads for bf16, two 16-byte loads for fp32), so the
// five fp64 sums per pair stay within a few dozen registers.  Each wave walks
// tokens with a fixed stride and keeps the next group of row passes in flight
// while it accumulates the current one.  A wave's row groups are folded with
// lane shuffles, the block's waves through LDS, both in a fixed order; block
// partials go to a scratch array laid out [pair * 5 + sum][column], which one
// wave per (set, stream, pair, sum) reduces in a fixed order -- so the moments
// are bit-identical from run to run.
#include <type_traits>

#include "rrp_device.hpp"
#include "rrp_kernels.hpp"

namespace rrp {

namespace {

constexpr int kNSum = 5;  // sum u, sum v, sum u^2, sum v^2, sum u*v
constexpr int kCP = 4;    // RoPE pairs per lane

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive elements of one row.
template <typename E> struct Quad;
template <> struct Quad<bf16_tag> {
    typedef u32x2 T;
    __device__ static void unpack(const T& w, float (&x)[4]) {
        x[0] = __uint_as_float(w.x << 16);
        x[1] = __uint_as_float(w.x & 0xFFFF0000u);
        x[2] = __uint_as_float(w.y << 16);
        x[3] = __uint_as_float(w.y & 0xFFFF0000u);
    }
    __device__ static T zero() { return T{0u, 0u}; }
};
template <> struct Quad<float> {
    typedef u32x4 T;
    __device__ static void unpack(const T& w, float (&x)[4]) {
        x[0] = __uint_as_float(w.x);
        x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z);
        x[3] = __uint_as_float(w.w);
    }
    __device__ static T zero() { return T{0u, 0u, 0u, 0u}; }
};

// LDS slot of pair k in a token's RoPE table.  A lane reads the four pairs
// 4s .. 4s + 3, so without padding the lanes of an 8-lane (16-lane) access fall
// on 2 (4) distinct 16-byte slot groups; one pad slot after every four pairs
// puts pair 4s + q at 5s + q, distinct modulo 16 for s < 16 (5 is odd).
__device__ __forceinline__ int cslot(int k) { return k + (k >> 2); }
template <int P> constexpr int ctab_slots() { return P + P / 4; }

// MAXP: row passes loaded per step (a step is double-buffered across tokens).
// WHOLE: both streams' head counts are multiples of RP, so every pass holds RP
// rows.  No lane is then masked: a pass's rows sit at offsets fixed per lane
// from a wave-uniform base, and the accumulation needs no row test.
template <typename E, int D, int LAYOUT, int MAXP, bool WHOLE>
__global__ __launch_bounds__(256) void calib_moments_kernel(const CalibArgs a) {
    constexpr int P = D / 2;
    constexpr int LP = P / kCP;  // lanes per row
    constexpr int RP = 64 / LP;  // rows per pass
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr size_t ROWB = (size_t)D * EB;
    using QT = typename Quad<E>::T;
    __shared__ double2 tab_all[4][ctab_slots<P>()];
    __shared__ double red[4][P * kNSum];

    const int lane = (int)__lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwave = (int)(blockDim.x >> 6);
    const int s = lane % LP;
    const int grp = lane / LP;
    double2* tab = tab_all[wave];

    // Blocks come in one run of nbq + nbk per angle set; a set's blocks read only
    // its heads (all heads when the set is shared).
    const int per_set = a.nbq + a.nbk;
    const int set = (int)blockIdx.x / per_set;
    const int local = (int)blockIdx.x % per_set;
    const bool is_k = local >= a.nbq;
    const int bs = is_k ? local - a.nbq : local;
    const int nb = is_k ? a.nbk : a.nbq;
    const unsigned char* src = static_cast<const unsigned char*>(is_k ? a.k : a.q);
    const int nh_all = is_k ? a.hk : a.hq;  // heads per token in the tensor
    const int nh = nh_all / a.n_sets;       // heads of this set
    const int h0 = set * nh;
    const int npass = (nh + RP - 1) / RP;
    const int nstep = (npass + MAXP - 1) / MAXP;
    const float invf = lane_inv_freq(a.inv_freq, lane, P);
    // Element offsets of the lane's two quads: half-split pairs (k, k + P) for
    // k in [4s, 4s + 4); interleaved pairs (2k, 2k + 1) for the same k.
    const int off0 = LAYOUT == 0 ? s * kCP : 2 * s * kCP;
    const int off1 = LAYOUT == 0 ? P + s * kCP : 2 * s * kCP + kCP;

    double acc[kCP][kNSum];
#pragma unroll
    for (int j = 0; j < kCP; ++j)
#pragma unroll
        for (int m = 0; m < kNSum; ++m) acc[j][m] = 0.0;

    const int64_t stride = (int64_t)nb * nwave;
    unsigned loff[MAXP][2];  // WHOLE: byte offsets of the lane's quads in pass i of a step
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
        loff[i][0] = (unsigned)((i * RP + grp) * ROWB + off0 * EB);
        loff[i][1] = (unsigned)((i * RP + grp) * ROWB + off1 * EB);
    }
    auto load_step = [&](int64_t t, int st, QT (&raw)[MAXP][2]) {
        if constexpr (WHOLE) {
            const unsigned char* base = src + ((size_t)t * nh_all + h0 + (size_t)st * MAXP * RP) * ROWB;
#pragma unroll
            for (int i = 0; i < MAXP; ++i) {
                if (st * MAXP + i >= npass) continue;  // uniform
                raw[i][0] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(base + loff[i][0]));
                raw[i][1] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(base + loff[i][1]));
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int row = (st * MAXP + i) * RP + grp;
            if (st * MAXP + i < npass && row < nh) {
                const unsigned char* rp = src + ((size_t)t * nh_all + h0 + row) * ROWB;
                raw[i][0] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(rp + off0 * EB));
                raw[i][1] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(rp + off1 * EB));
            } else {
                raw[i][0] = raw[i][1] = Quad<E>::zero();
            }
        }
    };

    int64_t t = (int64_t)bs * nwave + wave;
    int st = 0;
    QT cur[MAXP][2], nxt[MAXP][2];
    if (t < a.n_tokens) load_step(t, 0, cur);
    // Retire the first step here: inside the loop `cur` is then always a copy
    // made after its wait, and the loop's first use of it needs no wait (which
    // would otherwise also take the next step's prefetch on every iteration).
#pragma unroll
    for (int i = 0; i < MAXP; ++i) asm volatile("" ::"v"(cur[i][0]), "v"(cur[i][1]));
    double c[kCP], sn[kCP];
    while (t < a.n_tokens) {
        int64_t tn = t;
        int sn_step = st + 1;
        if (sn_step == nstep) {
            tn = t + stride;
            sn_step = 0;
        }
        if (tn < a.n_tokens) load_step(tn, sn_step, nxt);
        if (st == 0) {
            const int p = token_pos(a.pos, t);
            wave_lds_sync();  // previous token's table reads are complete
            if (lane < P) {
                double sa, ca;
                sincos_f64_of_f32(rope_angle_f32(p, invf), sa, ca);
                tab[cslot(lane)] = make_double2(ca, sa);
            }
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < kCP; ++j) {
                const double2 v = tab[cslot(s * kCP + j)];
                c[j] = v.x;
                sn[j] = v.y;
            }
        }
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int row = (st * MAXP + i) * RP + grp;
            if (!(st * MAXP + i < npass && (WHOLE || row < nh))) continue;
            float x0[4], x1[4];
            Quad<E>::unpack(cur[i][0], x0);
            Quad<E>::unpack(cur[i][1], x1);
#pragma unroll
            for (int j = 0; j < kCP; ++j) {
                double xa, xb;
                if constexpr (LAYOUT == 0) {
                    xa = x0[j];
                    xb = x1[j];
                } else if (j < kCP / 2) {
                    xa = x0[2 * j];
                    xb = x0[2 * j + 1];
                } else {
                    xa = x1[2 * (j - kCP / 2)];
                    xb = x1[2 * (j - kCP / 2) + 1];
                }
                const double u = xa * c[j] - xb * sn[j];
                const double v = xb * c[j] + xa * sn[j];
                acc[j][0] += u;
                acc[j][1] += v;
                acc[j][2] += u * u;
                acc[j][3] += v * v;
                acc[j][4] += u * v;
            }
        }
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            cur[i][0] = nxt[i][0];
            cur[i][1] = nxt[i][1];
        }
        t = tn;
        st = sn_step;
    }

    // Fold the wave's row groups (lanes s, s + LP, s + 2 LP, ...) in a fixed order.
#pragma unroll
    for (int m = LP; m < 64; m <<= 1)
#pragma unroll
        for (int j = 0; j < kCP; ++j)
#pragma unroll
            for (int q = 0; q < kNSum; ++q) acc[j][q] += shfl_xor_d(acc[j][q], m);
    if (grp == 0) {
#pragma unroll
        for (int j = 0; j < kCP; ++j)
#pragma unroll
            for (int q = 0; q < kNSum; ++q) red[wave][(s * kCP + j) * kNSum + q] = acc[j][q];
    }
    __syncthreads();
    const int nbt = per_set * a.n_sets;
    for (int e = (int)threadIdx.x; e < P * kNSum; e += (int)blockDim.x) {
        double sum = 0.0;
        for (int w = 0; w < nwave; ++w) sum += red[w][e];
        a.partials[(size_t)e * nbt + blockIdx.x] = sum;
    }
}

// Per-key-head angle sets.  A block's kSetWaves waves take kSetWaves sets of one
// stream (wave w: set sg * kSetWaves + w) and walk the same groups of TG tokens:
// the waves build the RoPE tables of the group's tokens into LDS (token j by
// wave j % kSetWaves), so each token's table is built once per block instead of
// once per set, and each wave then reads the rows (token j, head h) of its own
// set, flattened over the group and cut into passes of RP rows.  TG grows with
// fewer heads per set, so that a wave has at least eight passes per group (and
// per pair of barriers around the tables): at d = 128 the Q stream with four
// heads per set takes 8 tokens, the K stream with one head per set 32.  Each wave writes its set's partials to column
// set * (nbq + nbk) + (block's place in the set-group run), the layout
// calib_reduce_kernel reads.
constexpr int kSetWaves = 4;
constexpr int kMaxSetGroup = 32;  // tokens per group, at most (40 KB of tables at d = 128)
constexpr int kSetPasses = 8;     // row passes per wave and group, at least

// Tokens per group of the per-set kernel for a stream with `heads` heads per set
// and `rows_per_pass` rows in a pass (512 / head_dim).
__host__ __device__ inline int set_group_tokens(int heads, int rows_per_pass) {
    int tg = kSetWaves;
    while (tg < kMaxSetGroup && tg * heads < kSetPasses * rows_per_pass) tg *= 2;
    return tg;
}

// WHOLE: for both streams the heads per set divide the rows per pass, or the
// rows per pass divide them, and every token group is full.  A pass then
// starts at a row whose (token, head) is the same for every lane up to a
// per-lane constant: the rows are loaded from a wave-uniform base (a scalar
// cursor) plus fixed per-lane offsets, with no row test.
template <typename E, int D, int LAYOUT, int MAXP, bool WHOLE>
__global__ __launch_bounds__(64 * kSetWaves)
__attribute__((amdgpu_waves_per_eu(std::is_same<E, bf16_tag>::value ? 4 : 1)))  // bf16 fits 128 VGPRs
void calib_sets_kernel(const CalibArgs a) {
    constexpr int P = D / 2;
    constexpr int LP = P / kCP;  // lanes per row
    constexpr int RP = 64 / LP;  // rows per pass
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr size_t ROWB = (size_t)D * EB;
    using QT = typename Quad<E>::T;
    __shared__ double2 tab[kMaxSetGroup][ctab_slots<P>()];

    const int lane = (int)__lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int s = lane % LP;
    const int grp = lane / LP;

    // Neighbouring blocks take the same tokens for different set-groups, so the
    // rows of a token (every head) are read at about the same time.
    const int per_set = a.nbq + a.nbk;
    const int n_sg = (a.n_sets + kSetWaves - 1) / kSetWaves;
    const int sg = (int)blockIdx.x % n_sg;
    const int local = (int)blockIdx.x / n_sg;
    const bool is_k = local >= a.nbq;
    const int bs = is_k ? local - a.nbq : local;
    const int nb = is_k ? a.nbk : a.nbq;
    const int set = sg * kSetWaves + wave;
    const bool active = set < a.n_sets;  // waves past the last set still build tables
    const unsigned char* src = static_cast<const unsigned char*>(is_k ? a.k : a.q);
    const int nh_all = is_k ? a.hk : a.hq;
    const int g = nh_all / a.n_sets;  // heads per set
    const int h0 = set * g;
    const int tg = set_group_tokens(g, RP);  // tokens per group (uniform per block)
    const int nrows = tg * g;                // rows per token group
    const int npass = (nrows + RP - 1) / RP;
    const int nstep = (npass + MAXP - 1) / MAXP;
    const float invf = lane_inv_freq(a.inv_freq, lane, P);
    const int off0 = LAYOUT == 0 ? s * kCP : 2 * s * kCP;
    const int off1 = LAYOUT == 0 ? P + s * kCP : 2 * s * kCP + kCP;

    double acc[kCP][kNSum];
#pragma unroll
    for (int j = 0; j < kCP; ++j)
#pragma unroll
        for (int m = 0; m < kNSum; ++m) acc[j][m] = 0.0;

    // Token groups bs, bs + nb, ...: tokens tg * group + j.  A group's rows are
    // r = j * g + h (token j of the group, head h0 + h of the set) and the lane
    // takes r = pass * RP + grp; (j, h) is walked pass by pass with no division
    // (RP = qrp * g + rrp), and each loaded pass carries its j (-1: no row).
    const int64_t n_groups = (a.n_tokens + tg - 1) / tg;
    const int qrp = RP / g, rrp = RP % g;
    const int j_first = grp / g, h_first = grp % g;
    int lj = j_first, lh = h_first;  // the next pass to load
    int uj = 0, uh = 0;              // WHOLE: the same for the pass's first row (wave-uniform)
    const unsigned lconst0 = (unsigned)((j_first * nh_all + h_first) * ROWB + off0 * EB);
    const unsigned lconst1 = (unsigned)((j_first * nh_all + h_first) * ROWB + off1 * EB);
    auto load_step = [&](int64_t grp_t, int st, QT (&raw)[MAXP][2], int (&rj)[MAXP]) {
        if (st == 0) {
            lj = j_first;
            lh = h_first;
            uj = uh = 0;
        }
        const unsigned char* gbase = src + ((size_t)grp_t * tg * nh_all + h0) * ROWB;
        const int64_t tleft = a.n_tokens - grp_t * tg;  // tokens of the group that exist
        if constexpr (WHOLE) {
#pragma unroll
            for (int i = 0; i < MAXP; ++i) {
                if (active && st * MAXP + i < npass) {  // uniform
                    const unsigned char* pb = gbase + (size_t)(uj * nh_all + uh) * ROWB;
                    raw[i][0] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(pb + lconst0));
                    raw[i][1] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(pb + lconst1));
                    rj[i] = uj + j_first;
                } else {
                    rj[i] = -1;
                }
                uh += rrp;
                uj += qrp;
                if (uh >= g) {
                    uh -= g;
                    ++uj;
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const bool ok = active && lj < tg && lj < tleft;
            rj[i] = ok ? lj : -1;
            if (ok) {
                const unsigned char* rp = gbase + (size_t)(lj * nh_all + lh) * ROWB;
                raw[i][0] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(rp + off0 * EB));
                raw[i][1] = __builtin_nontemporal_load(reinterpret_cast<const QT*>(rp + off1 * EB));
            } else {
                raw[i][0] = raw[i][1] = Quad<E>::zero();
            }
            lh += rrp;
            lj += qrp;
            if (lh >= g) {
                lh -= g;
                ++lj;
            }
        }
    };

    int64_t gt = bs;
    int st = 0;
    QT cur[MAXP][2], nxt[MAXP][2];
    int cj[MAXP], nj[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) cj[i] = nj[i] = -1;
    if (gt < n_groups) load_step(gt, 0, cur, cj);
    // Retire the first step here: inside the loop `cur` is then always a copy
    // made after its wait, and the loop's first use of it needs no wait (which
    // would otherwise also take the next step's prefetch on every iteration).
#pragma unroll
    for (int i = 0; i < MAXP; ++i) asm volatile("" ::"v"(cur[i][0]), "v"(cur[i][1]));
    while (gt < n_groups) {
        int64_t gn = gt;
        int sn_step = st + 1;
        if (sn_step == nstep) {
            gn = gt + nb;
            sn_step = 0;
        }
        if (gn < n_groups) load_step(gn, sn_step, nxt, nj);
        if (st == 0) {
            __syncthreads();  // the previous group's table reads are complete
            for (int jj = wave; jj < tg; jj += kSetWaves) {
                const int64_t t = gt * tg + jj;
                if (lane < P && t < a.n_tokens) {
                    double sa, ca;
                    sincos_f64_of_f32(rope_angle_f32(token_pos(a.pos, t), invf), sa, ca);
                    tab[jj][cslot(lane)] = make_double2(ca, sa);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            const int j = cj[i];  // token of the row inside the group
            if (j < 0) continue;
            float x0[4], x1[4];
            Quad<E>::unpack(cur[i][0], x0);
            Quad<E>::unpack(cur[i][1], x1);
#pragma unroll
            for (int q = 0; q < kCP; ++q) {
                const double2 cs = tab[j][cslot(s * kCP + q)];
                double xa, xb;
                if constexpr (LAYOUT == 0) {
                    xa = x0[q];
                    xb = x1[q];
                } else if (q < kCP / 2) {
                    xa = x0[2 * q];
                    xb = x0[2 * q + 1];
                } else {
                    xa = x1[2 * (q - kCP / 2)];
                    xb = x1[2 * (q - kCP / 2) + 1];
                }
                const double u = xa * cs.x - xb * cs.y;
                const double v = xb * cs.x + xa * cs.y;
                acc[q][0] += u;
                acc[q][1] += v;
                acc[q][2] += u * u;
                acc[q][3] += v * v;
                acc[q][4] += u * v;
            }
        }
#pragma unroll
        for (int i = 0; i < MAXP; ++i) {
            cur[i][0] = nxt[i][0];
            cur[i][1] = nxt[i][1];
            cj[i] = nj[i];
        }
        gt = gn;
        st = sn_step;
    }

    // Fold the wave's row groups in a fixed order; the row-group-0 lanes write
    // their four pairs' sums to this set's column.
#pragma unroll
    for (int m = LP; m < 64; m <<= 1)
#pragma unroll
        for (int j = 0; j < kCP; ++j)
#pragma unroll
            for (int q = 0; q < kNSum; ++q) acc[j][q] += shfl_xor_d(acc[j][q], m);
    if (active && grp == 0) {
        const int nbt = per_set * a.n_sets;
        const size_t col = (size_t)set * per_set + local;
#pragma unroll
        for (int j = 0; j < kCP; ++j)
#pragma unroll
            for (int q = 0; q < kNSum; ++q) a.partials[(size_t)((s * kCP + j) * kNSum + q) * nbt + col] = acc[j][q];
    }
}

// One wave per (set, stream, pair, sum): lane l adds the partials of the set's
// stream blocks l, l + 64, ... in order, then the wave folds its lanes with a
// fixed xor butterfly (every lane ends with the same value), and lane 0 adds it
// to the caller's moments.
__global__ __launch_bounds__(256) void calib_reduce_kernel(const CalibFinalArgs a) {
    const int P = a.n_pairs;
    const int w = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (w >= a.n_sets * 2 * P * kNSum) return;  // uniform per wave
    const int lane = (int)__lane_id();
    const int set = w / (2 * P * kNSum);
    const int rem = w % (2 * P * kNSum);
    const int stream = rem / (P * kNSum);
    const int e = rem % (P * kNSum);  // pair * 5 + sum
    const int k = e / kNSum, j = e % kNSum;
    const int per_set = a.nbq + a.nbk;
    const int b0 = set * per_set + (stream ? a.nbq : 0);
    const int nb = stream ? a.nbk : a.nbq;
    if (nb == 0) return;  // stream not accumulated by this call
    const int nbt = per_set * a.n_sets;
    const double* part = a.partials + (size_t)e * nbt + b0;
    double sum = 0.0;
    for (int b = lane; b < nb; b += 64) sum += part[b];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += shfl_xor_d(sum, m);
    if (lane == 0) {
        double* mom = a.moments + (((size_t)set * P + k) * 2 + stream) * 6;
        mom[1 + j] += sum;
        if (j == 0) mom[0] += stream ? a.n_rows_k : a.n_rows_q;
    }
}

// One thread per (set, pair): estimator, centred covariance, phi* wrapped to
// (-pi/4, pi/4].
__global__ __launch_bounds__(512) void calib_angles_kernel(const CalibFinalArgs a) {
    const int k = (int)threadIdx.x;  // set * P + pair
    if (k >= a.n_sets * a.n_pairs) return;
    const double* mq = a.moments + (size_t)k * 12;
    const double* mk = mq + 6;
    const bool use_q = a.estimator != 1 && mq[0] > 0.0;
    const bool use_k = mk[0] > 0.0;
    double n = 0.0, E[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    if (a.estimator == 2 && use_q && use_k) {
        n = mq[0] + mk[0];
        for (int j = 0; j < 5; ++j) E[j] = 0.5 * (mq[1 + j] / mq[0] + mk[1 + j] / mk[0]);
    } else {
        double S[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
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
    double phi = 0.0;
    if (n > 0.0) {
        const double av = E[2] - E[0] * E[0];
        const double bv = E[3] - E[1] * E[1];
        const double cv = E[4] - E[0] * E[1];
        const double quarter_pi = 0.78539816339744830962;
        phi = 0.5 * atan2(av - bv, 2.0 * cv);
        if (phi > quarter_pi) phi -= 2.0 * quarter_pi;
        if (phi <= -quarter_pi) phi += 2.0 * quarter_pi;
    }
    a.angles_out[k] = (float)phi;
}

// Row passes of a stream kept in flight per wave (the next step's rows are
// loaded while the current step is accumulated).
constexpr int kCalibMaxPasses = 2;

template <typename E, int D, int LAYOUT>
hipError_t launch_t(const CalibArgs& a, hipStream_t st) {
    if (a.n_sets > 1) {
        const int groups = (a.n_sets + kSetWaves - 1) / kSetWaves;
        const int blocks = (a.nbq + a.nbk) * groups;
        constexpr int RP = 64 / (D / 2 / kCP);  // rows per pass
        auto aligned_heads = [&](int heads) {
            const int g = heads / a.n_sets;
            return g > 0 && (RP % g == 0 || g % RP == 0) && set_group_tokens(g, RP) * g % RP == 0;
        };
        auto full_groups = [&](int heads) { return a.n_tokens % set_group_tokens(heads / a.n_sets, RP) == 0; };
        if ((a.nbq == 0 || (aligned_heads(a.hq) && full_groups(a.hq))) && aligned_heads(a.hk) && full_groups(a.hk))
            hipLaunchKernelGGL((calib_sets_kernel<E, D, LAYOUT, kCalibMaxPasses, true>), dim3(blocks),
                               dim3(64 * kSetWaves), 0, st, a);
        else
            hipLaunchKernelGGL((calib_sets_kernel<E, D, LAYOUT, kCalibMaxPasses, false>), dim3(blocks),
                               dim3(64 * kSetWaves), 0, st, a);
        return hipGetLastError();
    }
    const int blocks = a.nbq + a.nbk;
    constexpr int RP = 64 / (D / 2 / kCP);  // rows per pass
    if ((a.nbq == 0 || a.hq % RP == 0) && a.hk % RP == 0)
        hipLaunchKernelGGL((calib_moments_kernel<E, D, LAYOUT, kCalibMaxPasses, true>), dim3(blocks), dim3(256), 0,
                           st, a);
    else
        hipLaunchKernelGGL((calib_moments_kernel<E, D, LAYOUT, kCalibMaxPasses, false>), dim3(blocks), dim3(256), 0,
                           st, a);
    return hipGetLastError();
}

}  // namespace

// Cost of one token's RoPE table build, counted in row passes, when a set's
// blocks are split between the Q and K streams by work rather than by rows.
constexpr int kCalibTableWeight = 2;

int calib_blocks(int64_t n_tokens, bool with_q, int hq, int hk, int head_dim, int n_sets, int* nbq, int* nbk) {
    // One shared set: one block per 128 tokens for both streams together, so a
    // wave walks 32 tokens with K only and more with Q (the streams share the
    // blocks by work); measured best against 32 to 512 tokens per block, since
    // shorter waves spend more on starting up and on writing partials.  Per-set
    // calibration: about 8 tokens per wave per stream.  At most kMaxCalibBlocks partial columns over
    // all sets.  The streams share a set's blocks in proportion to their work
    // per token (per token group for per-set calibration): the row passes plus
    // the table (worth about kCalibTableWeight passes).
    int64_t want = n_sets == 1 ? (n_tokens + 127) / 128 : (n_tokens * (with_q ? 2 : 1) + 31) / 32;
    if (want > kMaxCalibBlocks) want = kMaxCalibBlocks;
    want /= n_sets;  // per set (so all sets together stay within kMaxCalibBlocks)
    if (want < (with_q ? 2 : 1)) want = with_q ? 2 : 1;
    const int total = (int)want;
    if (!with_q || hq == 0) {
        *nbq = 0;
        *nbk = total;
    } else {
        // Work per token: row passes plus tables.  One shared set: a wave's passes
        // of one token and its table.  Per-set kernel: a wave's passes of a group
        // of tg tokens and its tg / kSetWaves tables, over tg.
        const int rp = 512 / head_dim;  // rows per pass
        auto work = [&](int heads) {
            if (n_sets == 1) return (double)((heads + rp - 1) / rp + kCalibTableWeight);
            const int g = heads / n_sets, tg = set_group_tokens(g, rp);
            return ((double)((tg * g + rp - 1) / rp) + (double)kCalibTableWeight * tg / kSetWaves) / tg;
        };
        const double wq = work(hq), wk = work(hk);
        int q = (int)((double)total * wq / (wq + wk));
        if (q < 1) q = 1;
        if (q > total - 1) q = total - 1;
        *nbq = q;
        *nbk = total - q;
    }
    return (*nbq + *nbk) * n_sets;
}

hipError_t launch_calibrate(const CalibArgs& a, int dtype, int head_dim, int layout, hipStream_t st) {
#define RRP_DISPATCH(E, D, LY) \
    if (head_dim == D && layout == LY) return launch_t<E, D, LY>(a, st);
    if (dtype == 1) {
        RRP_DISPATCH(bf16_tag, 64, 0) RRP_DISPATCH(bf16_tag, 64, 1)
        RRP_DISPATCH(bf16_tag, 128, 0) RRP_DISPATCH(bf16_tag, 128, 1)
    } else {
        RRP_DISPATCH(float, 64, 0) RRP_DISPATCH(float, 64, 1)
        RRP_DISPATCH(float, 128, 0) RRP_DISPATCH(float, 128, 1)
    }
#undef RRP_DISPATCH
    return hipErrorInvalidValue;
}

hipError_t launch_calibrate_final(const CalibFinalArgs& a, hipStream_t st) {
    if (a.nbq + a.nbk > 0) {
        const int waves = a.n_sets * 2 * a.n_pairs * kNSum;
        hipLaunchKernelGGL(calib_reduce_kernel, dim3((waves + 3) / 4), dim3(256), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.angles_out == nullptr) return hipSuccess;
    const int threads = ((a.n_sets * a.n_pairs + 63) / 64) * 64;
    hipLaunchKernelGGL(calib_angles_kernel, dim3(1), dim3(threads), 0, st, a);
    return hipGetLastError();
}

}  // namespace rrp
