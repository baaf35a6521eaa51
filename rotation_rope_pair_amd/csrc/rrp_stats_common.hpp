// rrp_stats_common.hpp -- device pieces shared by the diagnostic kernels
// (rrp_stats.hip: one support b; rrp_sweep.hpp: every support b = 1 .. head_dim
// in one launch).
//
// Every K row is rotated with the hot path's fp64 tables (RoPE + R_phi),
// Hadamard-transformed in fp64, quantised with its group's stored fp16 scale
// (fp32(m / 7) rounded to fp16, saturated), dequantised, and the lane adds
// (yhat - y)^2 and y^2 in fp64; the lanes holding a group share its absmax,
// the max of those and (max - min) evenly.  Wave, block and grid reductions run
// in a fixed order (bit-reproducible).
#pragma once
#include "rrp_device.hpp"
#include "rrp_kernels.hpp"

namespace rrp {

// The sweep's launchers, one per element type (rrp_sweep_bf16.hip, rrp_sweep_f32.hip).
hipError_t launch_sweep_bf16(const StatsArgs& a, int n_blocks, int head_dim, int layout, hipStream_t st);
hipError_t launch_sweep_f32(const StatsArgs& a, int n_blocks, int head_dim, int layout, hipStream_t st);

namespace {

constexpr int kNStat = 5;  // E, N, sum absmax, max absmax, sum range

// Per-lane running sums of one support's statistics.
struct StatAcc {
    double E = 0.0, N = 0.0, M = 0.0, maxM = 0.0, R = 0.0;
};

// Keeps the sums' updates where they are written: without it the compiler sinks
// them past the rare correction pass to the loop's end, holding every operand
// live (and spilled) across it.
__device__ __forceinline__ void pin(StatAcc& a) {
    asm volatile("" : "+v"(a.E), "+v"(a.N), "+v"(a.M), "+v"(a.maxM), "+v"(a.R));
}

// Fold the wave's lanes (fixed xor order), then the block's waves through LDS,
// and write the block's partials of statistic set `set` to partials laid out
// [set * 5 + statistic][block].  Called by every thread of the block.
__device__ __forceinline__ void block_stats_partials(StatAcc acc, int set, double (*red)[kNStat], double* partials) {
    const int lane = (int)__lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const int nwave = (int)(blockDim.x >> 6);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        acc.E += shfl_xor_d(acc.E, m);
        acc.N += shfl_xor_d(acc.N, m);
        acc.M += shfl_xor_d(acc.M, m);
        acc.maxM = fmax(acc.maxM, shfl_xor_d(acc.maxM, m));
        acc.R += shfl_xor_d(acc.R, m);
    }
    __syncthreads();  // red is free (a previous set's reads are done)
    if (lane == 0) {
        red[wave][0] = acc.E;
        red[wave][1] = acc.N;
        red[wave][2] = acc.M;
        red[wave][3] = acc.maxM;
        red[wave][4] = acc.R;
    }
    __syncthreads();
    if (threadIdx.x < kNStat) {
        const int e = (int)threadIdx.x;
        double v = red[0][e];
        for (int w = 1; w < nwave; ++w) v = (e == 3) ? fmax(v, red[w][e]) : v + red[w][e];
        partials[(size_t)(set * kNStat + e) * gridDim.x + blockIdx.x] = v;
    }
}

// ---------------------------------------------------------------------------
// Single-support diagnostics (stats_kernel).  The pass is bound by fp64 VALU
// issue, so it is laid out to issue as few instructions per element as
// possible.
//
// A lane holds 16 channels of a K row, whatever the element type: the runs of
// 8 at position s in both halves of the head,
//   x[ch][i] = y[ch * D/2 + s * 8 + i]   (ch < 2, i < 8),
// so L = D / 16 lanes hold a row and a wave holds R = 64 / L rows (a pass).
// The butterflies on the channel bits of i and on the half bit are
// in-register.  Those on the bits of s follow a transposition of the pass
// through LDS, after which the lane at position s' holds, for every run
// position u < L and both halves, the K8 = 8 / L channels i = s' * K8 + ii:
//   t[ch * 8 + u * K8 + ii] = y[ch * D/2 + u * 8 + s' * K8 + ii],
// so those butterflies are in-register too: the transform has no cross-lane
// moves.  Groups are then reduced in-lane over the runs of BIN consecutive
// entries they cover, and across the lanes (position bits `xmask`) that share
// them.
// ---------------------------------------------------------------------------
template <int D> struct SGeo {
    static constexpr int P = D / 2;
    static constexpr int L = D / 16;               // lanes per row
    static constexpr int R = 64 / L;               // rows per pass
    static constexpr int K8 = 8 / L;               // run offsets per lane after the transposition
    static constexpr int SLOTS = 576;              // 16-byte LDS slots of a pass's transposition (see tslot)
};

// 16-byte LDS slot holding channels (u * 8 + i, D/2 + u * 8 + i) of pass row r.
// A 16-byte access is served eight lanes (128 bytes) at a time, 16 lanes per
// 256-byte bank row; in every access of either direction of the transposition
// those lanes fall on different slots modulo 8 and modulo 16 (no bank
// conflict).  For D = 128 the two rows of a pair interleave (even and odd
// slots) and one side of the slot index is the lane's, the other a
// compile-time offset; for D = 64 the run position is xor-ed with the offset.
template <int D>
__device__ __forceinline__ int tslot(int r, int i, int u) {
    if constexpr (D == 128) return 142 * (r >> 1) + (r & 1) + 2 * i + 18 * u;
    else return 36 * r + 4 * i + (u ^ ((i >> 1) & 3));
}

// x (natural layout of lane (r, s)) -> t (transposed layout of the same lane).
template <int D>
__device__ __forceinline__ void transpose_in(double2* tb, int r, int s, const double (&x)[2][8], double (&t)[16]) {
    constexpr int L = SGeo<D>::L, K8 = SGeo<D>::K8;
#pragma unroll
    for (int i = 0; i < 8; ++i) tb[tslot<D>(r, i, s)] = make_double2(x[0][i], x[1][i]);
    wave_lds_sync();
#pragma unroll
    for (int ii = 0; ii < K8; ++ii)
#pragma unroll
        for (int u = 0; u < L; ++u) {
            const double2 v = tb[tslot<D>(r, s * K8 + ii, u)];
            t[u * K8 + ii] = v.x;
            t[8 + u * K8 + ii] = v.y;
        }
}

// The inverse: t (transposed) -> x (natural), through the same slots.
template <int D>
__device__ __forceinline__ void transpose_out(double2* tb, int r, int s, const double (&t)[16], double (&x)[2][8]) {
    constexpr int L = SGeo<D>::L, K8 = SGeo<D>::K8;
#pragma unroll
    for (int ii = 0; ii < K8; ++ii)
#pragma unroll
        for (int u = 0; u < L; ++u)
            tb[tslot<D>(r, s * K8 + ii, u)] = make_double2(t[u * K8 + ii], t[8 + u * K8 + ii]);
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double2 v = tb[tslot<D>(r, i, s)];
        x[0][i] = v.x;
        x[1][i] = v.y;
    }
}

// Butterflies on the bits of the run position (transposed layout), for the
// supports that reach them: bit h of u is channel bit 3 + log2(h).
template <int D>
__device__ __forceinline__ void fwht_runs(double (&t)[16], int b) {
    constexpr int L = SGeo<D>::L, K8 = SGeo<D>::K8;
#pragma unroll
    for (int h = 1; h < L; h <<= 1) {
        if (b > 8 * h) {
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int u = 0; u < L; ++u)
                    if ((u & h) == 0)
#pragma unroll
                        for (int ii = 0; ii < K8; ++ii) {
                            const int e0 = ch * 8 + u * K8 + ii, e1 = e0 + h * K8;
                            const double p = t[e0], q = t[e1];
                            t[e0] = p + q;
                            t[e1] = p - q;
                        }
        }
    }
}

// The stored scale of a group with absmax m, and 1 / that scale.
struct GScale {
    double shv;  // fp16(fp32(m / 7)) nearest-even, saturated at 65504, as a double
    double rcp;  // 1 / shv (0 when shv == 0: all codes 0)
};

__device__ __forceinline__ GScale group_scale(double m) {
    // m * (1/7) corrected once by the exact residual m - 7 q is the correctly
    // rounded m / 7 (the nearest reciprocal of 7 and one fused correction
    // step), so rounding it to fp32 gives fp32(m / 7) with no division.
    constexpr double kSeventh = 1.0 / 7.0;
    const double q0 = m * kSeventh;
    const double q = fma(fma(-7.0, q0, m), kSeventh, q0);
    GScale gs;
    gs.shv = (double)f16_bits_to_f32(f16_sat_bits((float)q));
    // hardware reciprocal, then two Newton steps: within an ulp of 1 / shv
    double rc = __builtin_amdgcn_rcp(gs.shv);
    rc = fma(fma(-gs.shv, rc, 1.0), rc, rc);
    rc = fma(fma(-gs.shv, rc, 1.0), rc, rc);
    gs.rcp = gs.shv > 0.0 ? rc : 0.0;
    return gs;
}

// Statistics of the lane's 16 entries t (any layout): groups are the runs of
// BIN consecutive entries, completed across the lanes whose position differs
// in the bits of xmask (each such lane adds w = 1 / (lanes per group) of the
// group-level sums).  Quantise with the stored scale, dequantise, add
// (yhat - y)^2, y^2, the group absmax, its max and (max - min).  Zero entries
// (rows past the last head) add nothing.
// Codes are taken as round(y / s_h) with no clamp to +-7: that is exact unless
// the scale saturated or is a coarse fp16 subnormal, in which case `far` is
// set.  FIX (the rare second pass over the same rows): add only the change of
// (yhat - y)^2 from clamping the codes.
// SCALED: t holds u = sqrt(b) y, the transform without its 1 / sqrt(b)
// (cb = 1 / sqrt(b), sb = sqrt(b)); the group's scale is taken from its y
// absmax, and the lane adds b (yhat - y)^2 and the u-values' absmax and range
// (sqrt(b) times y's), but no y^2 (the caller takes the energy once).
template <int BIN, int L, bool SCALED, bool FIX>
__device__ __forceinline__ void group_stats(const double (&t)[16], int xmask, double w, StatAcc& acc, bool& far,
                                            double cb = 1.0, double sb = 1.0) {
    constexpr int NG = 16 / BIN;           // groups of the lane
    constexpr int NB = NG < 4 ? NG : 4;    // groups handled at once (bounds the live registers)
#pragma unroll
    for (int g0 = 0; g0 < NG; g0 += NB) {
        double mx[NB], mn[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int v0 = (g0 + q) * BIN;
            if constexpr (BIN == 1) {
                mx[q] = t[v0];
                mn[q] = t[v0];
            } else {
                double hi[BIN / 2], lo[BIN / 2];
#pragma unroll
                for (int k = 0; k < BIN / 2; ++k) {
                    hi[k] = fmax(t[v0 + 2 * k], t[v0 + 2 * k + 1]);
                    lo[k] = fmin(t[v0 + 2 * k], t[v0 + 2 * k + 1]);
                }
#pragma unroll
                for (int n = BIN / 4; n >= 1; n >>= 1)
#pragma unroll
                    for (int k = 0; k < n; ++k) {
                        hi[k] = fmax(hi[k], hi[k + n]);
                        lo[k] = fmin(lo[k], lo[k + n]);
                    }
                mx[q] = hi[0];
                mn[q] = lo[0];
            }
        }
        if constexpr (L > 1) {
            if (xmask & 1) {
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    mx[q] = fmax(mx[q], s_xor<L, 1>(mx[q]));
                    mn[q] = fmin(mn[q], s_xor<L, 1>(mn[q]));
                }
            }
        }
        if constexpr (L > 2) {
            if (xmask & 2) {
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    mx[q] = fmax(mx[q], s_xor<L, 2>(mx[q]));
                    mn[q] = fmin(mn[q], s_xor<L, 2>(mn[q]));
                }
            }
        }
        if constexpr (L > 4) {
            if (xmask & 4) {
#pragma unroll
                for (int q = 0; q < NB; ++q) {
                    mx[q] = fmax(mx[q], s_xor<L, 4>(mx[q]));
                    mn[q] = fmin(mn[q], s_xor<L, 4>(mn[q]));
                }
            }
        }
        double shv[NB], rcp[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const double m = fmax(mx[q], -mn[q]);
            const GScale gs = group_scale(SCALED ? m * cb : m);
            shv[q] = SCALED ? gs.shv * sb : gs.shv;
            rcp[q] = SCALED ? gs.rcp * cb : gs.rcp;
            if constexpr (!FIX) {
                acc.M = fma(m, w, acc.M);
                acc.maxM = fmax(acc.maxM, m);
                acc.R = fma(mx[q] - mn[q], w, acc.R);
                far = far || m * rcp[q] > 7.49;  // a code could round past +-7
            }
        }
#pragma unroll
        for (int q = 0; q < NB; ++q)
#pragma unroll
            for (int k = 0; k < BIN; ++k) {
                const double y = t[(g0 + q) * BIN + k];
                if constexpr (!FIX) {
                    const double d = fma(rint(y * rcp[q]), shv[q], -y);
                    acc.E = fma(d, d, acc.E);
                    if constexpr (!SCALED) acc.N = fma(y, y, acc.N);
                } else {
                    const double c = rint(y * rcp[q]);
                    const double d0 = fma(c, shv[q], -y);
                    const double d1 = fma(fmin(fmax(c, -7.0), 7.0), shv[q], -y);
                    acc.E += fabs(c) > 7.0 ? d1 * d1 - d0 * d0 : 0.0;
                }
            }
    }
}

// One table entry: (C, S) = (cos, sin)(alpha + phi) / sqrt(b) composed by
// products of the fp64 (cos, sin) of alpha (ca, sa) and of phi (cp, sp), or
// (C + S, C - S) with the half butterfly folded in (FOLD).  Written with
// explicit fused operations so that every caller gets the same doubles (the
// shared-set table and the per-set composition below).
template <bool FOLD>
__device__ __forceinline__ double2 compose_entry(double ca, double sa, double cp, double sp, double rs) {
    const double C = fma(ca, cp, -(sa * sp)) * rs;
    const double S = fma(sa, cp, ca * sp) * rs;
    return FOLD ? make_double2(C + S, C - S) : make_double2(C, S);
}

// The token's fp64 table of the shared angle set: entry of pair k at
// tab_index(k) (compose_entry of the pair's RoPE angle and phi_k).  With one
// angle set per key head the table holds the bare RoPE (cos, sin) instead
// (cphi = 1, sphi = 0, rs = 1, no fold), composed per row (rotate_sets).
template <int D, bool FOLD>
__device__ __forceinline__ void token_table64(double2* tab, int lane, int p, float invf, double cphi, double sphi,
                                              double rs) {
    constexpr int P = D / 2;
    wave_lds_sync();  // the previous token's table reads are complete
    if (lane < P) {
        double sa, ca;
        sincos_f64_of_f32(rope_angle_f32(p, invf), sa, ca);
        tab[tab_index(lane)] = compose_entry<FOLD>(ca, sa, cphi, sphi, rs);
    }
    wave_lds_sync();
}

// One pair (a, b) turned by a table entry e, with explicit fused operations
// (so the shared-set and the per-set paths give the same doubles):
// (a C - b S, b C + a S), or (a U + b V, a V - b U) with the half butterfly
// folded in.
template <bool FOLD>
__device__ __forceinline__ void turn_pair(double& a, double& b, double2 e) {
    const double a0 = a, b0 = b;
    if constexpr (FOLD) {
        a = fma(a0, e.x, b0 * e.y);
        b = fma(a0, e.y, -(b0 * e.x));
    } else {
        a = fma(a0, e.x, -(b0 * e.y));
        b = fma(b0, e.x, a0 * e.y);
    }
}

// The two channels of pair slot j of a lane (see pair_index_of_lane).
template <int LAYOUT>
__device__ __forceinline__ void pair_slots(double (&x)[2][8], int j, double*& pa, double*& pb) {
    if constexpr (LAYOUT == 0) {
        pa = &x[0][j];
        pb = &x[1][j];
    } else {
        pa = &x[j / 4][2 * (j % 4)];
        pb = pa + 1;
    }
}

// RoPE + R_phi of the lane's pairs from the token's composed table (shared
// angle set): entry kidx[j] for pair slot j.
template <int LAYOUT, bool FOLD>
__device__ __forceinline__ void rotate_tab(double (&x)[2][8], const double2* tab, const int (&kidx)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        double* pa;
        double* pb;
        pair_slots<LAYOUT>(x, j, pa, pb);
        turn_pair<FOLD>(*pa, *pb, tab[kidx[j]]);
    }
}

// RoPE + R_phi of the lane's pairs with one angle set per key head: the bare
// RoPE (cos, sin) of pair kidx[j] from the token's table, composed with the
// row's set angles (cos, sin)(phi) held in registers (cs_phi[j]), exactly as
// the shared-set table composes them.
template <int LAYOUT, bool FOLD>
__device__ __forceinline__ void rotate_sets(double (&x)[2][8], const double2* tab, const int (&kidx)[8],
                                            const double2 (&cs_phi)[8], double rs) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double2 ra = tab[kidx[j]];
        double* pa;
        double* pb;
        pair_slots<LAYOUT>(x, j, pa, pb);
        turn_pair<FOLD>(*pa, *pb, compose_entry<FOLD>(ra.x, ra.y, cs_phi[j].x, cs_phi[j].y, rs));
    }
}

// The same with the row's set angles read from the block's table phi (entry
// (k, set) at k * kSetStride + set): phirow = phi + (the lane's first pair) *
// kSetStride + set, and pair slot j sits a compile-time offset further.
template <int D, int LAYOUT, bool FOLD>
__device__ __forceinline__ void rotate_sets_lds(double (&x)[2][8], const double2* tab, const int (&kidx)[8],
                                                const double2* phirow, double rs) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        constexpr int Q = D / 4;
        const int dk = LAYOUT == 0 ? j : (j / 4) * Q + (j % 4);  // pair of slot j minus the lane's first pair
        const double2 ra = tab[kidx[j]];
        const double2 ph = phirow[dk * kSetStride];
        double* pa;
        double* pb;
        pair_slots<LAYOUT>(x, j, pa, pb);
        turn_pair<FOLD>(*pa, *pb, compose_entry<FOLD>(ra.x, ra.y, ph.x, ph.y, rs));
    }
}

template <bool B> struct BoolC {
    static constexpr bool value = B;
};

template <typename E> struct SRow;
template <> struct SRow<bf16_tag> {
    static constexpr int NR = 2;  // 16-byte loads per lane and row
    template <int D>
    __device__ static void load(const unsigned char* row, int s, u32x4 (&raw)[NR]) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
            raw[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + (ch * (D / 2) + s * 8) * 2));
    }
    __device__ static void unpack(const u32x4 (&raw)[NR], double (&x)[2][8]) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            float f[8];
            unpack_chunk<bf16_tag, 8>(raw[ch], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[ch][i] = (double)f[i];
        }
    }
};
template <> struct SRow<float> {
    static constexpr int NR = 4;
    template <int D>
    __device__ static void load(const unsigned char* row, int s, u32x4 (&raw)[NR]) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                raw[2 * ch + h] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(row + (ch * (D / 2) + s * 8 + 4 * h) * 4));
    }
    __device__ static void unpack(const u32x4 (&raw)[NR], double (&x)[2][8]) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float f[4];
                unpack_chunk<float, 4>(raw[2 * ch + h], f);
#pragma unroll
                for (int i = 0; i < 4; ++i) x[ch][4 * h + i] = (double)f[i];
            }
    }
};

// Blocks of two waves, shared angle set or not (the same reduction order for
// identical sets either way; with one set per key head each wave keeps the
// fp64 tables of every set, 9 KB).
constexpr int kStatsWaves = 2;

// FULL: support b = D (every butterfly stage, unconditionally); with half-split
// pairs the half butterfly is then folded into the table (FOLD).  Otherwise b
// is read at run time.  PH: one angle set per key head (a.angle_sets = Hkv of
// them), key head kh using set kh; each wave keeps the fp64 tables of every
// set (pair-major).  BIN: see group_stats (with a.xmask, a.wgt).

}  // namespace

}  // namespace rrp
