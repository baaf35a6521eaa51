// rrp_sweep.hpp -- the support sweep: K range and quantisation error of the
// transformed K rows at every support b = 1, 2, 4, ..., head_dim, from one
// read of K in one launch.  Instantiated per element type by
// rrp_sweep_bf16.hip and rrp_sweep_f32.hip (compiled in parallel).
#pragma once
#include "rrp_stats_common.hpp"

namespace rrp {

namespace {

// ---------------------------------------------------------------------------
// Support sweep (sweep_kernel): the statistics of every support
// b = 1, 2, 4, ..., D from one read of K.  Each row is rotated once (RoPE +
// R_phi, no 1 / sqrt(b)) in the single-support kernel's lane layout, its
// energy taken once (the normalised transforms are orthogonal) and its b = 1
// statistics taken; then the Walsh-Hadamard butterflies run one channel bit at
// a time from the lowest, unnormalised: after the stage of bit j - 1 the lane
// holds u = H_b x for b = 2^j, whose statistics are taken with the 1 / sqrt(b)
// folded into each group's constants (group_stats, SCALED).  The in-run bits
// act on the natural layout, the run-position bits after the LDS
// transposition, and the half bit last (groups smaller than half the head
// take their statistics back in the natural layout).  The lane's sums are
// brought to the normalised transform's (E / b, M, maxM and R / sqrt(b)) once,
// at the end.
// ---------------------------------------------------------------------------
template <int D> struct Log2;
template <> struct Log2<64> { static constexpr int value = 6; };
template <> struct Log2<128> { static constexpr int value = 7; };

// 1 / sqrt(2^j) and sqrt(2^j), exact powers of two times the nearest doubles of
// 1 / sqrt(2) and sqrt(2).
__device__ __forceinline__ constexpr double rsqrt_pow2(int j) {
    double v = (j & 1) ? 0.70710678118654752440 : 1.0;
    for (int k = 0; k < j / 2; ++k) v *= 0.5;
    return v;
}
__device__ __forceinline__ constexpr double sqrt_pow2(int j) {
    double v = (j & 1) ? 1.41421356237309504880 : 1.0;
    for (int k = 0; k < j / 2; ++k) v *= 2.0;
    return v;
}

// Where a group of G channels sits in either layout of the pass: runs of BIN
// consecutive entries of a lane, completed across the lane position bits XM.
template <int D, int G> struct SweepGroups {
    static constexpr int P = D / 2, L = SGeo<D>::L, K8 = SGeo<D>::K8;
    // natural layout (supports 1 .. 8)
    static constexpr int BINN = G <= 8 ? G : (G <= P ? 8 : 16);
    static constexpr int XMN = G <= 8 ? 0 : (G <= P ? G / 8 - 1 : L - 1);
    // transposed layout (supports 16 .. D)
    static constexpr int BINT = G > 8 ? (G == D ? 16 : K8 * G / 8) : (G < K8 ? G : K8);
    static constexpr int XMT = G > 8 ? L - 1 : (G > K8 ? G / K8 - 1 : 0);
    static constexpr double WN = 1.0 / (double)(1 << __builtin_popcount(XMN));
    static constexpr double WT = 1.0 / (double)(1 << __builtin_popcount(XMT));
};

template <typename E, int D, int LAYOUT, bool PH, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void sweep_kernel(const StatsArgs a) {
    using Geo_ = SGeo<D>;
    using LM = LaneMap<Geo_::L>;
    using IO = SRow<E>;
    using GR = SweepGroups<D, G>;
    constexpr int P = Geo_::P, L = Geo_::L, R = Geo_::R;
    constexpr int NJ = Log2<D>::value + 1;  // supports 2^0 .. 2^(NJ-1)
    constexpr size_t ROWB = (size_t)D * ElemInfo<E>::bytes;
    constexpr int WAVES = kStatsWaves;
    __shared__ double2 tab_all[WAVES][tab_entries<P>()];
    __shared__ double2 phi_all[PH ? kSetStride * P : 1];
    __shared__ double2 tbuf_all[WAVES][Geo_::SLOTS];
    __shared__ double red[4][kNStat];

    const int lane = (int)__lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwave = (int)(blockDim.x >> 6);
    const int s = LM::s_of(lane);
    const int r = LM::grp_of(lane);
    double2* tab = tab_all[wave];
    double2* tb = tbuf_all[wave];

    double cphi = 1.0, sphi = 0.0;
    int kidx[8];
    pair_index_of_lane<D, LAYOUT, 8>(s, kidx);
    // One angle set per key head: the lane's row is key head r (set r) for the
    // whole kernel (see stats_kernel); each pass composes its pairs' entries of
    // set r in the block's (cos, sin)(phi) table with the token's bare RoPE
    // table (the sweep's registers leave no room to keep them, as the
    // single-support kernel does).
    const double2* phirow = phi_all;
    if constexpr (PH) {
        load_angle_sets<P>(phi_all, a.angles, a.angle_sets);  // ends with a block barrier
        phirow = phi_all + kidx[0] * kSetStride + (r < a.hk ? r : 0);
    } else if (a.angles != nullptr && lane < P) {
        sincos_f64_of_f32(a.angles[lane], sphi, cphi);
    }
    const float invf = lane_inv_freq(a.inv_freq, lane, P);
#pragma unroll
    for (int j = 0; j < 8; ++j) kidx[j] = tab_index(kidx[j]);
    const unsigned char* kb = static_cast<const unsigned char*>(a.k);
    const int hk = a.hk;
    const int npass = (hk + R - 1) / R;
    const int64_t stride = (int64_t)gridDim.x * nwave;

    auto load_pass = [&](int64_t t, int ps, u32x4 (&raw)[IO::NR]) {
        const int row = ps * R + r;
        if (row < hk) IO::template load<D>(kb + ((size_t)t * hk + row) * ROWB, s, raw);
        else
#pragma unroll
            for (int k = 0; k < IO::NR; ++k) raw[k] = u32x4{0, 0, 0, 0};
    };

    StatAcc acc[NJ];
    // One pass (R rows of a token): FIX false is the main pass, FIX true the
    // rare correction pass over the same rows.
    auto pass = [&](auto fixc, const u32x4 (&raw)[IO::NR], int ps, StatAcc (&acc)[NJ], bool& far) {
        constexpr bool FIX = decltype(fixc)::value;
        double x[2][8];
        IO::unpack(raw, x);
        if constexpr (PH) rotate_sets_lds<D, LAYOUT, false>(x, tab, kidx, phirow, 1.0);
        else rotate_tab<LAYOUT, false>(x, tab, kidx);
        double(&xv)[16] = reinterpret_cast<double(&)[16]>(x);
        // support 1 (with the energy), then the in-run bits: supports 2, 4, 8
        group_stats<GR::BINN, L, false, FIX>(xv, GR::XMN, GR::WN, acc[0], far);
        fwht_inreg_stage<8, 1>(x);
        group_stats<GR::BINN, L, true, FIX>(xv, GR::XMN, GR::WN, acc[1], far, rsqrt_pow2(1), sqrt_pow2(1));
        fwht_inreg_stage<8, 2>(x);
        group_stats<GR::BINN, L, true, FIX>(xv, GR::XMN, GR::WN, acc[2], far, rsqrt_pow2(2), sqrt_pow2(2));
        fwht_inreg_stage<8, 4>(x);
        group_stats<GR::BINN, L, true, FIX>(xv, GR::XMN, GR::WN, acc[3], far, rsqrt_pow2(3), sqrt_pow2(3));
        // the run-position bits (supports 16 .. D/2), transposed, then the half bit (support D)
        double tt[16];
        transpose_in<D>(tb, r, s, x, tt);
        // Statistics of the support just reached.  Groups smaller than half the
        // head are reduced in the natural layout (transposed back into x): there
        // they need fewer cross-lane stages.
        auto stats_t = [&](int j) {
            if constexpr (G < D / 2) {
                transpose_out<D>(tb, r, s, tt, x);
                group_stats<GR::BINN, L, true, FIX>(xv, GR::XMN, GR::WN, acc[j], far, rsqrt_pow2(j), sqrt_pow2(j));
            } else {
                group_stats<GR::BINT, L, true, FIX>(tt, GR::XMT, GR::WT, acc[j], far, rsqrt_pow2(j), sqrt_pow2(j));
            }
        };
#pragma unroll
        for (int h = 1, j = 4; h < L; h <<= 1, ++j) {
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int u = 0; u < L; ++u)
                    if ((u & h) == 0)
#pragma unroll
                        for (int ii = 0; ii < Geo_::K8; ++ii) {
                            const int e0 = ch * 8 + u * Geo_::K8 + ii, e1 = e0 + h * Geo_::K8;
                            const double p = tt[e0], q = tt[e1];
                            tt[e0] = p + q;
                            tt[e1] = p - q;
                        }
            stats_t(j);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double p = tt[e], q = tt[8 + e];
            tt[e] = p + q;
            tt[8 + e] = p - q;
        }
        stats_t(NJ - 1);
    };
    int64_t t = (int64_t)blockIdx.x * nwave + wave;
    int ps = 0;
    u32x4 cur[IO::NR], nxt[IO::NR];
    if (t < a.n_tokens) load_pass(t, 0, cur);
#pragma unroll
    for (int k = 0; k < IO::NR; ++k) asm volatile("" ::"v"(cur[k]));
    while (t < a.n_tokens) {
        int64_t tn = t;
        int pn = ps + 1;
        if (pn == npass) {
            tn = t + stride;
            pn = 0;
        }
        if (tn < a.n_tokens) load_pass(tn, pn, nxt);
        if (ps == 0) {
            if constexpr (PH) token_table64<D, false>(tab, lane, token_pos(a.pos, t), invf, 1.0, 0.0, 1.0);
            else token_table64<D, false>(tab, lane, token_pos(a.pos, t), invf, cphi, sphi, 1.0);
        }
        bool far = false;
        pass(BoolC<false>{}, cur, ps, acc, far);
#pragma unroll
        for (int j = 0; j < NJ; ++j) pin(acc[j]);
        if (__ballot(far) != 0) {  // rare: redo the pass, adding only the clamped codes' change
            u32x4 raw[IO::NR];
            load_pass(t, ps, raw);
            StatAcc fx[NJ];
            pass(BoolC<true>{}, raw, ps, fx, far);
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[j].E += fx[j].E;
        }
#pragma unroll
        for (int k = 0; k < IO::NR; ++k) cur[k] = nxt[k];
        t = tn;
        ps = pn;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        StatAcc o = acc[j];
        if (j > 0) {
            const double cb = rsqrt_pow2(j);
            o.E *= cb * cb;  // 1 / b, exact
            o.N = acc[0].N;
            o.M *= cb;
            o.maxM *= cb;
            o.R *= cb;
        }
        block_stats_partials(o, j, red, a.partials);
    }
}

template <typename E, int D, int LAYOUT, bool PH>
hipError_t launch_sweep_t(const StatsArgs& a, int n_blocks, hipStream_t st) {
    const dim3 grid((unsigned)n_blocks), block(64 * kStatsWaves);
#define RRP_SWEEP_G(G)                                                                   \
    if constexpr (G <= D)                                                                \
        if (a.group == G) {                                                              \
            hipLaunchKernelGGL((sweep_kernel<E, D, LAYOUT, PH, G>), grid, block, 0, st, a); \
            return hipGetLastError();                                                    \
        }
    RRP_SWEEP_G(2) RRP_SWEEP_G(4) RRP_SWEEP_G(8) RRP_SWEEP_G(16) RRP_SWEEP_G(32) RRP_SWEEP_G(64) RRP_SWEEP_G(128)
#undef RRP_SWEEP_G
    return hipErrorInvalidValue;
}

// Every head_dim, pair layout and angle-set mode of element type E.
template <typename E>
hipError_t launch_sweep_e(const StatsArgs& a, int n_blocks, int head_dim, int layout, hipStream_t st) {
#define RRP_DISPATCH(D, LY)                                                                \
    if (head_dim == D && layout == LY) {                                                  \
        if (a.angle_sets > 1) return launch_sweep_t<E, D, LY, true>(a, n_blocks, st);     \
        return launch_sweep_t<E, D, LY, false>(a, n_blocks, st);                          \
    }
    RRP_DISPATCH(64, 0) RRP_DISPATCH(64, 1) RRP_DISPATCH(128, 0) RRP_DISPATCH(128, 1)
#undef RRP_DISPATCH
    return hipErrorInvalidValue;
}

}  // namespace

}  // namespace rrp
