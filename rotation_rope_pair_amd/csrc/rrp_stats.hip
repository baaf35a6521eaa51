// rrp_stats.hip -- diagnostic pass: K range and quantisation error of the
// transformed K rows at one support b, or at every support b = 1 .. head_dim
// in one call (the support sweep: kSweepParts launches, each reading K once).
//
// Every K row goes through exactly the fp64 K transform and quantiser of the
// hot path (same device functions), is dequantised with its stored fp16
// scale, and the lane adds (yhat - y)^2 and y^2 in fp64; the lane holding a
// group's first channel adds that group's absmax and (max - min).  Wave, block
// and grid reductions run in a fixed order (bit-reproducible).
#include "rrp_device.hpp"
#include "rrp_kernels.hpp"

namespace rrp {

namespace {

constexpr int kNStat = 5;  // E, N, sum absmax, max absmax, sum range

// Per-lane running sums of one support's statistics.
struct StatAcc {
    double E = 0.0, N = 0.0, M = 0.0, maxM = 0.0, R = 0.0;
};

// Add one transformed K row (y in output channel order, lane position s) to the
// lane's sums: quantise every element with its group's stored fp16 scale,
// dequantise, and add (yhat - y)^2 and y^2; the lane holding a group's first
// channel adds the group's absmax and (max - min).
// SMALLG: groups smaller than one 16-byte chunk (reduced in registers).
template <int D, int CE, bool SMALLG>
__device__ __forceinline__ void add_row_stats(const double (&y)[2][CE], int g, int s, StatAcc& acc) {
    constexpr int P = D / 2;
    // The group's absmax is max(max, -min) (exact), so only max and min are reduced.
    if constexpr (!SMALLG) {
        // one group value per chunk: max, min over the group
        double cx[2], cn[2], ca[2];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            cx[ch] = y[ch][0];
            cn[ch] = y[ch][0];
#pragma unroll
            for (int i2 = 1; i2 < CE; ++i2) {
                cx[ch] = fmax(cx[ch], y[ch][i2]);
                cn[ch] = fmin(cn[ch], y[ch][i2]);
            }
        }
        group_reduce_chunkwise<D, CE, true>(cx, g);
        group_reduce_chunkwise<D, CE, false>(cn, g);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) ca[ch] = fmax(cx[ch], -cn[ch]);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            const GroupScale64 gs = group_scale64(ca[ch]);
#pragma unroll
            for (int i2 = 0; i2 < CE; ++i2) {
                const double diff = (double)code_of(y[ch][i2], gs.rcp) * gs.shv - y[ch][i2];
                acc.E += diff * diff;
                acc.N += y[ch][i2] * y[ch][i2];
            }
            if (((ch * P + s * CE) & (g - 1)) == 0) {  // the lane holding the group's first channel
                acc.M += ca[ch];
                acc.maxM = fmax(acc.maxM, ca[ch]);
                acc.R += cx[ch] - cn[ch];
            }
        }
    } else {
        double am[2][CE], mx[2][CE], mn[2][CE];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int i2 = 0; i2 < CE; ++i2) {
                mx[ch][i2] = y[ch][i2];
                mn[ch][i2] = y[ch][i2];
            }
        group_reduce_inreg<CE, true>(mx, g);
        group_reduce_inreg<CE, false>(mn, g);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int i2 = 0; i2 < CE; ++i2) am[ch][i2] = fmax(mx[ch][i2], -mn[ch][i2]);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int i2 = 0; i2 < CE; ++i2) {
                const GroupScale64 gs = group_scale64(am[ch][i2]);
                const double diff = (double)code_of(y[ch][i2], gs.rcp) * gs.shv - y[ch][i2];
                acc.E += diff * diff;
                acc.N += y[ch][i2] * y[ch][i2];
                if ((i2 & (g - 1)) == 0) {
                    acc.M += am[ch][i2];
                    acc.maxM = fmax(acc.maxM, am[ch][i2]);
                    acc.R += mx[ch][i2] - mn[ch][i2];
                }
            }
    }
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

// PH: one angle set per key head (a.angle_sets = Hkv of them), key head kh using
// set kh; the fp64 tables of every set are kept per wave (pair-major).
template <typename E, int D, int LAYOUT, int BT, bool SMALLG, bool PH>
__global__ __launch_bounds__(256) void stats_kernel(const StatsArgs a) {
    using G = Geo<E, D>;
    using LM = LaneMap<G::L>;
    constexpr int CE = G::CE, P = G::P, R = G::R;
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr size_t ROWB = (size_t)D * EB;
    constexpr bool FOLD = (LAYOUT == 0) && (BT == D);
    __shared__ float2 tab32_all[4][PH ? 1 : tab_entries<P>()];  // fp32 tables (unused by per-set tables)
    __shared__ double2 tab64_all[4][PH ? kSetStride * P : tab_entries<P>()];
    __shared__ double2 phi_all[PH ? kSetStride * P : 1];
    __shared__ double red[4][kNStat];

    const int lane = (int)__lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwave = (int)(blockDim.x >> 6);
    const int s = LM::s_of(lane);
    const int grp = LM::grp_of(lane);
    float2* tab32 = tab32_all[wave];
    double2* tab64 = tab64_all[wave];

    double cphi = 1.0, sphi = 0.0;
    if constexpr (PH) load_angle_sets<P>(phi_all, a.angles, a.angle_sets);
    else if (a.angles != nullptr && lane < P) sincos_f64_of_f32(a.angles[lane], sphi, cphi);
    const float invf = lane_inv_freq(a.inv_freq, lane, P);
    const int s_src = s ^ lane_perm_mask<D, CE>(BT ? BT : a.support_b);  // permuted loads, see fwht_row
    int kidx[CE];
    pair_index_of_lane<D, LAYOUT, CE>(s_src, kidx);
    if constexpr (PH) {
#pragma unroll
        for (int j = 0; j < CE; ++j) kidx[j] *= kSetStride;  // pair-major per-set tables
    } else {
#pragma unroll
        for (int j = 0; j < CE; ++j) kidx[j] = tab_index(kidx[j]);  // padded shared table
    }
    const unsigned char* kb = static_cast<const unsigned char*>(a.k);
    const int npass = (a.hk + R - 1) / R;
    const int g = a.group;
    const int64_t stride = (int64_t)gridDim.x * nwave;

    auto load_pass = [&](int64_t t, int ps, u32x4 (&raw)[2]) {
        const int row = ps * R + grp;
        if (row < a.hk) {
            const unsigned char* rp = kb + ((size_t)t * a.hk + row) * ROWB;
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
                raw[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp + chunk_offset<E, D>(ch, s_src)));
        } else {
            raw[0] = raw[1] = u32x4{0, 0, 0, 0};
        }
    };

    StatAcc acc;
    int64_t t = (int64_t)blockIdx.x * nwave + wave;
    int ps = 0;
    u32x4 cur[2], nxt[2];
    if (t < a.n_tokens) load_pass(t, 0, cur);
    // Retire the first pass here: inside the loop `cur` is then always a copy
    // made after its wait, and the loop's first use of it needs no wait (which
    // would otherwise also take the next pass's prefetch on every iteration).
    asm volatile("" ::"v"(cur[0]), "v"(cur[1]));
    while (t < a.n_tokens) {
        // keep the next pass (this token's or the next token's first) in flight
        int64_t tn = t;
        int pn = ps + 1;
        if (pn == npass) {
            tn = t + stride;
            pn = 0;
        }
        if (tn < a.n_tokens) load_pass(tn, pn, nxt);
        if (ps == 0) {
            if constexpr (PH) token_tables_sets<D, FOLD>(nullptr, tab64, lane, token_pos(a.pos, t), invf, phi_all, a.angle_sets, a.rsqrt_b);
            else token_tables<D, FOLD>(tab32, tab64, lane, token_pos(a.pos, t), invf, cphi, sphi, a.rsqrt_b);
        }
        if (ps * R + grp < a.hk) {
            float yf[2][CE];
            unpack_chunk<E, CE>(cur[0], yf[0]);
            unpack_chunk<E, CE>(cur[1], yf[1]);
            double y[2][CE];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int i2 = 0; i2 < CE; ++i2) y[ch][i2] = (double)yf[ch][i2];
            rotate_lds<LAYOUT, FOLD>(y, PH ? tab64 + (ps * R + grp) : tab64, kidx);
            fwht_row<D, CE, BT, FOLD>(y, a.support_b, s);
            add_row_stats<D, CE, SMALLG>(y, g, s, acc);
        }
        cur[0] = nxt[0];
        cur[1] = nxt[1];
        t = tn;
        ps = pn;
    }
    block_stats_partials(acc, 0, red, a.partials);
}

// ---------------------------------------------------------------------------
// Support sweep: the statistics of every support b = 1, 2, 4, ..., D from
// kSweepParts reads of K (one launch per part of the supports).  Each row is
// rotated once per launch (RoPE + R_phi, natural channel order),
// its b = 1 statistics are taken, then the Walsh-Hadamard butterflies are
// applied one channel bit at a time from the lowest, each followed by a factor
// 1/sqrt(2): after the stage of bit j - 1 the row holds the normalised block
// transform of support 2^j (to a few fp64 roundings), and its statistics are
// taken.
// ---------------------------------------------------------------------------

// Natural-order lane butterfly (fp64): the lane with the position bit clear
// keeps a + b, the other a - b (a = the bit-clear lane's value).
template <int L, int CE, int M>
__device__ __forceinline__ void lane_stage_natural(double (&x)[2][CE], int s) {
    const bool hi = (s & M) != 0;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int i = 0; i < CE; ++i) {
            const double p = s_xor<L, M>(x[ch][i]);
            x[ch][i] = hi ? p - x[ch][i] : x[ch][i] + p;
        }
}

// Butterfly on channel bit BIT (channel c = ch * D/2 + s * CE + i).
template <int D, int CE, int BIT>
__device__ __forceinline__ void sweep_stage(double (&y)[2][CE], int s) {
    constexpr int L = D / (2 * CE);
    constexpr int LCE = CE == 8 ? 3 : 2;  // log2 CE
    if constexpr (BIT < LCE) {
        fwht_inreg_stage<CE, (1 << BIT)>(y);
    } else if constexpr ((1 << (BIT - LCE)) < L) {
        lane_stage_natural<L, CE, (1 << (BIT - LCE))>(y, s);
    } else {
#pragma unroll
        for (int i = 0; i < CE; ++i) {
            const double a0 = y[0][i], a1 = y[1][i];
            y[0][i] = a0 + a1;
            y[1][i] = a0 - a1;
        }
    }
}

// Statistics of supports 2^J .. 2^(J1-1) (those from 2^J0 on) for a row holding
// the normalised support-2^(J-1) transform (the rotated row itself for J = 0);
// acc[J - J0] holds support 2^J.
template <int D, int CE, bool SMALLG, int J, int J0, int J1>
struct SweepRest {
    __device__ static void run(double (&y)[2][CE], int g, int s, StatAcc (&acc)[J1 - J0]) {
        if constexpr (J > 0) {
            // one more butterfly stage, renormalised in place: y stays H_b / sqrt(b) x
            sweep_stage<D, CE, J - 1>(y, s);
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int i = 0; i < CE; ++i) y[ch][i] *= 0.70710678118654752440;
        }
        if constexpr (J >= J0) add_row_stats<D, CE, SMALLG>(y, g, s, acc[J - J0]);
        if constexpr (J + 1 < J1) SweepRest<D, CE, SMALLG, J + 1, J0, J1>::run(y, g, s, acc);
    }
};

template <int D> struct Log2;
template <> struct Log2<64> { static constexpr int value = 6; };
template <> struct Log2<128> { static constexpr int value = 7; };

// Supports 2^J0 .. 2^(J1-1) of the sweep (the sweep runs as several launches,
// each keeping its supports' sums in registers).
template <typename E, int D, int LAYOUT, bool SMALLG, int J0, int J1, bool PH>
__global__ __launch_bounds__(256) void stats_sweep_kernel(const StatsArgs a) {
    using G = Geo<E, D>;
    using LM = LaneMap<G::L>;
    constexpr int CE = G::CE, P = G::P, R = G::R;
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr size_t ROWB = (size_t)D * EB;
    constexpr int NJ = J1 - J0;
    __shared__ float2 tab32_all[4][PH ? 1 : tab_entries<P>()];  // fp32 tables (unused by per-set tables)
    __shared__ double2 tab64_all[4][PH ? kSetStride * P : tab_entries<P>()];
    __shared__ double2 phi_all[PH ? kSetStride * P : 1];
    __shared__ double red[4][kNStat];

    const int lane = (int)__lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwave = (int)(blockDim.x >> 6);
    const int s = LM::s_of(lane);
    const int grp = LM::grp_of(lane);
    float2* tab32 = tab32_all[wave];
    double2* tab64 = tab64_all[wave];

    double cphi = 1.0, sphi = 0.0;
    if constexpr (PH) load_angle_sets<P>(phi_all, a.angles, a.angle_sets);
    else if (a.angles != nullptr && lane < P) sincos_f64_of_f32(a.angles[lane], sphi, cphi);
    const float invf = lane_inv_freq(a.inv_freq, lane, P);
    int kidx[CE];
    pair_index_of_lane<D, LAYOUT, CE>(s, kidx);  // natural chunk order
    if constexpr (PH) {
#pragma unroll
        for (int j = 0; j < CE; ++j) kidx[j] *= kSetStride;  // pair-major per-set tables
    } else {
#pragma unroll
        for (int j = 0; j < CE; ++j) kidx[j] = tab_index(kidx[j]);  // padded shared table
    }
    const unsigned char* kb = static_cast<const unsigned char*>(a.k);
    const int npass = (a.hk + R - 1) / R;
    const int g = a.group;
    const int64_t stride = (int64_t)gridDim.x * nwave;

    auto load_pass = [&](int64_t t, int ps, u32x4 (&raw)[2]) {
        const int row = ps * R + grp;
        if (row < a.hk) {
            const unsigned char* rp = kb + ((size_t)t * a.hk + row) * ROWB;
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
                raw[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rp + chunk_offset<E, D>(ch, s)));
        } else {
            raw[0] = raw[1] = u32x4{0, 0, 0, 0};
        }
    };

    StatAcc acc[NJ];
    int64_t t = (int64_t)blockIdx.x * nwave + wave;
    int ps = 0;
    u32x4 cur[2], nxt[2];
    if (t < a.n_tokens) load_pass(t, 0, cur);
    // Retire the first pass here: inside the loop `cur` is then always a copy
    // made after its wait, and the loop's first use of it needs no wait (which
    // would otherwise also take the next pass's prefetch on every iteration).
    asm volatile("" ::"v"(cur[0]), "v"(cur[1]));
    while (t < a.n_tokens) {
        int64_t tn = t;
        int pn = ps + 1;
        if (pn == npass) {
            tn = t + stride;
            pn = 0;
        }
        if (tn < a.n_tokens) load_pass(tn, pn, nxt);
        if (ps == 0) {
            if constexpr (PH) token_tables_sets<D, false>(nullptr, tab64, lane, token_pos(a.pos, t), invf, phi_all, a.angle_sets, 1.0);
            else token_tables<D, false>(tab32, tab64, lane, token_pos(a.pos, t), invf, cphi, sphi, 1.0);
        }
        if (ps * R + grp < a.hk) {
            float yf[2][CE];
            unpack_chunk<E, CE>(cur[0], yf[0]);
            unpack_chunk<E, CE>(cur[1], yf[1]);
            double y[2][CE];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int i2 = 0; i2 < CE; ++i2) y[ch][i2] = (double)yf[ch][i2];
            rotate_lds<LAYOUT, false>(y, PH ? tab64 + (ps * R + grp) : tab64, kidx);
            SweepRest<D, CE, SMALLG, 0, J0, J1>::run(y, g, s, acc);
        }
        cur[0] = nxt[0];
        cur[1] = nxt[1];
        t = tn;
        ps = pn;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) block_stats_partials(acc[j], J0 + j, red, a.partials);
}

// One wave per (set, statistic): lane l combines the partials of blocks l,
// l + 64, ... in order, then a fixed xor butterfly folds the lanes (every lane
// ends with the same value).  Partials are laid out [set * 5 + statistic][block];
// stats_out row `set` is {E, N, sum absmax, max absmax, sum range, n_groups,
// n_rows, support} (support 0 for a single-support call).
__global__ __launch_bounds__(256) void stats_final_kernel(const StatsFinalArgs a) {
    const int w = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    const int lane = (int)__lane_id();
    if (w < a.n_sets * kNStat) {
        const int set = w / kNStat, e = w % kNStat;
        const double* part = a.partials + (size_t)w * a.n_blocks;
        double v = 0.0;
        for (int b = lane; b < a.n_blocks; b += 64) v = (e == 3) ? fmax(v, part[b]) : v + part[b];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const double o = shfl_xor_d(v, m);
            v = (e == 3) ? fmax(v, o) : v + o;
        }
        if (lane == 0) a.stats_out[set * 8 + e] = v;
    } else if (w == a.n_sets * kNStat && lane < a.n_sets) {
        a.stats_out[lane * 8 + 5] = a.n_groups;
        a.stats_out[lane * 8 + 6] = a.n_rows;
        a.stats_out[lane * 8 + 7] = a.sweep ? (double)(1 << lane) : 0.0;
    }
}

// The sweep's supports are split over kSweepParts launches (each keeps its
// supports' sums in registers and reads K once).
constexpr int kSweepParts = 4;

template <typename E, int D, int LAYOUT, bool SG, bool PH, int J0, int NB, int W>
void launch_sweep_parts(const StatsArgs& a, int n_blocks, hipStream_t st) {
    if constexpr (J0 < NB) {
        constexpr int J1 = J0 + W < NB ? J0 + W : NB;
        hipLaunchKernelGGL((stats_sweep_kernel<E, D, LAYOUT, SG, J0, J1, PH>), dim3(n_blocks), dim3(256), 0, st, a);
        launch_sweep_parts<E, D, LAYOUT, SG, PH, J1, NB, W>(a, n_blocks, st);
    }
}

template <typename E, int D, int LAYOUT, bool PH>
hipError_t launch_p(const StatsArgs& a, int n_blocks, bool sweep, hipStream_t st) {
    constexpr int CE = Geo<E, D>::CE;
    const bool small = a.group < CE;
    if (sweep) {
        constexpr int NB = Log2<D>::value + 1;
        constexpr int W = (NB + kSweepParts - 1) / kSweepParts;  // supports per launch
        if (small) launch_sweep_parts<E, D, LAYOUT, true, PH, 0, NB, W>(a, n_blocks, st);
        else launch_sweep_parts<E, D, LAYOUT, false, PH, 0, NB, W>(a, n_blocks, st);
        return hipGetLastError();
    }
#define RRP_LAUNCH(BT, SG) \
    hipLaunchKernelGGL((stats_kernel<E, D, LAYOUT, BT, SG, PH>), dim3(n_blocks), dim3(256), 0, st, a)
    if (a.support_b == D) {
        if (small) RRP_LAUNCH(D, true); else RRP_LAUNCH(D, false);
    } else {
        if (small) RRP_LAUNCH(0, true); else RRP_LAUNCH(0, false);
    }
#undef RRP_LAUNCH
    return hipGetLastError();
}

template <typename E, int D, int LAYOUT>
hipError_t launch_t(const StatsArgs& a, int n_blocks, bool sweep, hipStream_t st) {
    if (a.angle_sets > 1) return launch_p<E, D, LAYOUT, true>(a, n_blocks, sweep, st);
    return launch_p<E, D, LAYOUT, false>(a, n_blocks, sweep, st);
}

}  // namespace

int stats_blocks(int64_t n_tokens) {
    int64_t b = (n_tokens + 15) / 16;  // about 4 tokens per wave
    if (b < 1) b = 1;
    if (b > kMaxStatsBlocks) b = kMaxStatsBlocks;
    return (int)b;
}

hipError_t launch_stats(const StatsArgs& a, int n_blocks, int dtype, int head_dim, int layout, bool sweep,
                        hipStream_t st) {
#define RRP_DISPATCH(E, D, LY) \
    if (head_dim == D && layout == LY) return launch_t<E, D, LY>(a, n_blocks, sweep, st);
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

hipError_t launch_stats_final(const StatsFinalArgs& a, hipStream_t st) {
    const int waves = a.n_sets * kNStat + 1;
    hipLaunchKernelGGL(stats_final_kernel, dim3((waves + 3) / 4), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace rrp
