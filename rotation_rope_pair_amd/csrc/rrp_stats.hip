// rrp_stats.hip -- diagnostic pass at one support b: K range and quantisation
// error of the transformed K rows (stats_kernel), and the final reduction of
// every diagnostic's block partials (stats_final_kernel).
#include "rrp_stats_common.hpp"

namespace rrp {

namespace {

template <typename E, int D, int LAYOUT, bool FULL, bool PH, int BIN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void stats_kernel(const StatsArgs a) {
    constexpr bool FOLD = FULL && LAYOUT == 0;
    using G = SGeo<D>;
    using LM = LaneMap<G::L>;
    using IO = SRow<E>;
    constexpr int P = G::P, L = G::L, R = G::R;
    constexpr size_t ROWB = (size_t)D * ElemInfo<E>::bytes;
    constexpr int WAVES = kStatsWaves;
    __shared__ double2 tab_all[WAVES][tab_entries<P>()];
    // the passes' transpositions; with one angle set per key head it first
    // stages the sets' (cos, sin)(phi) for the lanes to take into registers
    __shared__ double2 tbuf_all[WAVES][G::SLOTS];
    __shared__ double red[4][kNStat];
    static_assert(!PH || WAVES * G::SLOTS >= kSetStride * P, "staging of the angle sets");

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
    // One angle set per key head (at most 8, so a token's key rows are one pass
    // and the lane's row r is key head r, hence set r, for the whole kernel):
    // the lane keeps (cos, sin)(phi) of its pairs in that set in registers and
    // composes them with the token's bare RoPE table (rotate_sets).
    double2 cs_phi[PH ? 8 : 1];
    if constexpr (PH) {
        double2* stage = &tbuf_all[0][0];
        load_angle_sets<P>(stage, a.angles, a.angle_sets);  // ends with a block barrier
        const int set = r < a.hk ? r : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) cs_phi[j] = stage[kidx[j] * kSetStride + set];
        __syncthreads();  // read before the buffer serves the transpositions
    } else if (a.angles != nullptr && lane < P) {
        sincos_f64_of_f32(a.angles[lane], sphi, cphi);
    }
    const float invf = lane_inv_freq(a.inv_freq, lane, P);
#pragma unroll
    for (int j = 0; j < 8; ++j) kidx[j] = tab_index(kidx[j]);
    const unsigned char* kb = static_cast<const unsigned char*>(a.k);
    const int hk = a.hk, b = FULL ? D : a.support_b, xmask = a.xmask;
    const double w = a.wgt;
    const int npass = (hk + R - 1) / R;
    const bool transpose = FULL || b > 8;          // butterflies on the run position
    // groups smaller than half the head: reduced in the natural layout (fewer
    // cross-lane stages than the transposed one, for the cost of transposing back)
    const bool back = transpose && a.group < D / 2;
    const int64_t stride = (int64_t)gridDim.x * nwave;

    // rows past the last head read as zeros (they add nothing to any sum)
    auto load_pass = [&](int64_t t, int ps, u32x4 (&raw)[IO::NR]) {
        const int row = ps * R + r;
        if (row < hk) IO::template load<D>(kb + ((size_t)t * hk + row) * ROWB, s, raw);
        else
#pragma unroll
            for (int k = 0; k < IO::NR; ++k) raw[k] = u32x4{0, 0, 0, 0};
    };

    StatAcc acc;
    // One pass (R rows of a token): FIX false is the main pass, FIX true the
    // rare correction pass over the same rows.
    auto pass = [&](auto fixc, const u32x4 (&raw)[IO::NR], bool& far) {
        constexpr bool FIX = decltype(fixc)::value;
        double x[2][8];
        IO::unpack(raw, x);
        if constexpr (PH) rotate_sets<LAYOUT, FOLD>(x, tab, kidx, cs_phi, a.rsqrt_b);
        else rotate_tab<LAYOUT, FOLD>(x, tab, kidx);
        if (b > 1) fwht_inreg_stage<8, 1>(x);
        if (b > 2) fwht_inreg_stage<8, 2>(x);
        if (b > 4) fwht_inreg_stage<8, 4>(x);
        if (!FOLD && b > P) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double p = x[0][i], q = x[1][i];
                x[0][i] = p + q;
                x[1][i] = p - q;
            }
        }
        // x[ch][i] is entry ch * 8 + i of the natural layout
        double(&xv)[16] = reinterpret_cast<double(&)[16]>(x);
        if (transpose) {
            double tt[16];
            transpose_in<D>(tb, r, s, x, tt);
            fwht_runs<D>(tt, b);
            if (back) {
                transpose_out<D>(tb, r, s, tt, x);
                group_stats<BIN, L, false, FIX>(xv, xmask, w, acc, far);
            } else {
                group_stats<BIN, L, false, FIX>(tt, xmask, w, acc, far);
            }
        } else {
            group_stats<BIN, L, false, FIX>(xv, xmask, w, acc, far);
        }
    };
    int64_t t = (int64_t)blockIdx.x * nwave + wave;
    int ps = 0;
    u32x4 cur[IO::NR], nxt[IO::NR];
    if (t < a.n_tokens) load_pass(t, 0, cur);
    // Retire the first pass here: inside the loop `cur` is then always a copy
    // made after its wait, and the loop's first use of it needs no wait (which
    // would otherwise also take the next pass's prefetch on every iteration).
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
            else token_table64<D, FOLD>(tab, lane, token_pos(a.pos, t), invf, cphi, sphi, a.rsqrt_b);
        }
        bool far = false;
        pass(BoolC<false>{}, cur, far);
        pin(acc);
        if (__ballot(far) != 0) {  // rare: redo the pass, adding only the clamped codes' change
            u32x4 raw[IO::NR];
            load_pass(t, ps, raw);
            pass(BoolC<true>{}, raw, far);
        }
#pragma unroll
        for (int k = 0; k < IO::NR; ++k) cur[k] = nxt[k];
        t = tn;
        ps = pn;
    }
    block_stats_partials(acc, 0, red, a.partials);
}

// One block per (set, statistic): thread i combines the partials of blocks i,
// i + 256, ... in order, a fixed xor butterfly folds each wave, and thread 0
// combines the four waves in order.  Partials are laid out
// [set * 5 + statistic][block]; stats_out row `set` is {E, N, sum absmax,
// max absmax, sum range, n_groups, n_rows, support} (support 0 for a
// single-support call); block n_sets * 5 writes the last three columns.
__global__ __launch_bounds__(256) void stats_final_kernel(const StatsFinalArgs a) {
    __shared__ double wsum[4];
    const int w = (int)blockIdx.x;
    const int tid = (int)threadIdx.x, lane = (int)__lane_id(), wave = tid >> 6;
    if (w == a.n_sets * kNStat) {
        if (tid < a.n_sets) {
            a.stats_out[tid * 8 + 5] = a.n_groups;
            a.stats_out[tid * 8 + 6] = a.n_rows;
            a.stats_out[tid * 8 + 7] = a.sweep ? (double)(1 << tid) : 0.0;
        }
        return;
    }
    const int set = w / kNStat, e = w % kNStat;
    const bool is_max = e == 3;
    const double* part = a.partials + (size_t)w * a.n_blocks;
    double v = 0.0;
#pragma unroll 4
    for (int b = tid; b < a.n_blocks; b += 256) v = is_max ? fmax(v, part[b]) : v + part[b];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const double o = shfl_xor_d(v, m);
        v = is_max ? fmax(v, o) : v + o;
    }
    if (lane == 0) wsum[wave] = v;
    __syncthreads();
    if (tid == 0) {
        double r = wsum[0];
        for (int k = 1; k < 4; ++k) r = is_max ? fmax(r, wsum[k]) : r + wsum[k];
        a.stats_out[set * 8 + e] = r;
    }
}

template <typename E, int D, int LAYOUT, bool FULL, bool PH>
hipError_t launch_single(const StatsArgs& a, int n_blocks, hipStream_t st) {
    const dim3 grid((unsigned)n_blocks), block(64 * kStatsWaves);
    switch (a.bin) {
        case 2: hipLaunchKernelGGL((stats_kernel<E, D, LAYOUT, FULL, PH, 2>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((stats_kernel<E, D, LAYOUT, FULL, PH, 4>), grid, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((stats_kernel<E, D, LAYOUT, FULL, PH, 8>), grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL((stats_kernel<E, D, LAYOUT, FULL, PH, 16>), grid, block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename E, int D, int LAYOUT, bool PH>
hipError_t launch_p(const StatsArgs& args, int n_blocks, hipStream_t st) {
    // Where a group's channels sit after the transform (see stats_kernel):
    // BIN consecutive entries of a lane, completed across the lanes of xmask.
    StatsArgs a = args;
    constexpr int L = SGeo<D>::L, K8 = SGeo<D>::K8, P = D / 2;
    const int g = a.group, b = a.support_b;
    if (b > 8 && g >= D / 2) {   // transposed layout: a group holds every run offset
        a.bin = g == D ? 16 : K8 * g / 8;
        a.xmask = L - 1;
    } else if (g <= 8) {         // natural layout: a run of the lane
        a.bin = g;
        a.xmask = 0;
    } else if (g <= P) {         // natural layout: runs of g / 8 lanes
        a.bin = 8;
        a.xmask = g / 8 - 1;
    } else {                     // natural layout: the whole row
        a.bin = 16;
        a.xmask = L - 1;
    }
    a.wgt = 1.0 / (double)(1 << __builtin_popcount(a.xmask));
    if (b == D) return launch_single<E, D, LAYOUT, true, PH>(a, n_blocks, st);
    return launch_single<E, D, LAYOUT, false, PH>(a, n_blocks, st);
}

template <typename E, int D, int LAYOUT>
hipError_t launch_t(const StatsArgs& a, int n_blocks, hipStream_t st) {
    if (a.angle_sets > 1) return launch_p<E, D, LAYOUT, true>(a, n_blocks, st);
    return launch_p<E, D, LAYOUT, false>(a, n_blocks, st);
}

}  // namespace

int stats_blocks(int64_t n_tokens, bool sweep) {
    // about 4 tokens per wave in blocks of two waves (the sweep's partials
    // hold every support, so its grid is capped lower)
    int64_t b = (n_tokens + 7) / 8;
    const int64_t cap = sweep ? kMaxStatsBlocks / 2 : kMaxStatsBlocks;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (int)b;
}

hipError_t launch_stats(const StatsArgs& a, int n_blocks, int dtype, int head_dim, int layout, bool sweep,
                        hipStream_t st) {
    if (sweep)
        return dtype == 1 ? launch_sweep_bf16(a, n_blocks, head_dim, layout, st)
                          : launch_sweep_f32(a, n_blocks, head_dim, layout, st);
#define RRP_DISPATCH(E, D, LY) \
    if (head_dim == D && layout == LY) return launch_t<E, D, LY>(a, n_blocks, st);
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
    hipLaunchKernelGGL(stats_final_kernel, dim3(a.n_sets * kNStat + 1), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace rrp
