// rrp_stats.hip -- diagnostic pass: K range and quantisation error of the
// transformed K rows at one support b.
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

// SMALLG: groups smaller than one 16-byte chunk (reduced in registers).
template <typename E, int D, int LAYOUT, int BT, bool SMALLG>
__global__ __launch_bounds__(256) void stats_kernel(const StatsArgs a) {
    using G = Geo<E, D>;
    using LM = LaneMap<G::L>;
    constexpr int CE = G::CE, P = G::P, R = G::R;
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr size_t ROWB = (size_t)D * EB;
    constexpr bool FOLD = (LAYOUT == 0) && (BT == D);
    __shared__ float2 tab32_all[4][P];
    __shared__ double2 tab64_all[4][P];
    __shared__ double red[4][kNStat];

    const int lane = (int)__lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwave = (int)(blockDim.x >> 6);
    const int s = LM::s_of(lane);
    const int grp = LM::grp_of(lane);
    float2* tab32 = tab32_all[wave];
    double2* tab64 = tab64_all[wave];

    double cphi = 1.0, sphi = 0.0;
    if (a.angles != nullptr && lane < P) sincos_f64_of_f32(a.angles[lane], sphi, cphi);
    const float invf = lane < P ? a.inv_freq[lane] : 0.0f;
    const int s_src = s ^ lane_perm_mask<D, CE>(BT ? BT : a.support_b);  // permuted loads, see fwht_row
    int kidx[CE];
    pair_index_of_lane<D, LAYOUT, CE>(s_src, kidx);
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

    double accE = 0.0, accN = 0.0, accM = 0.0, maxM = 0.0, accR = 0.0;
    int64_t t = (int64_t)blockIdx.x * nwave + wave;
    int ps = 0;
    u32x4 cur[2], nxt[2];
    if (t < a.n_tokens) load_pass(t, 0, cur);
    while (t < a.n_tokens) {
        // keep the next pass (this token's or the next token's first) in flight
        int64_t tn = t;
        int pn = ps + 1;
        if (pn == npass) {
            tn = t + stride;
            pn = 0;
        }
        if (tn < a.n_tokens) load_pass(tn, pn, nxt);
        if (ps == 0) token_tables<D, FOLD>(tab32, tab64, lane, a.pos[t], invf, cphi, sphi, a.rsqrt_b);
        if (ps * R + grp < a.hk) {
            float yf[2][CE];
            unpack_chunk<E, CE>(cur[0], yf[0]);
            unpack_chunk<E, CE>(cur[1], yf[1]);
            double y[2][CE];
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int i2 = 0; i2 < CE; ++i2) y[ch][i2] = (double)yf[ch][i2];
            rotate_lds<LAYOUT, FOLD>(y, tab64, kidx);
            fwht_row<D, CE, BT, FOLD>(y, a.support_b, s);
            if constexpr (!SMALLG) {
                // one group value per chunk: absmax, max, min over the group
                double ca[2], cx[2], cn[2];
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    ca[ch] = 0.0;
                    cx[ch] = y[ch][0];
                    cn[ch] = y[ch][0];
#pragma unroll
                    for (int i2 = 0; i2 < CE; ++i2) {
                        ca[ch] = fmax(ca[ch], fabs(y[ch][i2]));
                        cx[ch] = fmax(cx[ch], y[ch][i2]);
                        cn[ch] = fmin(cn[ch], y[ch][i2]);
                    }
                }
                group_reduce_chunkwise<D, CE, true>(ca, g);
                group_reduce_chunkwise<D, CE, true>(cx, g);
                group_reduce_chunkwise<D, CE, false>(cn, g);
#pragma unroll
                for (int ch = 0; ch < 2; ++ch) {
                    const GroupScale64 gs = group_scale64(ca[ch]);
#pragma unroll
                    for (int i2 = 0; i2 < CE; ++i2) {
                        const double diff = (double)code_of(y[ch][i2], gs.rcp) * gs.shv - y[ch][i2];
                        accE += diff * diff;
                        accN += y[ch][i2] * y[ch][i2];
                    }
                    if (((ch * P + s * CE) & (g - 1)) == 0) {  // the lane holding the group's first channel
                        accM += ca[ch];
                        maxM = fmax(maxM, ca[ch]);
                        accR += cx[ch] - cn[ch];
                    }
                }
            } else {
                double am[2][CE], mx[2][CE], mn[2][CE];
#pragma unroll
                for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                    for (int i2 = 0; i2 < CE; ++i2) {
                        am[ch][i2] = fabs(y[ch][i2]);
                        mx[ch][i2] = y[ch][i2];
                        mn[ch][i2] = y[ch][i2];
                    }
                group_reduce_inreg<CE, true>(am, g);
                group_reduce_inreg<CE, true>(mx, g);
                group_reduce_inreg<CE, false>(mn, g);
#pragma unroll
                for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                    for (int i2 = 0; i2 < CE; ++i2) {
                        const GroupScale64 gs = group_scale64(am[ch][i2]);
                        const double diff = (double)code_of(y[ch][i2], gs.rcp) * gs.shv - y[ch][i2];
                        accE += diff * diff;
                        accN += y[ch][i2] * y[ch][i2];
                        if ((i2 & (g - 1)) == 0) {
                            accM += am[ch][i2];
                            maxM = fmax(maxM, am[ch][i2]);
                            accR += mx[ch][i2] - mn[ch][i2];
                        }
                    }
            }
        }
        cur[0] = nxt[0];
        cur[1] = nxt[1];
        t = tn;
        ps = pn;
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        accE += shfl_xor_d(accE, m);
        accN += shfl_xor_d(accN, m);
        accM += shfl_xor_d(accM, m);
        maxM = fmax(maxM, shfl_xor_d(maxM, m));
        accR += shfl_xor_d(accR, m);
    }
    if (lane == 0) {
        red[wave][0] = accE;
        red[wave][1] = accN;
        red[wave][2] = accM;
        red[wave][3] = maxM;
        red[wave][4] = accR;
    }
    __syncthreads();
    if (threadIdx.x < kNStat) {
        const int e = (int)threadIdx.x;
        double v = red[0][e];
        for (int w = 1; w < nwave; ++w) v = (e == 3) ? fmax(v, red[w][e]) : v + red[w][e];
        a.partials[(size_t)e * gridDim.x + blockIdx.x] = v;
    }
}

// One wave per statistic: lane l combines the partials of blocks l, l + 64, ...
// in order, then a fixed xor butterfly folds the lanes (every lane ends with
// the same value).  Partials are laid out [statistic][block].
__global__ __launch_bounds__(512) void stats_final_kernel(const StatsFinalArgs a) {
    const int e = (int)(threadIdx.x >> 6);
    const int lane = (int)__lane_id();
    if (e < kNStat) {
        const double* part = a.partials + (size_t)e * a.n_blocks;
        double v = 0.0;
        for (int b = lane; b < a.n_blocks; b += 64) v = (e == 3) ? fmax(v, part[b]) : v + part[b];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const double o = shfl_xor_d(v, m);
            v = (e == 3) ? fmax(v, o) : v + o;
        }
        if (lane == 0) a.stats_out[e] = v;
    } else if (e == kNStat && lane == 0) {
        a.stats_out[5] = a.n_groups;
        a.stats_out[6] = a.n_rows;
        a.stats_out[7] = 0.0;
    }
}

template <typename E, int D, int LAYOUT>
hipError_t launch_t(const StatsArgs& a, int n_blocks, hipStream_t st) {
    constexpr int CE = Geo<E, D>::CE;
    const bool small = a.group < CE;
#define RRP_LAUNCH(BT, SG) \
    hipLaunchKernelGGL((stats_kernel<E, D, LAYOUT, BT, SG>), dim3(n_blocks), dim3(256), 0, st, a)
    if (a.support_b == D) {
        if (small) RRP_LAUNCH(D, true); else RRP_LAUNCH(D, false);
    } else {
        if (small) RRP_LAUNCH(0, true); else RRP_LAUNCH(0, false);
    }
#undef RRP_LAUNCH
    return hipGetLastError();
}

}  // namespace

int stats_blocks(int64_t n_tokens) {
    int64_t b = (n_tokens + 15) / 16;  // about 4 tokens per wave
    if (b < 1) b = 1;
    if (b > kMaxStatsBlocks) b = kMaxStatsBlocks;
    return (int)b;
}

hipError_t launch_stats(const StatsArgs& a, int n_blocks, int dtype, int head_dim, int layout, hipStream_t st) {
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
    hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(64 * (kNStat + 1)), 0, st, a);
    return hipGetLastError();
}

}  // namespace rrp
