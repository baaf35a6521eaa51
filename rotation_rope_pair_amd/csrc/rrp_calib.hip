// rrp_calib.hip -- calibration pass: fp64 post-RoPE pair moments pooled over
// heads and tokens, then the closed-form minimax-variance angle per pair.
//
// Blocks [0, nbq) accumulate the Q stream, blocks [nbq, nbq + nbk) the K
// stream.  Each wave walks tokens with a fixed stride; every lane keeps fp64
// sums for the CE pairs whose two channels it holds (n is known on the host).
// A wave's row groups are folded with lane shuffles, the block's waves through
// LDS, both in a fixed order; block partials go to a scratch array that a
// single-block kernel sums in block order -- so the moments are bit-identical
// from run to run.
#include "rrp_device.hpp"
#include "rrp_kernels.hpp"

namespace rrp {

namespace {

constexpr int kNSum = 5;  // sum u, sum v, sum u^2, sum v^2, sum u*v

template <typename E, int D, int LAYOUT, int MAXP>
__global__ __launch_bounds__(256) void calib_moments_kernel(const CalibArgs a) {
    using G = Geo<E, D>;
    constexpr int CE = G::CE, P = G::P, L = G::L, R = G::R;
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr size_t ROWB = (size_t)D * EB;
    __shared__ double2 tab_all[4][P];
    __shared__ double red[4][P][kNSum];

    const int lane = (int)__lane_id();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nwave = (int)(blockDim.x >> 6);
    const int s = lane & (L - 1);
    const int grp = lane / L;
    double2* tab = tab_all[wave];

    const bool is_k = (int)blockIdx.x >= a.nbq;
    const int bs = is_k ? (int)blockIdx.x - a.nbq : (int)blockIdx.x;
    const int nb = is_k ? a.nbk : a.nbq;
    const unsigned char* src = static_cast<const unsigned char*>(is_k ? a.k : a.q);
    const int nh = is_k ? a.hk : a.hq;
    const int npass = (nh + R - 1) / R;
    const float invf = lane < P ? a.inv_freq[lane] : 0.0f;
    int kidx[CE];
    pair_index_of_lane<D, LAYOUT, CE>(s, kidx);

    double acc[CE][kNSum];
#pragma unroll
    for (int j = 0; j < CE; ++j)
#pragma unroll
        for (int m = 0; m < kNSum; ++m) acc[j][m] = 0.0;

    for (int64_t t = (int64_t)bs * nwave + wave; t < a.n_tokens; t += (int64_t)nb * nwave) {
        const int p = a.pos[t];
        double c[CE], sn[CE];
        for (int p0 = 0; p0 < npass; p0 += MAXP) {
            u32x4 raw[MAXP][2];
#pragma unroll
            for (int i = 0; i < MAXP; ++i) {
                const int row = (p0 + i) * R + grp;
                if (p0 + i < npass && row < nh) {
                    const unsigned char* rp = src + ((size_t)t * nh + row) * ROWB;
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch)
                        raw[i][ch] = __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4*>(rp + chunk_offset<E, D>(ch, s)));
                } else {
                    raw[i][0] = raw[i][1] = u32x4{0, 0, 0, 0};
                }
            }
            if (p0 == 0) {
                if (lane < P) {
                    double sa, ca;
                    sincos_f64_of_f32(rope_angle_f32(p, invf), sa, ca);
                    tab[lane] = make_double2(ca, sa);
                }
                wave_lds_sync();
#pragma unroll
                for (int j = 0; j < CE; ++j) {
                    const double2 v = tab[kidx[j]];
                    c[j] = v.x;
                    sn[j] = v.y;
                }
                wave_lds_sync();
            }
#pragma unroll
            for (int i = 0; i < MAXP; ++i) {
                const int row = (p0 + i) * R + grp;
                if (!(p0 + i < npass)) break;
                if (row >= nh) continue;
                float x[2][CE];
                unpack_chunk<E, CE>(raw[i][0], x[0]);
                unpack_chunk<E, CE>(raw[i][1], x[1]);
#pragma unroll
                for (int j = 0; j < CE; ++j) {
                    double xa, xb;
                    if constexpr (LAYOUT == 0) {
                        xa = x[0][j];
                        xb = x[1][j];
                    } else {
                        const int ch = j / (CE / 2), i2 = 2 * (j % (CE / 2));
                        xa = x[ch][i2];
                        xb = x[ch][i2 + 1];
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
        }
    }

    // Fold the wave's R row groups (lanes s, s + L, s + 2L, ...) in a fixed order.
#pragma unroll
    for (int m = L; m < 64; m <<= 1)
#pragma unroll
        for (int j = 0; j < CE; ++j)
#pragma unroll
            for (int q = 0; q < kNSum; ++q) acc[j][q] += shfl_xor_d(acc[j][q], m);
    if (grp == 0) {
#pragma unroll
        for (int j = 0; j < CE; ++j)
#pragma unroll
            for (int q = 0; q < kNSum; ++q) red[wave][kidx[j]][q] = acc[j][q];
    }
    __syncthreads();
    for (int e = (int)threadIdx.x; e < P * kNSum; e += (int)blockDim.x) {
        double sum = 0.0;
        for (int w = 0; w < nwave; ++w) sum += (&red[w][0][0])[e];
        a.partials[(size_t)blockIdx.x * P * kNSum + e] = sum;
    }
}

// One block: 2 * P * 5 threads sum the block partials of their (stream, pair,
// sum) in block order, add them to the caller's moments, then P threads
// finalise the angles from the accumulated moments.
__global__ __launch_bounds__(1024) void calib_final_kernel(const CalibFinalArgs a) {
    __shared__ double M[2][kMaxPairs][6];
    const int P = a.n_pairs;
    const int tid = (int)threadIdx.x;
    if (tid < 2 * P * kNSum) {
        const int stream = tid / (P * kNSum);
        const int rem = tid % (P * kNSum);
        const int k = rem / kNSum, j = rem % kNSum;
        const int b0 = stream ? a.nbq : 0;
        const int nb = stream ? a.nbk : a.nbq;
        double* mom = a.moments + ((size_t)k * 2 + stream) * 6;
        double val = mom[1 + j];
        if (nb > 0) {
            double sum = 0.0;
            for (int b = 0; b < nb; ++b) sum += a.partials[((size_t)(b0 + b) * P + k) * kNSum + j];
            val += sum;
            mom[1 + j] = val;
        }
        M[stream][k][1 + j] = val;
        if (j == 0) {
            double n = mom[0];
            if (nb > 0) {
                n += stream ? a.n_rows_k : a.n_rows_q;
                mom[0] = n;
            }
            M[stream][k][0] = n;
        }
    }
    __syncthreads();
    if (a.angles_out == nullptr || tid >= P) return;
    const double* mq = M[0][tid];
    const double* mk = M[1][tid];
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
    a.angles_out[tid] = (float)phi;
}

template <typename E, int D, int LAYOUT>
hipError_t launch_t(const CalibArgs& a, hipStream_t st) {
    constexpr int MAXP = 4;
    const int blocks = a.nbq + a.nbk;
    hipLaunchKernelGGL((calib_moments_kernel<E, D, LAYOUT, MAXP>), dim3(blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int calib_blocks(int64_t n_tokens, bool with_q, int hq, int hk, int* nbq, int* nbk) {
    // About 8 tokens per wave per stream, at most kMaxReduceBlocks blocks, split
    // between the streams in proportion to their rows.
    int64_t want = (n_tokens * (with_q ? 2 : 1) + 31) / 32;
    if (want < (with_q ? 2 : 1)) want = with_q ? 2 : 1;
    if (want > kMaxReduceBlocks) want = kMaxReduceBlocks;
    const int total = (int)want;
    if (!with_q || hq == 0) {
        *nbq = 0;
        *nbk = total;
    } else {
        int q = (int)((int64_t)total * hq / (hq + hk));
        if (q < 1) q = 1;
        if (q > total - 1) q = total - 1;
        *nbq = q;
        *nbk = total - q;
    }
    return *nbq + *nbk;
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
    const int threads = ((2 * a.n_pairs * kNSum + 63) / 64) * 64;
    hipLaunchKernelGGL(calib_final_kernel, dim3(1), dim3(threads), 0, st, a);
    return hipGetLastError();
}

}  // namespace rrp
