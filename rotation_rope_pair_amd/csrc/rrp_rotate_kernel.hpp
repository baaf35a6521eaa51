// rrp_rotate_kernel.hpp -- the fused rotate + quantise kernel template and its
// launcher, shared by the two translation units that instantiate it (large
// batches: one wave per token; small batches: a token's row passes split over
// several waves).  Everything here has internal linkage.
#pragma once

#include "rrp_device.hpp"
#include "rrp_rotate.hpp"

namespace rrp {

namespace {

// K and V rows are transformed and quantised in fp64: the group scales and
// codes are integer decisions taken from y, made in the precision of their
// definition for every group size.
typedef double KV;

// Quantise one K row held as y[2][CE] (output order) in lane s; write codes / scales.
// SMALLG: groups smaller than one 16-byte chunk (g < CE), reduced in registers.
template <int D, int CE, bool SMALLG>
__device__ __forceinline__ void quantize_store_k_row(const KV (&y)[2][CE], int s, int group,
                                                     uint8_t* __restrict__ codes_row,
                                                     uint16_t* __restrict__ scales_row,
                                                     float* __restrict__ s_dbg_row, bool write_cache) {
    constexpr int P = D / 2;
    unsigned word[2] = {0u, 0u};  // nibble-packed codes of each chunk
    if constexpr (!SMALLG) {
        KV m[2];
        k_group_absmax_chunks<D, CE>(y, group, m);
        GroupScale64 gs[2];
        gs[0] = group_scale64(m[0]);
        if (group > P) gs[1] = gs[0];  // one group spans both halves: same scale
        else gs[1] = group_scale64(m[1]);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
            for (int i = 0; i < CE; ++i) word[ch] |= ((unsigned)code_of(y[ch][i], gs[ch].rcp) & 0xFu) << (4 * i);
            const int c0 = ch * P + s * CE;
            if ((c0 & (group - 1)) == 0) {  // this lane holds the group's first channel
                const int j = c0 / group;
                if (write_cache) scales_row[j] = gs[ch].sh;
                if (s_dbg_row) s_dbg_row[j] = gs[ch].s32;
            }
        }
    } else {
        KV m[2][CE];
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int i = 0; i < CE; ++i) m[ch][i] = fabs(y[ch][i]);
        group_reduce_inreg<CE, true>(m, group);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int i = 0; i < CE; ++i) {
                const GroupScale64 gs = group_scale64(m[ch][i]);
                word[ch] |= ((unsigned)code_of(y[ch][i], gs.rcp) & 0xFu) << (4 * i);
                if ((i & (group - 1)) == 0) {
                    const int j = (ch * P + s * CE + i) / group;
                    if (write_cache) scales_row[j] = gs.sh;
                    if (s_dbg_row) s_dbg_row[j] = gs.s32;
                }
            }
    }
    if (!write_cache) return;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        const int byte0 = (ch * P + s * CE) / 2;
        if constexpr (CE == 8)
            __builtin_nontemporal_store(word[ch], reinterpret_cast<unsigned*>(codes_row + byte0));
        else
            __builtin_nontemporal_store((unsigned short)word[ch], reinterpret_cast<unsigned short*>(codes_row + byte0));
    }
}

template <typename E, int D>
__device__ __forceinline__ void load_row_chunks(const unsigned char* __restrict__ row, int s_src, u32x4 (&r)[2]) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
        r[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + chunk_offset<E, D>(ch, s_src)));
}

// Direct global -> LDS loads of one row pass (gfx950 global_load_lds_dwordx4):
// lane i's 16 bytes of chunk ch land at dst[ch][i].  The data holds no VGPRs
// while in flight; the caller waits on vmcnt before reading dst.
template <typename E, int D>
__device__ __forceinline__ void stage_row_chunks(const unsigned char* __restrict__ row, int s_src, u32x4 (*dst)[64]) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(row + chunk_offset<E, D>(ch, s_src)),
                                         (__attribute__((address_space(3))) void*)(dst[ch]), 16, 0, 0);
}

// Row passes kept in VGPRs per token: one Q pass (two Q passes measured
// slower: 155 instead of 136 VGPRs, two instead of three waves per SIMD) and
// one K pass (two when a pass holds fewer than 8 rows).  Q/K launches with
// shared angles also have the next kStagedQPasses Q passes in flight, in LDS.
template <int R> struct Depth {
    static constexpr int Q = 1;
    static constexpr int K = R >= 8 ? 1 : 2;
};

// BT: compile-time Hadamard support (BT == D, the full-head case) or 0 (runtime b).
// HAS_V: also turn the V rows by the full-head Hadamard and quantise them into
// the V half of the cache (no RoPE, no pair rotation).
// PH: one angle set per key head (a.angle_sets = Hkv of them); query head h uses
// set h * sets / Hq, key head kh set kh.  Each wave keeps the fp64 tables of
// every set (9 KB) and Q rounds its entries to fp32 as it reads them (the values
// of the shared path's fp32 table); with the block's cos / sin of the sets
// (9 KB), blocks of kPerSetWaves = 4 waves take 46 KB, three per CU.
// SPLIT: each token's row passes are shared by a.split waves (small batches).
constexpr int kPerSetWaves = 4;
// Q passes staged through LDS per token (after the first, which goes to VGPRs).
constexpr int kStagedQPasses = 3;

template <typename E, int D, int LAYOUT, bool SMALLG, int BT, bool HAS_V, bool PH, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(1, PH ? 64 * kPerSetWaves : 256)))
void rotate_quantize_kernel(const RotateArgs a) {
    using G = Geo<E, D>;
    using LM = LaneMap<G::L>;
    constexpr int CE = G::CE, P = G::P, R = G::R;
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr int ROWB = D * EB;
    constexpr int MQ = Depth<R>::Q, MK = Depth<R>::K;
    static_assert(MQ == 1 || SPLIT || PH || HAS_V, "Q staging assumes one Q pass in flight");
    constexpr bool FOLD = (LAYOUT == 0) && (BT == D);
    constexpr int WMAX = PH ? kPerSetWaves : 4;  // waves per block
    __shared__ float2 tab32_all[WMAX][PH ? 1 : tab_entries<P>()];
    __shared__ double2 tab64_all[WMAX][PH ? kSetStride * P : tab_entries<P>()];
    __shared__ double2 phi_all[PH ? kSetStride * P : 1];
    // STAGE (Q/K with shared angles, one token per wave): the token's Q passes
    // after the first go straight to LDS at the token's start, so every row of
    // the token is in flight at once without holding VGPRs.
    constexpr bool STAGE = !SPLIT && !PH && !HAS_V;
    constexpr int NS = STAGE ? kStagedQPasses : 1;
    __shared__ u32x4 stage_all[STAGE ? WMAX : 1][NS][2][64];

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
    const float invf = lane < P ? a.inv_freq[lane] : 0.0f;
    if constexpr (STAGE) asm volatile("" ::"v"(invf), "v"(cphi), "v"(sphi));  // retired before the first row loads
    // Rows are loaded permuted (lane s holds position s ^ perm), see fwht_row.
    const int s_src = s ^ lane_perm_mask<D, CE>(BT ? BT : a.support_b);
    const int s_src_v = s ^ lane_perm_mask<D, CE>(D);  // V: full-head support
    int kidx[CE];
    pair_index_of_lane<D, LAYOUT, CE>(s_src, kidx);
    if constexpr (PH) {
#pragma unroll
        for (int j = 0; j < CE; ++j) kidx[j] *= kSetStride;  // pair-major per-set tables
    } else {
#pragma unroll
        for (int j = 0; j < CE; ++j) kidx[j] = tab_index(kidx[j]);  // padded shared table
    }

    const int hq = a.hq_rows, hk = a.hk;
    const int nq = (hq + R - 1) / R, nk = (hk + R - 1) / R;
    const int ngroups = D / a.group;
    const unsigned char* qb = static_cast<const unsigned char*>(a.q);
    const unsigned char* kb = static_cast<const unsigned char*>(a.k);
    const unsigned char* vb = static_cast<const unsigned char*>(a.v);
    unsigned char* qo = static_cast<unsigned char*>(a.q_out);
    const int ld_off = grp * ROWB;  // this lane's row inside a pass

    // A token's row passes, in the order Q, K, V, are split over a.split waves
    // (one wave per token for large batches); wave unit u takes token u / split
    // and the passes [j * N / split, (j + 1) * N / split) of it, j = u % split.
    const int split = SPLIT ? a.split : 1;
    const int npass = nq + (HAS_V ? 2 : 1) * nk;
    const int64_t n_units = SPLIT ? a.n_tokens * split : a.n_tokens;
    for (int64_t u = (int64_t)blockIdx.x * nwave + wave; u < n_units; u += (int64_t)gridDim.x * nwave) {
        int64_t t = u;
        int q0 = 0, q1 = nq, k0 = 0, k1 = nk, v0 = 0, v1 = nk;
        if constexpr (SPLIT) {
            t = u / split;
            const int j = (int)(u - t * split);
            const int u0 = j * npass / split, u1 = (j + 1) * npass / split;
            q0 = min(u0, nq);
            q1 = min(u1, nq);
            k0 = min(max(u0 - nq, 0), nk);
            k1 = min(max(u1 - nq, 0), nk);
            v0 = min(max(u0 - nq - nk, 0), nk);
            v1 = min(max(u1 - nq - nk, 0), nk);
        }
        // A wave walking several tokens: the previous token's accesses have
        // completed (its reads of the staging buffer included), and the
        // compiler knows it, so no load of this token waits on a register of
        // the last one.  Free for the first token.
        if constexpr (STAGE) wait_vm_lds_all();
        // wave-uniform row bases of this token
        const unsigned char* qt = qb + (size_t)t * a.hq * ROWB;
        const unsigned char* kt = kb + (size_t)t * hk * ROWB;
        const unsigned char* vt = vb + (size_t)t * hk * ROWB;
        unsigned char* qot = qo + (size_t)t * a.hq * ROWB;

        // Issue the loads of the first MQ Q passes and MK K passes (and V passes).
        u32x4 rq[MQ][2], rk[MK][2], rv[HAS_V ? MK : 1][2];
#pragma unroll
        for (int i = 0; i < MQ; ++i)
            if (q0 + i < q1 && (q0 + i) * R + grp < hq)
                load_row_chunks<E, D>(qt + (q0 + i) * R * ROWB + ld_off, s_src, rq[i]);
#pragma unroll
        for (int i = 0; i < MK; ++i)
            if (k0 + i < k1 && (k0 + i) * R + grp < hk)
                load_row_chunks<E, D>(kt + (k0 + i) * R * ROWB + ld_off, s_src, rk[i]);
        if constexpr (HAS_V) {
#pragma unroll
            for (int i = 0; i < MK; ++i)
                if (v0 + i < v1 && (v0 + i) * R + grp < hk)
                    load_row_chunks<E, D>(vt + (v0 + i) * R * ROWB + ld_off, s_src_v, rv[i]);
        }
        // Q passes q0 + 1 .. q0 + ns go to LDS (STAGE only).
        int ns = 0;
        if constexpr (STAGE) {
            ns = min(q1 - q0 - 1, NS);
#pragma unroll
            for (int i = 0; i < NS; ++i)
                if (i < ns && (q0 + 1 + i) * R + grp < hq)
                    stage_row_chunks<E, D>(qt + (q0 + 1 + i) * R * ROWB + ld_off, s_src, stage_all[wave][i]);
            asm volatile("" ::: "memory");  // issue order: before the table build and the first stores
        }
        // Position and slot after the row loads: the first wait on them then
        // covers the rows too, and no row load waits for them.
        const int p = a.pos[t];
        const int64_t slot = a.slot_mapping ? a.slot_mapping[t] : t;
        const bool in_cache = slot >= 0 && slot < a.n_slots;

        if constexpr (PH)
            token_tables_sets<D, FOLD>(nullptr, tab64, lane, p, invf, phi_all, a.angle_sets, a.rsqrt_b);
        else token_tables<D, FOLD>(tab32, tab64, lane, p, invf, cphi, sphi, a.rsqrt_b);
        // Every row of the token has landed.  The table build has already
        // waited for the position, issued after them, so this adds no wait of
        // its own; unconditional, so the compiler knows it on every path.
        if constexpr (STAGE) wait_vm_all();

        // ---- Q rows (fp32) ----
        for (int c0 = q0; c0 < q1; c0 += MQ) {
            const int si = c0 - q0 - 1;  // staging slot of this pass (STAGE, MQ == 1)
            if (STAGE && si >= 0 && si < ns) {
                if (c0 * R + grp < hq) {
                    rq[0][0] = stage_all[wave][si][0][lane];
                    rq[0][1] = stage_all[wave][si][1][lane];
                }
            } else if (c0 > q0) {
#pragma unroll
                for (int i = 0; i < MQ; ++i)
                    if (c0 + i < q1 && (c0 + i) * R + grp < hq)
                        load_row_chunks<E, D>(qt + (c0 + i) * R * ROWB + ld_off, s_src, rq[i]);
            }
#pragma unroll
            for (int i = 0; i < MQ; ++i) {
                const int pass = c0 + i;
                if (pass >= q1) break;
                const int h = pass * R + grp;
                if (h >= hq) continue;
                float x[2][CE];
                unpack_chunk<E, CE>(rq[i][0], x[0]);
                unpack_chunk<E, CE>(rq[i][1], x[1]);
                if constexpr (PH) {
                    // set of query head h: floor((h + 1/2) * sets / Hq), exact in fp32
                    const int qset = (int)(((float)h + 0.5f) * a.q_set_scale);
                    rotate_lds<LAYOUT, FOLD>(x, tab64 + qset, kidx);
                } else {
                    rotate_lds<LAYOUT, FOLD>(x, tab32, kidx);
                }
                fwht_row<D, CE, BT, FOLD>(x, a.support_b, s);
                if (qo) {
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch)
                        __builtin_nontemporal_store(pack_chunk<E, CE>(x[ch]),
                            reinterpret_cast<u32x4*>(qot + (h * ROWB + chunk_offset<E, D>(ch, s))));
                }
                if (a.q_dbg) {
                    float* dst = a.q_dbg + ((size_t)t * a.hq + h) * D;
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                        for (int i2 = 0; i2 < CE; ++i2) dst[ch * P + s * CE + i2] = x[ch][i2];
                }
            }
        }

        // ---- K rows (KV precision) ----
        __builtin_amdgcn_sched_barrier(0);  // keep the K phase's LDS reads out of the Q phase
        for (int c0 = k0; c0 < k1; c0 += MK) {
            if (c0 > k0) {
#pragma unroll
                for (int i = 0; i < MK; ++i)
                    if (c0 + i < k1 && (c0 + i) * R + grp < hk)
                        load_row_chunks<E, D>(kt + (c0 + i) * R * ROWB + ld_off, s_src, rk[i]);
            }
#pragma unroll
            for (int i = 0; i < MK; ++i) {
                const int pass = c0 + i;
                if (pass >= k1) break;
                const int h = pass * R + grp;
                if (h >= hk) continue;
                float xf[2][CE];
                unpack_chunk<E, CE>(rk[i][0], xf[0]);
                unpack_chunk<E, CE>(rk[i][1], xf[1]);
                KV x[2][CE];
#pragma unroll
                for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                    for (int i2 = 0; i2 < CE; ++i2) x[ch][i2] = (KV)xf[ch][i2];
                const int kset = PH ? h : 0;  // key head h uses set h
                rotate_lds<LAYOUT, FOLD>(x, tab64 + kset, kidx);
                fwht_row<D, CE, BT, FOLD>(x, a.support_b, s);
                const size_t trow = (size_t)t * hk + h;
                if (a.k_dbg) {
                    float* dst = a.k_dbg + trow * D;
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                        for (int i2 = 0; i2 < CE; ++i2) dst[ch * P + s * CE + i2] = (float)x[ch][i2];
                }
                const size_t crow = in_cache ? (size_t)slot * hk + h : 0;
                quantize_store_k_row<D, CE, SMALLG>(x, s, a.group, a.k_codes + crow * (D / 2),
                                                    a.k_scales + crow * ngroups,
                                                    a.s_dbg ? a.s_dbg + trow * ngroups : nullptr, in_cache);
            }
        }

        // ---- V rows (KV precision): H_D / sqrt(D), then the K quantiser ----
        if constexpr (HAS_V) {
            for (int c0 = v0; c0 < v1; c0 += MK) {
                if (c0 > v0) {
#pragma unroll
                    for (int i = 0; i < MK; ++i)
                        if (c0 + i < v1 && (c0 + i) * R + grp < hk)
                            load_row_chunks<E, D>(vt + (c0 + i) * R * ROWB + ld_off, s_src_v, rv[i]);
                }
#pragma unroll
                for (int i = 0; i < MK; ++i) {
                    const int pass = c0 + i;
                    if (pass >= v1) break;
                    const int h = pass * R + grp;
                    if (h >= hk) continue;
                    float xf[2][CE];
                    unpack_chunk<E, CE>(rv[i][0], xf[0]);
                    unpack_chunk<E, CE>(rv[i][1], xf[1]);
                    KV x[2][CE];
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                        for (int i2 = 0; i2 < CE; ++i2) x[ch][i2] = (KV)xf[ch][i2];
                    fwht_row<D, CE, D, false>(x, D, s);
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                        for (int i2 = 0; i2 < CE; ++i2) x[ch][i2] *= (KV)a.rsqrt_v;
                    const size_t trow = (size_t)t * hk + h;
                    if (a.v_dbg) {
                        float* dst = a.v_dbg + trow * D;
#pragma unroll
                        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                            for (int i2 = 0; i2 < CE; ++i2) dst[ch * P + s * CE + i2] = (float)x[ch][i2];
                    }
                    const size_t crow = in_cache ? (size_t)slot * hk + h : 0;
                    quantize_store_k_row<D, CE, SMALLG>(x, s, a.group, a.v_codes + crow * (D / 2),
                                                        a.v_scales + crow * ngroups,
                                                        a.vs_dbg ? a.vs_dbg + trow * ngroups : nullptr, in_cache);
                }
            }
        }
    }
}

// Launch one compile-time family: SPLIT = false for large batches (grid-stride
// over tokens, one wave each), SPLIT = true for small ones (each of a token's
// row passes on a wave of its own, so a decode batch is not serialised on one
// wave per token).  The split family takes batches of at most kSmallBatchWaves
// passes in all.
constexpr int kSmallBatchWaves = 4096;
// Grid caps of the large-batch family; past them waves walk several tokens each.
// Q/K with shared angles: 32K blocks of 4 waves, one token per wave up to 128K
// tokens, so the running waves sweep the batch in token order (at the 128K
// prefill 428 us, against 432 us at 8K blocks and 441 us at 4K).  With V rows
// or per-set angles, a token is more work and 8K blocks measured best (32K:
// 0.534 against 0.515 ms with V; 530 against 483 us per set).
constexpr int64_t kMaxRotateBlocks = 8192;
constexpr int64_t kMaxRotateBlocksQK = 32768;

template <typename E, int D, int LAYOUT, bool SPLIT>
hipError_t launch_t(const RotateArgs& args, hipStream_t st) {
    RotateArgs a = args;
    const bool ph = a.angle_sets > 1;
    // Small batches (the split family): one wave per block so the work spreads
    // over all CUs.  One wave per token: blocks of 4 waves at any batch size
    // (2048 tokens at d 64 took 11.8 us with 1-wave blocks, 7.8 us with 4).
    const int wpb = SPLIT ? 1 : (ph ? kPerSetWaves : 4);
    a.split = 1;
    if constexpr (SPLIT) {
        constexpr int R = Geo<E, D>::R;
        const int nq = (a.hq_rows + R - 1) / R, nk = (a.hk + R - 1) / R;
        const int npass = nq + (a.v != nullptr ? 2 : 1) * nk;
        int64_t split = (kSmallBatchWaves + a.n_tokens - 1) / (a.n_tokens > 0 ? a.n_tokens : 1);
        if (split > npass) split = npass;
        a.split = split < 1 ? 1 : (int)split;
    }
    int64_t blocks = (a.n_tokens * a.split + wpb - 1) / wpb;
    const int64_t cap = (!SPLIT && !ph && a.v == nullptr) ? kMaxRotateBlocksQK : kMaxRotateBlocks;
    if (blocks > cap) blocks = cap;
    const bool smallg = a.group < Geo<E, D>::CE;
    const dim3 grid((unsigned)blocks), block(64 * wpb);
#define RRP_LAUNCH(SG, BT, HV, PHV) \
    hipLaunchKernelGGL((rotate_quantize_kernel<E, D, LAYOUT, SG, BT, HV, PHV, SPLIT>), grid, block, 0, st, a)
#define RRP_LAUNCH_B(SG, HV, PHV)                       \
    if (a.support_b == D) { RRP_LAUNCH(SG, D, HV, PHV); } \
    else { RRP_LAUNCH(SG, 0, HV, PHV); }
#define RRP_LAUNCH_P(SG, HV)                        \
    if (ph) { RRP_LAUNCH_B(SG, HV, true); } else { RRP_LAUNCH_B(SG, HV, false); }
    if (a.v != nullptr) {
        if (smallg) { RRP_LAUNCH_P(true, true); } else { RRP_LAUNCH_P(false, true); }
    } else {
        if (smallg) { RRP_LAUNCH_P(true, false); } else { RRP_LAUNCH_P(false, false); }
    }
#undef RRP_LAUNCH_P
#undef RRP_LAUNCH_B
#undef RRP_LAUNCH
    return hipGetLastError();
}

template <bool SPLIT>
hipError_t dispatch(const RotateArgs& a, int dtype, int head_dim, int layout, hipStream_t st) {
#define RRP_DISPATCH(E, D, LY) \
    if (head_dim == D && layout == LY) return launch_t<E, D, LY, SPLIT>(a, st);
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

}  // namespace

}  // namespace rrp
