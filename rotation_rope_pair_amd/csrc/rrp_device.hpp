// rrp_device.hpp -- device building blocks for gfx950 (CDNA4, wave64).
//
// Row layout in registers.  One attention-head row (head_dim = D channels) is
// spread over L = D / (2 * CE) lanes; CE = 16 / sizeof(elem) is the number of
// channels in one 16-byte chunk.  A lane at row position s holds two chunks:
//   chunk 0: channels [s*CE, s*CE + CE)            (lower half of the head)
//   chunk 1: channels [D/2 + s*CE, D/2 + s*CE + CE) (upper half of the head)
// so both channels of a half-split RoPE pair (k, k + D/2) sit in the same lane
// and every global access is one 128-bit load or store per chunk.  A wave holds
// R = 64 / L rows at once ("a pass").
//
// Channel index c = ch * D/2 + s * CE + i.  A Walsh-Hadamard butterfly on bit
// j of c is in-register for the bits of i and ch and a lane exchange (DPP,
// inside one 16-lane DPP row) for the bits of s.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "rrp_rotate.hpp"  // kMaxAngleSets

namespace rrp {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Wait until every vector memory operation of the wave has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt fields left at "no wait").  Issued
// through the builtin, so the compiler's own wait-count tracking sees it: a
// direct global -> LDS load waited for here needs no further wait before the
// LDS reads that follow, even with stores issued in between.  The empty asm
// keeps memory accesses from moving across the wait.
__device__ __forceinline__ void wait_vm_all() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
}

// Wait until every vector memory and LDS operation of the wave has completed
// (vmcnt(0) lgkmcnt(0)), again visible to the compiler's tracking.
__device__ __forceinline__ void wait_vm_lds_all() {
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("" ::: "memory");
}

struct bf16_tag {};  // element type marker: bf16 stored as uint16 bit patterns

template <typename E> struct ElemInfo;
template <> struct ElemInfo<float> { static constexpr int bytes = 4; };
template <> struct ElemInfo<bf16_tag> { static constexpr int bytes = 2; };

template <typename E, int D>
struct Geo {
    static constexpr int CE = 16 / ElemInfo<E>::bytes;  // channels per 16-byte chunk
    static constexpr int P = D / 2;                      // RoPE pairs per row
    static constexpr int L = D / (2 * CE);               // lanes per row
    static constexpr int R = 64 / L;                     // rows per wave pass
    static_assert(L >= 1 && L <= 16 && (L & (L - 1)) == 0, "row must fit one DPP row");
};

// ---------------------------------------------------------------------------
// Lane map.  Row position s and row index inside the pass of a lane.  For
// 8-lane rows the third position bit is lane bit 3 (rows interleave in groups
// of four lanes), so every position bit is a single-instruction DPP exchange:
// quad_perm for bits 0 and 1, row_ror:8 for bit 2.
// ---------------------------------------------------------------------------
template <int L>
struct LaneMap {
    static constexpr bool SPLIT = (L == 8);
    __device__ static int s_of(int lane) { return SPLIT ? ((lane & 3) | ((lane >> 1) & 4)) : (lane & (L - 1)); }
    __device__ static int grp_of(int lane) {
        return SPLIT ? (((lane >> 2) & 1) | ((lane >> 3) & 6)) : (lane / L);
    }
    // lane-index xor realising the row-position xor M
    static constexpr int lane_mask(int M) { return (SPLIT && M == 4) ? 8 : M; }
};

// ---------------------------------------------------------------------------
// Cross-lane moves inside a 16-lane DPP row.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned v) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(unsigned, v)));
}

// 32-bit value held by lane (lane ^ M), M < 16.
template <int M>
__device__ __forceinline__ unsigned lane_xor_u32(unsigned v) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "xor within a DPP row");
    if constexpr (M == 1) return dpp_u32<0xB1>(v);                       // quad_perm [1,0,3,2]
    else if constexpr (M == 2) return dpp_u32<0x4E>(v);                  // quad_perm [2,3,0,1]
    else if constexpr (M == 4) return dpp_u32<0x1B>(dpp_u32<0x141>(v));  // half-row mirror, then quad reverse
    else return dpp_u32<0x128>(v);                                       // row_ror:8
}
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    return __builtin_bit_cast(float, lane_xor_u32<M>(__builtin_bit_cast(unsigned, v)));
}
template <int M>
__device__ __forceinline__ double lane_xor(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = lane_xor_u32<M>((unsigned)u), hi = lane_xor_u32<M>((unsigned)(u >> 32));
    return __builtin_bit_cast(double, (hi << 32) | lo);
}
// Value held by the lane of the same row at position s ^ M.
template <int L, int M, typename V>
__device__ __forceinline__ V s_xor(V v) {
    return lane_xor<LaneMap<L>::lane_mask(M)>(v);
}

// Full-wave xor shuffle (ds_bpermute) for the reductions across rows.
__device__ __forceinline__ double shfl_xor_d(double v, int m) {
    int lane = (int)__lane_id();
    uint64_t u = __builtin_bit_cast(uint64_t, v);
    int lo = __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, (int)(uint32_t)u);
    int hi = __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, (int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// LDS ordering between lanes of one wave (wave-private LDS regions).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Element formats.
// ---------------------------------------------------------------------------
template <typename E, int CE>
__device__ __forceinline__ void unpack_chunk(const u32x4& w, float (&x)[CE]) {
    if constexpr (ElemInfo<E>::bytes == 4) {
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    } else {
        const unsigned ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = __uint_as_float(ww[j] << 16);
            x[2 * j + 1] = __uint_as_float(ww[j] & 0xFFFF0000u);
        }
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16, round to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2_t));
}

template <typename E, int CE>
__device__ __forceinline__ u32x4 pack_chunk(const float (&y)[CE]) {
    u32x4 w;
    if constexpr (ElemInfo<E>::bytes == 4) {
        w.x = __float_as_uint(y[0]); w.y = __float_as_uint(y[1]);
        w.z = __float_as_uint(y[2]); w.w = __float_as_uint(y[3]);
    } else {
        w.x = pack_bf16x2(y[0], y[1]); w.y = pack_bf16x2(y[2], y[3]);
        w.z = pack_bf16x2(y[4], y[5]); w.w = pack_bf16x2(y[6], y[7]);
    }
    return w;
}

// fp32 -> fp16 (nearest even) saturated at 65504, as bits; and back.
__device__ __forceinline__ unsigned short f16_sat_bits(float s) {
    _Float16 h = (_Float16)fminf(s, 65504.0f);
    return __builtin_bit_cast(unsigned short, h);
}
__device__ __forceinline__ float f16_bits_to_f32(unsigned short b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// Byte offset of chunk `ch` of row position s inside a row.
template <typename E, int D>
__device__ __forceinline__ int chunk_offset(int ch, int s) {
    using G = Geo<E, D>;
    return (ch * G::P + s * G::CE) * ElemInfo<E>::bytes;
}

// ---------------------------------------------------------------------------
// Angles.
// ---------------------------------------------------------------------------

// The lane's RoPE frequency from the kernel argument block; the empty asm uses
// it at once, so its load is waited for here, before the token loop.  Waited
// for at its first use inside the loop instead, the wait cannot be told apart
// from the loop's own loads and takes all of them, the next token's prefetched
// rows included, on every token.
__device__ __forceinline__ float lane_inv_freq(const float* inv_freq, int lane, int n_pairs) {
    const float f = lane < n_pairs ? inv_freq[lane] : 0.0f;
    asm volatile("" ::"v"(f));
    return f;
}

// A token's position, read through the scalar unit (read-only input): its
// wait is then separate from the wave's row loads.
__device__ __forceinline__ int token_pos(const int32_t* pos, int64_t t) {
    return ((const __attribute__((address_space(4))) int32_t*)pos)[t];
}

// RoPE angle of one pair at position p: a single fp32 product, never fused.
__device__ __forceinline__ float rope_angle_f32(int p, float w) {
#pragma clang fp contract(off)
    return (float)p * w;
}

// An fp64 constant handed to an FMA from scalar registers.  Left to itself the
// compiler keeps the polynomial coefficients below in vector registers for the
// whole kernel (two per coefficient) and copies each one before every
// accumulate-form FMA; read from scalar registers they cost neither.
__device__ __forceinline__ double sreg(double c) {
    asm volatile("" : "+s"(c));
    return c;
}

// sin and cos, in fp64, of an fp32 angle with |alpha| <= 2^24 (every RoPE
// angle p * freq with p < 2^24 and freq <= 1; also the pair angles).
// Cody-Waite reduction by pi/2 (n = nearest integer to alpha * 2/pi, then
// r = alpha - n * pi/2 with pi/2 split into two doubles and each product taken
// exactly inside an FMA), followed by the Taylor series of sin and cos on
// |r| <= pi/4 up to the r^17 / r^16 terms (truncation below 1e-18), and the
// quadrant n mod 4.  Straight-line code: no branch, no table.
__device__ __forceinline__ void sincos_f64_of_f32(float alpha, double& s_out, double& c_out) {
    const double a = (double)alpha;
    const double kTwoOverPi = 0.63661977236758134308;  // 2/pi
    const double kPio2Hi = 1.5707963267948966;           // pi/2 rounded to fp64
    const double kPio2Lo = 6.123233995736766e-17;        // pi/2 - kPio2Hi, rounded
    const double n = rint(a * kTwoOverPi);
    double r = fma(-n, kPio2Hi, a);
    r = fma(-n, kPio2Lo, r);
    const double z = r * r;
    // sin r = r + r z (-1/3! + z (1/5! + z (-1/7! + ...)))
    double ps = 1.0 / 355687428096000.0;            // 1/17!
    ps = fma(ps, z, sreg(-1.0 / 1307674368000.0));  // 1/15!
    ps = fma(ps, z, sreg(1.0 / 6227020800.0));      // 1/13!
    ps = fma(ps, z, sreg(-1.0 / 39916800.0));       // 1/11!
    ps = fma(ps, z, sreg(1.0 / 362880.0));          // 1/9!
    ps = fma(ps, z, sreg(-1.0 / 5040.0));           // 1/7!
    ps = fma(ps, z, sreg(1.0 / 120.0));             // 1/5!
    ps = fma(ps, z, sreg(-1.0 / 6.0));              // 1/3!
    const double sr = fma(r * z, ps, r);
    // cos r = 1 + z (-1/2! + z (1/4! + z (-1/6! + ...)))
    double pc = 1.0 / 20922789888000.0;             // 1/16!
    pc = fma(pc, z, sreg(-1.0 / 87178291200.0));    // 1/14!
    pc = fma(pc, z, sreg(1.0 / 479001600.0));       // 1/12!
    pc = fma(pc, z, sreg(-1.0 / 3628800.0));        // 1/10!
    pc = fma(pc, z, sreg(1.0 / 40320.0));           // 1/8!
    pc = fma(pc, z, sreg(-1.0 / 720.0));            // 1/6!
    pc = fma(pc, z, sreg(1.0 / 24.0));              // 1/4!
    pc = fma(pc, z, -0.5);                          // 1/2!
    const double cr = fma(z, pc, 1.0);
    const int q = (int)n & 3;
    double sv = (q & 1) ? cr : sr;
    double cv = (q & 1) ? sr : cr;
    if (q & 2) sv = -sv;
    if ((q + 1) & 2) cv = -cv;
    s_out = sv;
    c_out = cv;
}

// ---------------------------------------------------------------------------
// Per-token rotation table, evaluated once per token in fp64 from the fp64
// (cos, sin) of the fp32 RoPE angle and of phi_k:
//   (C_k, S_k) = (cos, sin)(alpha_k + phi_k) / sqrt(b)   (composed by products)
// FOLD (half-split pairs, b = D): the butterfly between the two halves of the
// head is folded into the rotation, which then needs (U, V) = (C + S, C - S):
//   y_k + y_{k+D/2} = a U + b V,   y_k - y_{k+D/2} = a V - b U
// for the pair (a, b) = (x_k, x_{k+D/2}).  Lane j < P writes entry j of the
// wave's two LDS tables: fp64 (K rows) and the same values rounded once to
// fp32 (Q rows).
// ---------------------------------------------------------------------------
// Shared-set tables hold one padding entry after every 8 pairs (entry of pair k
// at k + k / 8).  The lanes of a row each read a block of consecutive pairs, so
// without padding their entries sit 8 pairs apart and fall in the same LDS
// banks; with it they fall in different ones (fp32 and fp64 entries alike).
constexpr int kTabPad = 8;
template <int P>
constexpr int tab_entries() { return P + P / kTabPad; }
__device__ __forceinline__ int tab_index(int k) { return k + k / kTabPad; }

template <int D, bool FOLD>
__device__ __forceinline__ void token_tables(float2* tab32, double2* tab64, int lane, int p, float invf,
                                             double cphi, double sphi, double rs) {
    constexpr int P = D / 2;
    wave_lds_sync();  // the previous token's table reads are complete
    if (lane < P) {
        double sa, ca;
        sincos_f64_of_f32(rope_angle_f32(p, invf), sa, ca);
        const double C = (ca * cphi - sa * sphi) * rs, S = (sa * cphi + ca * sphi) * rs;
        const double e0 = FOLD ? C + S : C, e1 = FOLD ? C - S : S;
        const int e = tab_index(lane);
        tab64[e] = make_double2(e0, e1);
        tab32[e] = make_float2((float)e0, (float)e1);
    }
    wave_lds_sync();
}

// ---------------------------------------------------------------------------
// Per-head angle sets: one set of pair angles per key head (query heads use
// their key head's set).  Tables are pair-major, entry (k, set) at
// k * kSetStride + set: a lane's sets sit together, the rows of one pass
// (different sets, same pairs) read neighbouring entries, a pair's offset is a
// compile-time multiple of the lane's base, and the padding entry spreads the
// lanes' pairs over the LDS banks.  The block keeps
// cos / sin of every set's angles in LDS (phi); each token's composed fp64
// tables are built for every set (tab64).
// ---------------------------------------------------------------------------
// cos / sin of angles[set][k] (n_sets x P floats) into phi[k * kSetStride + set]
// (block-wide; ends with a block barrier).
template <int P>
__device__ __forceinline__ void load_angle_sets(double2* phi, const float* angles, int n_sets) {
    for (int e = (int)threadIdx.x; e < n_sets * P; e += (int)blockDim.x) {
        double sv = 0.0, cv = 1.0;
        if (angles != nullptr) sincos_f64_of_f32(angles[e], sv, cv);
        phi[(e % P) * kSetStride + e / P] = make_double2(cv, sv);
    }
    __syncthreads();
}

// tab32 (the same entries rounded to fp32) may be null.
template <int D, bool FOLD>
__device__ __forceinline__ void token_tables_sets(float2* tab32, double2* tab64, int lane, int p, float invf,
                                                  const double2* phi, int n_sets, double rs) {
    constexpr int P = D / 2;
    wave_lds_sync();  // the previous token's table reads are complete
    if (lane < P) {
        double sa, ca;
        sincos_f64_of_f32(rope_angle_f32(p, invf), sa, ca);
        for (int g = 0; g < n_sets; ++g) {
            const double2 cs = phi[lane * kSetStride + g];
            const double C = (ca * cs.x - sa * cs.y) * rs, S = (sa * cs.x + ca * cs.y) * rs;
            const double e0 = FOLD ? C + S : C, e1 = FOLD ? C - S : S;
            tab64[lane * kSetStride + g] = make_double2(e0, e1);
            if (tab32 != nullptr) tab32[lane * kSetStride + g] = make_float2((float)e0, (float)e1);
        }
    }
    wave_lds_sync();
}

// Pair index of each coefficient slot of a lane holding the data of row
// position s_src:
//   half-split: slot j = pair s_src*CE + j (chunks 0 / 1 hold its two channels)
//   interleaved: slot j = ch*CE/2 + i, pair (ch*D/2 + s_src*CE + 2i) / 2
template <int D, int LAYOUT, int CE>
__device__ __forceinline__ void pair_index_of_lane(int s_src, int (&k)[CE]) {
#pragma unroll
    for (int j = 0; j < CE; ++j) {
        if constexpr (LAYOUT == 0) k[j] = s_src * CE + j;
        else k[j] = (j / (CE / 2)) * (D / 4) + s_src * (CE / 2) + (j % (CE / 2));
    }
}

// RoPE + R_phi (+ the folded half butterfly) of the lane's pairs, reading each
// pair's table entry from LDS just before it is used.
template <int LAYOUT, bool FOLD, int CE, typename V, typename T2>
__device__ __forceinline__ void rotate_lds(V (&x)[2][CE], const T2* tab, const int (&kidx)[CE]) {
#pragma unroll
    for (int j = 0; j < CE; ++j) {
        const T2 cs = tab[kidx[j]];
        const V e0 = cs.x, e1 = cs.y;
        V* pa;
        V* pb;
        if constexpr (LAYOUT == 0) {
            pa = &x[0][j];
            pb = &x[1][j];
        } else {
            pa = &x[j / (CE / 2)][2 * (j % (CE / 2))];
            pb = pa + 1;
        }
        const V a = *pa, b = *pb;
        if constexpr (FOLD) {
            *pa = a * e0 + b * e1;  // a U + b V
            *pb = a * e1 - b * e0;  // a V - b U
        } else {
            *pa = a * e0 - b * e1;  // a C - b S
            *pb = b * e0 + a * e1;  // b C + a S
        }
    }
}

// ---------------------------------------------------------------------------
// Walsh-Hadamard butterflies (Sylvester order, unnormalised: the 1/sqrt(b) is
// in the table).
// ---------------------------------------------------------------------------

// (a, b) -> (a + b, a - b) on every in-register pair at channel distance H.
template <int CE, int H, typename V>
__device__ __forceinline__ void fwht_inreg_stage(V (&x)[2][CE]) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int i = 0; i < CE; ++i)
            if ((i & H) == 0) {
                const V a = x[ch][i], b = x[ch][i + H];
                x[ch][i] = a + b;
                x[ch][i + H] = a - b;
            }
}

// Lane stages.  Every lane computes own + sgn * partner (sgn = -1 where the
// position bit is set): the lane with the bit clear gets a + b, the other
// b - a.  That is the Sylvester butterfly applied to the two inputs swapped,
// so the rows are loaded with their chunk positions xor-ed by every crossed
// position bit (lane_perm_mask): the transform then comes out exactly in
// natural order.
//
// fp32: one v_fmac_f32_dpp per value (partner read through DPP, multiplied by
// sgn and added to own).  The compiler does not form this instruction, so it
// is written out; the s_nop before the block gives the DPP source read two
// wait states after any earlier VALU write, the s_nop after it covers a DPP
// read of the block's last result by the following code.
#define RRP_FMAC(DST, SRC, SGN, CTRL) \
    "v_fmac_f32_dpp " DST ", " SRC ", " SGN " " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
// 8 values, each read from the partner lane's copy of its own register.
#define RRP_FMAC_SELF_8(CTRL)                                                                         \
    asm volatile("s_nop 1\n" RRP_FMAC("%0", "%0", "%8", CTRL) RRP_FMAC("%1", "%1", "%8", CTRL)       \
                 RRP_FMAC("%2", "%2", "%8", CTRL) RRP_FMAC("%3", "%3", "%8", CTRL)                    \
                 RRP_FMAC("%4", "%4", "%8", CTRL) RRP_FMAC("%5", "%5", "%8", CTRL)                    \
                 RRP_FMAC("%6", "%6", "%8", CTRL) RRP_FMAC("%7", "%7", "%8", CTRL) "s_nop 1"          \
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),             \
                   "+v"(x[6]), "+v"(x[7])                                                             \
                 : "v"(sgn))
// 8 values whose partner copy was prepared in src[] (lane xor 4: half-row mirror first).
#define RRP_FMAC_SRC_8(CTRL)                                                                          \
    asm volatile("s_nop 1\n" RRP_FMAC("%0", "%8", "%16", CTRL) RRP_FMAC("%1", "%9", "%16", CTRL)     \
                 RRP_FMAC("%2", "%10", "%16", CTRL) RRP_FMAC("%3", "%11", "%16", CTRL)                \
                 RRP_FMAC("%4", "%12", "%16", CTRL) RRP_FMAC("%5", "%13", "%16", CTRL)                \
                 RRP_FMAC("%6", "%14", "%16", CTRL) RRP_FMAC("%7", "%15", "%16", CTRL) "s_nop 1"      \
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),             \
                   "+v"(x[6]), "+v"(x[7])                                                             \
                 : "v"(src[0]), "v"(src[1]), "v"(src[2]), "v"(src[3]), "v"(src[4]), "v"(src[5]),      \
                   "v"(src[6]), "v"(src[7]), "v"(sgn))
#define RRP_FMAC_SELF_4(CTRL)                                                                         \
    asm volatile("s_nop 1\n" RRP_FMAC("%0", "%0", "%4", CTRL) RRP_FMAC("%1", "%1", "%4", CTRL)       \
                 RRP_FMAC("%2", "%2", "%4", CTRL) RRP_FMAC("%3", "%3", "%4", CTRL) "s_nop 1"          \
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])                                     \
                 : "v"(sgn))
#define RRP_FMAC_SRC_4(CTRL)                                                                          \
    asm volatile("s_nop 1\n" RRP_FMAC("%0", "%4", "%8", CTRL) RRP_FMAC("%1", "%5", "%8", CTRL)       \
                 RRP_FMAC("%2", "%6", "%8", CTRL) RRP_FMAC("%3", "%7", "%8", CTRL) "s_nop 1"          \
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])                                     \
                 : "v"(src[0]), "v"(src[1]), "v"(src[2]), "v"(src[3]), "v"(sgn))

// x[i] += sgn * x[i] of lane (lane ^ LM), for one chunk of CE values.
template <int CE, int LM>
__device__ __forceinline__ void fmac_lane_chunk(float (&x)[CE], float sgn) {
    if constexpr (LM == 4) {
        float src[CE];
#pragma unroll
        for (int i = 0; i < CE; ++i) src[i] = dpp_f<0x141>(x[i]);  // half-row mirror
        if constexpr (CE == 8) RRP_FMAC_SRC_8("quad_perm:[3,2,1,0]");
        else RRP_FMAC_SRC_4("quad_perm:[3,2,1,0]");
    } else if constexpr (CE == 8) {
        if constexpr (LM == 1) RRP_FMAC_SELF_8("quad_perm:[1,0,3,2]");
        else if constexpr (LM == 2) RRP_FMAC_SELF_8("quad_perm:[2,3,0,1]");
        else RRP_FMAC_SELF_8("row_ror:8");
    } else {
        static_assert(CE == 4, "chunk of 4 or 8 values");
        if constexpr (LM == 1) RRP_FMAC_SELF_4("quad_perm:[1,0,3,2]");
        else if constexpr (LM == 2) RRP_FMAC_SELF_4("quad_perm:[2,3,0,1]");
        else RRP_FMAC_SELF_4("row_ror:8");
    }
}

template <int L, int CE, int M>
__device__ __forceinline__ void lane_stage(float (&x)[2][CE], int s) {
    const float sgn = (s & M) ? -1.0f : 1.0f;
    fmac_lane_chunk<CE, LaneMap<L>::lane_mask(M)>(x[0], sgn);
    fmac_lane_chunk<CE, LaneMap<L>::lane_mask(M)>(x[1], sgn);
}

// fp64: two 32-bit DPP moves for the partner, then one fma.
template <int L, int CE, int M>
__device__ __forceinline__ void lane_stage(double (&x)[2][CE], int s) {
    const double sgn = (s & M) ? -1.0 : 1.0;
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int i = 0; i < CE; ++i) x[ch][i] = fma(sgn, s_xor<L, M>(x[ch][i]), x[ch][i]);
}

// Row positions crossed by the lane stages of a support-b transform: the
// chunk-position permutation applied to the loaded rows.
template <int D, int CE>
__device__ __forceinline__ int lane_perm_mask(int b) {
    constexpr int L = D / (2 * CE);
    int m = 0;
    for (int M = 1; M < L; M <<= 1)
        if (b > M * CE) m |= M;
    return m;
}

// Block Walsh-Hadamard transform of support b on a row loaded with the
// lane_perm_mask(b) permutation.  BT != 0: b is the compile-time constant BT;
// FOLDED: the half butterfly (b = D) was already applied by rotate_lds.
template <int D, int CE, int BT, bool FOLDED, typename V>
__device__ __forceinline__ void fwht_row(V (&x)[2][CE], int b_rt, int s) {
    constexpr int L = D / (2 * CE);
    const int b = BT ? BT : b_rt;
    if (b > 1) fwht_inreg_stage<CE, 1>(x);
    if (b > 2) fwht_inreg_stage<CE, 2>(x);
    if constexpr (CE > 4) { if (b > 4) fwht_inreg_stage<CE, 4>(x); }
    if constexpr (L > 1) { if (b > CE) lane_stage<L, CE, 1>(x, s); }
    if constexpr (L > 2) { if (b > 2 * CE) lane_stage<L, CE, 2>(x, s); }
    if constexpr (L > 4) { if (b > 4 * CE) lane_stage<L, CE, 4>(x, s); }
    if constexpr (L > 8) { if (b > 8 * CE) lane_stage<L, CE, 8>(x, s); }
    if constexpr (!FOLDED) {
        if (b > D / 2) {
#pragma unroll
            for (int i = 0; i < CE; ++i) {
                const V a = x[0][i], c = x[1][i];
                x[0][i] = a + c;
                x[1][i] = a - c;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Group reductions (output channel order).  Groups are `g` consecutive
// channels, g a power of two.  For g >= CE a group covers whole chunks: reduce
// the lane's chunk, then across the g / CE positions of the group (and across
// both halves when g == D).  For g < CE a group lies inside one lane.
// ---------------------------------------------------------------------------
template <int L, int M, bool IS_MAX, typename V>
__device__ __forceinline__ V red_lane(V v) {
    const V o = s_xor<L, M>(v);
    return IS_MAX ? fmax(v, o) : fmin(v, o);
}

template <int D, int CE, bool IS_MAX, typename V>
__device__ __forceinline__ void group_reduce_chunkwise(V (&m)[2], int g) {
    constexpr int L = D / (2 * CE);
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        if constexpr (L > 1) { if (g > CE) m[ch] = red_lane<L, 1, IS_MAX>(m[ch]); }
        if constexpr (L > 2) { if (g > 2 * CE) m[ch] = red_lane<L, 2, IS_MAX>(m[ch]); }
        if constexpr (L > 4) { if (g > 4 * CE) m[ch] = red_lane<L, 4, IS_MAX>(m[ch]); }
        if constexpr (L > 8) { if (g > 8 * CE) m[ch] = red_lane<L, 8, IS_MAX>(m[ch]); }
    }
    if (g > D / 2) {
        const V t = IS_MAX ? fmax(m[0], m[1]) : fmin(m[0], m[1]);
        m[0] = t;
        m[1] = t;
    }
}

// g < CE: after the stages every value holds the reduction over its aligned
// run of g values.
template <int CE, bool IS_MAX, typename V>
__device__ __forceinline__ void group_reduce_inreg(V (&v)[2][CE], int g) {
#pragma unroll
    for (int h = 1; h < CE; h <<= 1) {
        if (h < g) {
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                V t[CE];
#pragma unroll
                for (int i = 0; i < CE; ++i) t[i] = IS_MAX ? fmax(v[ch][i], v[ch][i ^ h]) : fmin(v[ch][i], v[ch][i ^ h]);
#pragma unroll
                for (int i = 0; i < CE; ++i) v[ch][i] = t[i];
            }
        }
    }
}

template <int D, int CE, typename V>
__device__ __forceinline__ void k_group_absmax_chunks(const V (&y)[2][CE], int g, V (&m)[2]) {
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
        V t = fabs(y[ch][0]);
#pragma unroll
        for (int i = 1; i < CE; ++i) t = fmax(t, fabs(y[ch][i]));
        m[ch] = t;
    }
    group_reduce_chunkwise<D, CE, true>(m, g);
}

// ---------------------------------------------------------------------------
// Group quantiser: s32 = fp32(max|y| / 7) (fp64 division, one rounding),
// stored scale = fp16(s32) nearest-even saturated, codes with 1 / stored scale.
// ---------------------------------------------------------------------------
struct GroupScale64 {
    float s32;
    unsigned short sh;
    double shv;
    double rcp;  // 1 / shv, or 0 when the stored scale is 0
};

__device__ __forceinline__ GroupScale64 group_scale64(double m) {
    GroupScale64 r;
    r.s32 = (float)(m / 7.0);
    r.sh = f16_sat_bits(r.s32);
    r.shv = (double)f16_bits_to_f32(r.sh);
    r.rcp = r.shv > 0.0 ? 1.0 / r.shv : 0.0;
    return r;
}

// Code of y under a group scale: round half to even, clamp to [-7, 7].
__device__ __forceinline__ int code_of(double y, double rcp) {
    const int q = (int)rint(y * rcp);  // v_cvt_i32_f64 saturates
    return min(max(q, -7), 7);
}
__device__ __forceinline__ int code_of(float y, double rcp) {
    const int q = (int)rintf(y * (float)rcp);  // v_cvt_i32_f32 saturates
    return min(max(q, -7), 7);
}

}  // namespace rrp
