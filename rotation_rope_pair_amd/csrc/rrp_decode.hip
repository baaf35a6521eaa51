// rrp_decode.hip -- decode attention logits straight from the KV4 cache.
//
// score[b][h][j] = sum_c q[b][h][c] * code(slot, kv, c) * s_h(slot, kv, c / g)
// for key j of sequence b at slot seq_start[b] + j, key head kv = h / (Hq / Hkv).
//
// One wavefront takes one (sequence, key head, chunk of kKeysPerWave keys).  The
// contraction over channels runs on the matrix cores: v_mfma_f32_16x16x32_f16
// with A = 16 keys x 32 channels of INT4 codes turned into f16 (exact small
// integers) and B = 32 channels x 16 columns holding the Hq / Hkv query heads
// that share the key head (f16, each head scaled by a power of two so that its
// largest value sits just below 2^15; fp32 queries as a hi + lo pair of f16
// terms).  Products of f16 values are exact in the fp32 accumulator.  Each MFMA
// contracts 32 channels, arranged so that the per-group partial sums can be
// kept apart (see KBM and SWAP in the kernel); the group scales (fp16 -> fp32)
// multiply those partial sums in fp32, so the codes never meet a rounded scale.
//
// Lane roles (16x16x32 layout): A row i = lane % 16 (key), k block kb = lane / 16
// (8 channels per MFMA); B column j = lane % 16 (query head); D holds keys
// 4 * (lane / 16) + r, r = 0..3, of column lane % 16.  Which channels an MFMA
// contracts is a free choice as long as A and B agree (see KBM and SWAP).
// Inside a lane's 8 channels the element order is (0, 4, 1, 5, 2, 6, 3, 7): that
// is the order in which the nibble-to-f16 conversion produces them, and B is laid
// out the same way.
#include <type_traits>

#include "rrp_device.hpp"
#include "rrp_kernels.hpp"

namespace rrp {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Keys per wave (one chunk).  With the chunk staged through LDS the chunk
// sets the waves per SIMD: 112 keys (7.5 KB per wave, five waves per SIMD)
// measured 0.557-0.558 ms on the 256-sequence decode batch, 128 keys (8.5 KB,
// four) 0.563-0.564 ms, 96 keys 0.561 ms, 64 keys 0.577 ms and 256 keys (17 KB,
// two) 0.664 ms.  Before staging, 128 and 256 measured the same and 512 slower.
constexpr int kKeysPerWave = 112;
// 16-key tiles loaded per step: one (66 VGPRs, 7 waves per SIMD) measured
// faster than two (104 VGPRs, 4 waves per SIMD).
constexpr int kTilesPerStep = 1;

// Channel offset (inside a lane's 8 channels) of half8 element e.
__device__ __forceinline__ constexpr int elem_channel(int e) { return (e >> 1) + 4 * (e & 1); }

// Eight two's-complement INT4 codes (nibble n = channel n) -> half8 in element order.
// Each code is made offset binary (x ^ 8, 0..15) and dropped into the mantissa of
// an f16 whose exponent makes the nibble's lowest bit worth 1: nibbles at bits
// 0-3 of a 16-bit half under the exponent of 1024 (value 1024 + n), nibbles at
// bits 4-7 under the exponent of 64 (value 64 + n).  One packed subtraction of
// 1032 or 72 then leaves the code exactly.  A shift by 8 brings channels 2, 3
// (and 6, 7 in the high half) to the same places, so a word costs one shift,
// four bit operations and four packed subtractions.
// nibble ^ 8 under the mask, the magic exponent elsewhere: one three-input bit
// operation (the xor is folded in, since the magic and the mask do not overlap).
__device__ __forceinline__ unsigned nib_magic(unsigned w, unsigned mask, unsigned magic) {
    const unsigned k = magic | (0x88888888u & mask);
    return ((w ^ k) & mask) | (k & ~mask);
}

__device__ __forceinline__ half8 codes_to_half8(unsigned w) {
    const unsigned y = w >> 8;
    const half2v off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const half2v off_hi = {(_Float16)72.0f, (_Float16)72.0f};
    const half2v h0 = __builtin_bit_cast(half2v, nib_magic(w, 0x000F000Fu, 0x64006400u)) - off_lo;  // channels 0, 4
    const half2v h1 = __builtin_bit_cast(half2v, nib_magic(w, 0x00F000F0u, 0x54005400u)) - off_hi;  // channels 1, 5
    const half2v h2 = __builtin_bit_cast(half2v, nib_magic(y, 0x000F000Fu, 0x64006400u)) - off_lo;  // channels 2, 6
    const half2v h3 = __builtin_bit_cast(half2v, nib_magic(y, 0x00F000F0u, 0x54005400u)) - off_hi;  // channels 3, 7
    half8 r;
    r[0] = h0[0]; r[1] = h0[1];
    r[2] = h1[0]; r[3] = h1[1];
    r[4] = h2[0]; r[5] = h2[1];
    r[6] = h3[0]; r[7] = h3[1];
    return r;
}

// Zero the elements of a half8 whose channel (8 * kb + elem_channel(e)) is not in
// sub-group u of size GS (GS < 32).
template <int GS>
__device__ __forceinline__ half8 mask_subgroup(half8 a, int kb, int u) {
    half8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = ((8 * kb + elem_channel(e)) / GS == u) ? a[e] : (_Float16)0.0f;
    return r;
}

template <typename E> struct QLoad;
template <> struct QLoad<bf16_tag> {
    // 8 consecutive channels of a bf16 row -> fp32
    __device__ static void load(const void* row, int c0, float (&x)[8]) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + c0);
        float t[8];
        unpack_chunk<bf16_tag, 8>(w, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = t[e];
    }
};
template <> struct QLoad<float> {
    __device__ static void load(const void* row, int c0, float (&x)[8]) {
        const float* p = static_cast<const float*>(row) + c0;
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(p);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(p + 4);
        x[0] = __uint_as_float(w0.x); x[1] = __uint_as_float(w0.y);
        x[2] = __uint_as_float(w0.z); x[3] = __uint_as_float(w0.w);
        x[4] = __uint_as_float(w1.x); x[5] = __uint_as_float(w1.y);
        x[6] = __uint_as_float(w1.z); x[7] = __uint_as_float(w1.w);
    }
};

// Largest of v over the four lanes l, l + 16, l + 32, l + 48.
__device__ __forceinline__ float max_over_kb(float v) {
    const int lane = (int)__lane_id();
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 16) << 2, __float_as_int(v))));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(v))));
    return v;
}

template <typename E, int D, int GS>
__global__ __launch_bounds__(256) void decode_scores_kernel(const DecodeArgs a) {
    constexpr int NM = D / 32;                                  // MFMAs per 16-key tile
    constexpr int NG = D / GS;                                  // groups per key row
    constexpr int SPLIT = ElemInfo<E>::bytes == 4 ? 2 : 1;      // f16 terms per query value
    constexpr int SROW = NG * 2;                                // scale bytes per key row
    // Channel order.  Groups of at least D/4 channels ("kb-major"): lane block kb
    // owns the contiguous quarter [kb D/4, (kb + 1) D/4) of every row, read with one
    // 16-byte (D = 128) or 8-byte (D = 64) load per key, and MFMA m takes its m-th
    // 8-channel piece; a group then covers whole lane blocks, and its partial sum is
    // separated by masking the query operand to those blocks.  Smaller groups
    // ("m-major"): MFMA m takes the 32 consecutive channels [32 m, 32 m + 32),
    // lane block kb the 8 at 32 m + 8 kb.
    constexpr bool KBM = GS >= D / 4;
    // Two groups per row (kb-major): lane blocks 0-1 hold group 0, 2-3 group 1.
    // Swapping the upper half-wave of word 2i with the lower half-wave of word
    // 2i + 1 (v_permlane32_swap) turns each pair of words into one operand of
    // each group, so every MFMA stays inside one group and the query operand
    // needs no per-group masked copies.
    constexpr bool SWAP = KBM && NG == 2;
    constexpr int LSPAN = D / 4;                // channels per lane block (kb-major)
    constexpr int KPG = KBM ? GS / LSPAN : 1;   // lane blocks per group (kb-major)

    // STAGE (d = 128, two groups per row: 4-byte scale rows): a wave's whole
    // chunk of codes and scales goes straight to LDS with direct loads at its
    // start, so all of it is in flight at once without holding VGPRs.
    constexpr bool STAGE = KBM && NM == 4 && SROW == 4 && kTilesPerStep == 1;
    constexpr int NT = kKeysPerWave / 16;         // tiles per chunk
    constexpr int NSL = (kKeysPerWave + 63) / 64;  // scale loads per chunk (64 keys each)
    static_assert(kKeysPerWave % 16 == 0, "whole tiles per chunk");
    __shared__ u32x4 st_codes[STAGE ? 4 : 1][STAGE ? NT : 1][64];
    __shared__ __attribute__((aligned(16))) unsigned st_scales[STAGE ? 4 : 1][STAGE ? 64 * NSL : 1];

    const int lane = (int)__lane_id();
    // wave-uniform (scalar) indices, so row bases stay in scalar registers
    const int hk = a.hk;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    int kvh, chunk;
    int64_t b;
    if (a.grid3d) {
        // grid (hk / 4, chunks, sequences): the indices need no division
        kvh = (int)blockIdx.x * 4 + wave;
        chunk = (int)blockIdx.y;
        b = a.seq_base + blockIdx.z;
    } else {
        const int64_t wid = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
        kvh = (int)(wid % hk);
        const int64_t rest = wid / hk;
        chunk = (int)(rest % a.n_chunks);
        b = a.seq_base + rest / a.n_chunks;
    }
    if (b >= a.n_seqs) return;
    int len = a.seq_len[b];
    len = len < a.max_len ? len : a.max_len;
    const int k_begin = chunk * kKeysPerWave;
    if (k_begin >= len) return;                                 // uniform per wave
    const int k_end = min(len, k_begin + kKeysPerWave);
    const int64_t start = a.seq_start[b];

    const int col = lane & 15;  // A row (key in tile) / B and D column (query head)
    const int kb = lane >> 4;   // A / B channel block; D key quad
    const int G = a.group_heads;
    const bool head_ok = col < G;
    const int h = kvh * G + col;

    const unsigned char* codes = a.k_codes;
    const unsigned char* scales = reinterpret_cast<const unsigned char*>(a.k_scales);
    const size_t code_row = (size_t)D / 2, scale_row = SROW;
    const size_t slot_stride_c = (size_t)hk * code_row, slot_stride_s = (size_t)hk * scale_row;
    const unsigned lane_c = (unsigned)((KBM ? LSPAN / 2 : 4) * kb);  // this lane's bytes in a code row
    // Every key of this wave's chunk sits inside the cache (the usual case):
    // keys are then only clamped to the chunk, and addressed by 32-bit offsets
    // from the chunk's first row.
    const bool chunk_in_cache = start + k_begin >= 0 && start + k_end <= a.n_slots;

    auto body = [&](auto in_cache_tag) {
        constexpr bool FAST = decltype(in_cache_tag)::value;
        // Row address of `key` inside the codes or the scales.  Loads are issued
        // unconditionally from a valid address and their values are never
        // masked: a key past the sequence (clamped to its last key) or outside
        // the cache (read at slot 0) only feeds its own row of the MFMA result,
        // which is not stored (past the end) or stored as NaN (outside the
        // cache).  So no branch or wait separates a load from its use.
        const unsigned char* cbase = codes + (size_t)kvh * code_row;
        const unsigned char* sbase = scales + (size_t)kvh * scale_row;
        if constexpr (FAST) {
            cbase += (start + k_begin) * (int64_t)slot_stride_c;
            sbase += (start + k_begin) * (int64_t)slot_stride_s;
        }
        auto row_of = [&](int key, bool scale_half) -> const unsigned char* {
            const unsigned char* base = scale_half ? sbase : cbase;
            const unsigned extra = scale_half ? 0u : lane_c;
            if constexpr (FAST) {
                const unsigned stride = (unsigned)(scale_half ? slot_stride_s : slot_stride_c);
                const unsigned kc = (unsigned)(min(key, k_end - 1) - k_begin);
                return base + (size_t)(kc * stride + extra);
            } else {
                const size_t stride = scale_half ? slot_stride_s : slot_stride_c;
                const int64_t slot = start + key;
                const bool ok = slot >= 0 && slot < a.n_slots;
                return base + (size_t)(ok ? slot : 0) * stride + extra;
            }
        };

        // A loads for the tile starting at key0: NM words (8 codes each) of key key0 + col.
        // The code loads are plain (cached) loads: a slot's key-head rows share
        // 128-byte lines (two heads at d = 128) that neighbouring waves of a block
        // read, and with a nontemporal hint each half of a line came from HBM on
        // its own (8-10 % slower on the decode batch).
        auto load_a = [&](int key0, unsigned (&w)[NM]) {
            const unsigned char* row = row_of(key0 + col, false);
            if constexpr (KBM && NM == 4) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(row);
                w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
            } else if constexpr (KBM) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(row);
                w[0] = v.x; w[1] = v.y;
            } else {
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    w[m] = *reinterpret_cast<const unsigned*>(row + 16 * m);
            }
        };
        // Scales of groups [g0, g0 + NS) of the lane's four D keys key0 + 4 kb + r, as fp32.
        auto load_s = [&](int key0, int g0, auto& sv) {
            constexpr int NS = sizeof(sv[0]) / sizeof(float);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const unsigned char* row = row_of(key0 + 4 * kb + r, true) + 2 * g0;
                if constexpr (NS == 1) {
                    const unsigned short v = *reinterpret_cast<const unsigned short*>(row);
                    sv[r][0] = f16_bits_to_f32(v);
                } else if constexpr (NS == 2) {
                    const unsigned v = *reinterpret_cast<const unsigned*>(row);
                    sv[r][0] = f16_bits_to_f32(v & 0xFFFFu);
                    sv[r][1] = f16_bits_to_f32(v >> 16);
                } else {
#pragma unroll
                    for (int q4 = 0; q4 < NS / 4; ++q4) {
                        const u32x2 v = *reinterpret_cast<const u32x2*>(row + 8 * q4);
                        sv[r][4 * q4 + 0] = f16_bits_to_f32(v.x & 0xFFFFu);
                        sv[r][4 * q4 + 1] = f16_bits_to_f32(v.x >> 16);
                        sv[r][4 * q4 + 2] = f16_bits_to_f32(v.y & 0xFFFFu);
                        sv[r][4 * q4 + 3] = f16_bits_to_f32(v.y >> 16);
                    }
                }
            }
        };

        // Groups of at least 32 channels: the key's whole scale row (<= 8 bytes) is
        // loaded with its codes, kept as raw fp16 words until used.  Smaller groups:
        // each MFMA's scales are read when it is used.
        constexpr int NSW = KBM ? (SROW + 3) / 4 : 1;
        auto load_sw = [&](int key0, unsigned (&sw)[4][NSW]) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const unsigned char* row = row_of(key0 + 4 * kb + r, true);
                if constexpr (SROW == 2) {
                    sw[r][0] = *reinterpret_cast<const unsigned short*>(row);
                } else if constexpr (SROW == 4) {
                    sw[r][0] = *reinterpret_cast<const unsigned*>(row);
                } else if constexpr (NSW >= 2) {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(row);
                    sw[r][0] = v.x;
                    sw[r][1] = v.y;
                }
            }
        };

        // Steps of kTilesPerStep tiles; the next step's codes and scales are in
        // flight while the current step is computed.
        constexpr int TP = kTilesPerStep;
        unsigned wc[TP][NM], wn[TP][NM];
        unsigned sc[TP][4][NSW], sn[TP][4][NSW];
        auto load_step = [&](int s0, unsigned (&w)[TP][NM], unsigned (&sw)[TP][4][NSW]) {
#pragma unroll
            for (int tt = 0; tt < TP; ++tt) {
                load_a(s0 + 16 * tt, w[tt]);
                if constexpr (KBM) load_sw(s0 + 16 * tt, sw[tt]);
            }
        };
        // Steps whose keys all lie in the chunk (FAST, groups of at least d/4):
        // every lane's row offsets from the step's first row are the same at each
        // step, so they are computed once and only the wave-uniform base moves.
        constexpr bool CONST_OFF = FAST && KBM;
        unsigned off_a[TP], off_s[TP][4];
#pragma unroll
        for (int tt = 0; tt < TP; ++tt) {
            off_a[tt] = (unsigned)((16 * tt + col) * (int)slot_stride_c) + lane_c;
#pragma unroll
            for (int r = 0; r < 4; ++r) off_s[tt][r] = (unsigned)((16 * tt + 4 * kb + r) * (int)slot_stride_s);
        }
        auto load_step_full = [&](int s0, unsigned (&w)[TP][NM], unsigned (&sw)[TP][4][NSW]) {
            const unsigned char* cb = cbase + (size_t)(unsigned)(s0 - k_begin) * slot_stride_c;
            const unsigned char* sb = sbase + (size_t)(unsigned)(s0 - k_begin) * slot_stride_s;
#pragma unroll
            for (int tt = 0; tt < TP; ++tt) {
                if constexpr (NM == 4) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(cb + off_a[tt]);
                    w[tt][0] = v.x; w[tt][1] = v.y; w[tt][2] = v.z; w[tt][3] = v.w;
                } else {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(cb + off_a[tt]);
                    w[tt][0] = v.x; w[tt][1] = v.y;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const unsigned char* row = sb + off_s[tt][r];
                    if constexpr (SROW == 2) {
                        sw[tt][r][0] = *reinterpret_cast<const unsigned short*>(row);
                    } else if constexpr (SROW == 4) {
                        sw[tt][r][0] = *reinterpret_cast<const unsigned*>(row);
                    } else if constexpr (NSW >= 2) {
                        const u32x2 v = *reinterpret_cast<const u32x2*>(row);
                        sw[tt][r][0] = v.x;
                        sw[tt][r][1] = v.y;
                    }
                }
            }
        };
        auto load_any = [&](int s0, unsigned (&w)[TP][NM], unsigned (&sw)[TP][4][NSW]) {
            if constexpr (CONST_OFF) {
                if (s0 + 16 * TP <= k_end) {
                    load_step_full(s0, w, sw);
                    return;
                }
            }
            load_step(s0, w, sw);
        };
        constexpr bool DMA = STAGE && FAST;
        if constexpr (DMA) {
            // Codes: tile tt's load puts lane (col, kb)'s 16 bytes (key k_begin +
            // 16 tt + col, bytes 16 kb of its row) at st_codes[wave][tt][lane].
            // Scales: lane i of load j puts key k_begin + 64 j + i's scale row at
            // st_scales[wave][64 j + i].  Keys past the chunk's end read its last key.
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                if (k_begin + 16 * tt < k_end) {
                    const unsigned kc = (unsigned)(min(k_begin + 16 * tt + col, k_end - 1) - k_begin);
                    __builtin_amdgcn_global_load_lds(
                        static_cast<const void*>(cbase + (size_t)(kc * (unsigned)slot_stride_c + lane_c)),
                        (__attribute__((address_space(3))) void*)st_codes[wave][tt], 16, 0, 0);
                }
#pragma unroll
            for (int j = 0; j < NSL; ++j)
                if (k_begin + 64 * j < k_end) {
                    const unsigned kc = (unsigned)(min(k_begin + 64 * j + lane, k_end - 1) - k_begin);
                    __builtin_amdgcn_global_load_lds(
                        static_cast<const void*>(sbase + (size_t)(kc * (unsigned)slot_stride_s)),
                        (__attribute__((address_space(3))) void*)&st_scales[wave][64 * j], 4, 0, 0);
                }
            asm volatile("" ::: "memory");  // issued before the query loads
        } else {
            load_any(k_begin, wc, sc);  // the first codes are in flight while the queries are prepared
        }

        // ---- B operand: this lane's query channels (kb-major: LSPAN kb + 8 m + elem_channel(e);
        //      m-major: 32 m + 8 kb + elem_channel(e)) ----
        // Every lane loads, so the loads need no branch: a lane past the group's
        // query heads (col >= G) reads the group's first head and zeroes what it
        // read.  (Loads inside a divergent branch each waited for their data
        // before the branch joined.)
        float qv[NM][8];
        float qmax = 0.0f;
        const void* qrow = static_cast<const unsigned char*>(a.q) +
                           ((size_t)b * a.hq + (head_ok ? h : kvh * G)) * D * ElemInfo<E>::bytes;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            float x[8];
            int c0;
            if constexpr (SWAP) {
                // operand m = 2i (group 0) / 2i + 1 (group 1) after the half-wave swap
                const int i = m >> 1;
                if ((m & 1) == 0) c0 = kb < 2 ? LSPAN * kb + 16 * i : LSPAN * (kb - 2) + 16 * i + 8;
                else c0 = kb < 2 ? LSPAN * (kb + 2) + 16 * i : LSPAN * kb + 16 * i + 8;
            } else {
                c0 = KBM ? LSPAN * kb + 8 * m : 32 * m + 8 * kb;
            }
            QLoad<E>::load(qrow, c0, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qv[m][e] = head_ok ? x[elem_channel(e)] : 0.0f;
                qmax = fmaxf(qmax, fabsf(qv[m][e]));
            }
        }
        qmax = max_over_kb(qmax);
        // power of two that brings the head's largest magnitude into [2^14, 2^15)
        const int qexp = (qmax > 0.0f && qmax <= 3.4e38f) ? 14 - ilogbf(qmax) : 0;
        half8 bq[SPLIT][NM];
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = ldexpf(qv[m][e], qexp);
                const _Float16 hi = (_Float16)v;
                bq[0][m][e] = hi;
                if constexpr (SPLIT == 2) bq[SPLIT - 1][m][e] = (_Float16)(v - (float)hi);
            }
        float* out_row = a.scores + ((size_t)b * a.hq + h) * a.max_len;
        const float descale = ldexpf(1.0f, -qexp);
        // One 16-key tile: dequantise, contract on the matrix cores, scale, store.
        auto tile = [&](int key0, const unsigned (&w)[NM], const unsigned (&sw)[4][NSW]) {
            half8 am[NM];
            if constexpr (SWAP) {
                // words 2i, 2i + 1 -> one operand of group 0 and one of group 1
#pragma unroll
                for (int i = 0; i < NM / 2; ++i) {
                    const auto xy = __builtin_amdgcn_permlane32_swap(w[2 * i], w[2 * i + 1], false, false);
                    am[2 * i] = codes_to_half8(xy[0]);
                    am[2 * i + 1] = codes_to_half8(xy[1]);
                }
            } else {
#pragma unroll
                for (int m = 0; m < NM; ++m) am[m] = codes_to_half8(w[m]);
            }

            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (SWAP) {
#pragma unroll
                for (int gq = 0; gq < 2; ++gq) {
                    f32x4 dq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int m = gq; m < NM; m += 2)
#pragma unroll
                        for (int t = 0; t < SPLIT; ++t)
                            dq = __builtin_amdgcn_mfma_f32_16x16x32_f16(am[m], bq[t][m], dq, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float scl = f16_bits_to_f32((unsigned short)(sw[r][0] >> (16 * gq)));
                        acc[r] = fmaf(scl, dq[r], acc[r]);
                    }
                }
            } else if constexpr (KBM) {
#pragma unroll
                for (int gq = 0; gq < NG; ++gq) {
                    f32x4 dq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int t = 0; t < SPLIT; ++t) {
                            half8 bm;
                            if constexpr (NG == 1) bm = bq[t][m];
                            else bm = (kb / KPG == gq) ? bq[t][m] : half8{};
                            dq = __builtin_amdgcn_mfma_f32_16x16x32_f16(am[m], bm, dq, 0, 0, 0);
                        }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float scl = f16_bits_to_f32((unsigned short)(sw[r][gq >> 1] >> (16 * (gq & 1))));
                        acc[r] = fmaf(scl, dq[r], acc[r]);
                    }
                }
            } else {
                constexpr int SUB = 32 / GS;  // groups inside one MFMA
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    if constexpr (SUB <= 2) {
                        float sm[4][SUB];
                        load_s(key0, m * SUB, sm);
#pragma unroll
                        for (int u = 0; u < SUB; ++u) {
                            const half8 amu = mask_subgroup<GS>(am[m], kb, u);
                            f32x4 dq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                            for (int t = 0; t < SPLIT; ++t)
                                dq = __builtin_amdgcn_mfma_f32_16x16x32_f16(amu, bq[t][m], dq, 0, 0, 0);
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[r] = fmaf(sm[r][u], dq[r], acc[r]);
                        }
                    } else {
                        // many small groups: one sub-group (and its scale) at a time
#pragma unroll 1
                        for (int u = 0; u < SUB; ++u) {
                            float su[4][1];
                            load_s(key0, m * SUB + u, su);
                            const half8 amu = mask_subgroup<GS>(am[m], kb, u);
                            f32x4 dq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                            for (int t = 0; t < SPLIT; ++t)
                                dq = __builtin_amdgcn_mfma_f32_16x16x32_f16(amu, bq[t][m], dq, 0, 0, 0);
#pragma unroll
                            for (int r = 0; r < 4; ++r) acc[r] = fmaf(su[r][0], dq[r], acc[r]);
                        }
                    }
                }
            }

            if (head_ok) {
                const int kq = key0 + 4 * kb;  // this lane's four consecutive keys
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (FAST) {
                        o[r] = acc[r] * descale;
                    } else {
                        const int64_t slot = start + kq + r;
                        o[r] = (slot >= 0 && slot < a.n_slots) ? acc[r] * descale : __builtin_nanf("");
                    }
                }
                // plain stores: the logits are read again by the softmax that follows
                if (a.vec_store && kq + 3 < k_end) {
                    *reinterpret_cast<f32x4*>(out_row + kq) = o;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (kq + r < k_end) out_row[kq + r] = o[r];
                }
            }
        };

        if constexpr (DMA) {
            // The staged chunk has landed (the query loads, issued after it, were
            // waited for by the query preparation already).
            wait_vm_all();
            for (int tt = 0; tt < NT && k_begin + 16 * tt < k_end; ++tt) {
                const u32x4 v = st_codes[wave][tt][lane];
                const u32x4 sv = *reinterpret_cast<const u32x4*>(&st_scales[wave][16 * tt + 4 * kb]);
                unsigned w4[NM], s4[4][NSW];
#pragma unroll
                for (int m = 0; m < NM; ++m) w4[m] = v[m];
#pragma unroll
                for (int r = 0; r < 4; ++r) s4[r][0] = sv[r];
                tile(k_begin + 16 * tt, w4, s4);
            }
            return;
        }
        // Retire the first step's loads here (the queries were prepared while they
        // were in flight): inside the loop the current step is then always a copy
        // made after its wait, and its first use needs no wait, which would
        // otherwise also take part of the next step's prefetch on every step.
#pragma unroll
        for (int tt = 0; tt < TP; ++tt) {
#pragma unroll
            for (int m = 0; m < NM; ++m) asm volatile("" ::"v"(wc[tt][m]));
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int x = 0; x < NSW; ++x) asm volatile("" ::"v"(sc[tt][r][x]));
        }
        for (int s0 = k_begin; s0 < k_end; s0 += 16 * TP) {
            if (s0 + 16 * TP < k_end) load_any(s0 + 16 * TP, wn, sn);
#pragma unroll
            for (int tt = 0; tt < TP; ++tt)
                if (s0 + 16 * tt < k_end) tile(s0 + 16 * tt, wc[tt], sc[tt]);
#pragma unroll
            for (int tt = 0; tt < TP; ++tt) {
#pragma unroll
                for (int m = 0; m < NM; ++m) wc[tt][m] = wn[tt][m];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int x = 0; x < NSW; ++x) sc[tt][r][x] = sn[tt][r][x];
            }
        }
    };
    if (chunk_in_cache) body(std::true_type{});
    else body(std::false_type{});
}

// A dispatch covers at most 2^32 - 1 work-items per grid dimension, and the y
// and z block counts at most 65535 each.
constexpr int64_t kMaxGridThreads = 0xFFFFFFFFll;
constexpr int64_t kMaxGridYZ = 65535;

// Sequences one launch may take; 0 if a single sequence does not fit.
int64_t decode_seqs_per_launch(int64_t n_chunks, int hk) {
    const bool grid3d = hk % 4 == 0 && n_chunks <= kMaxGridYZ;
    if (grid3d) return kMaxGridYZ;
    const int64_t waves_per_seq = n_chunks * hk;
    const int64_t max_waves = kMaxGridThreads / 256 * 4;
    const int64_t s = max_waves / waves_per_seq;
    return s < kMaxGridYZ ? s : kMaxGridYZ;
}

template <typename E, int D, int GS>
hipError_t launch_range(DecodeArgs a, hipStream_t st) {
    // Four key heads of one (sequence, chunk) per block.  With hk a multiple of 4
    // (and the chunk count within the y grid limit) the block's place comes
    // straight from a 3-D grid, else from a 1-D one.  Batches with more sequences
    // than one grid holds go out as consecutive launches over sequence ranges.
    a.grid3d = (a.hk % 4 == 0 && a.n_chunks <= kMaxGridYZ) ? 1 : 0;
    const int64_t per_launch = decode_seqs_per_launch(a.n_chunks, a.hk);
    if (per_launch < 1) return hipErrorInvalidConfiguration;
    const int64_t n_seqs = a.n_seqs;
    for (int64_t s0 = 0; s0 < n_seqs; s0 += per_launch) {
        const int64_t ns = n_seqs - s0 < per_launch ? n_seqs - s0 : per_launch;
        a.seq_base = s0;
        a.n_seqs = s0 + ns;  // the kernel's bound: the 1-D grid's last block may overhang the range
        dim3 grid;
        if (a.grid3d) {
            grid = dim3((unsigned)(a.hk / 4), (unsigned)a.n_chunks, (unsigned)ns);
        } else {
            const int64_t waves = ns * a.n_chunks * a.hk;
            grid = dim3((unsigned)((waves + 3) / 4));
        }
        hipLaunchKernelGGL((decode_scores_kernel<E, D, GS>), grid, dim3(256), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename E, int D>
hipError_t launch_d(const DecodeArgs& a, int group, hipStream_t st) {
#define RRP_G(GS) \
    if (group == GS) return launch_range<E, D, GS>(a, st);
    RRP_G(2) RRP_G(4) RRP_G(8) RRP_G(16) RRP_G(32) RRP_G(64)
    if constexpr (D >= 128) { RRP_G(128) }
#undef RRP_G
    return hipErrorInvalidValue;
}

}  // namespace

int64_t decode_chunks(int max_len) { return ((int64_t)max_len + kKeysPerWave - 1) / kKeysPerWave; }
int64_t decode_launches(int64_t n_seqs, int64_t n_chunks, int hk) {
    const int64_t per_launch = decode_seqs_per_launch(n_chunks, hk);
    return per_launch < 1 ? 0 : (n_seqs + per_launch - 1) / per_launch;
}
int decode_chunk_keys() { return kKeysPerWave; }

hipError_t launch_decode_scores(const DecodeArgs& a, int dtype, int head_dim, int group, hipStream_t st) {
    if (dtype == 1) {
        if (head_dim == 64) return launch_d<bf16_tag, 64>(a, group, st);
        if (head_dim == 128) return launch_d<bf16_tag, 128>(a, group, st);
    } else {
        if (head_dim == 64) return launch_d<float, 64>(a, group, st);
        if (head_dim == 128) return launch_d<float, 128>(a, group, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace rrp
