// rrp_rotate.hpp -- argument block and launcher of the rotate + quantise kernel
// (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rrp {

constexpr int kMaxPairs = 64;     // head_dim <= 128
constexpr int kMaxAngleSets = 8;  // per-head angle sets held in LDS per token
// Entry stride of a pair in the per-set LDS tables (pair-major, one padding
// entry so that neighbouring lanes' pairs fall in different LDS banks).
constexpr int kSetStride = kMaxAngleSets + 1;

// RoPE frequencies travel in the kernel argument block: every lane reads its
// own pair's entry, so no device table has to be allocated or kept.
struct RotateArgs {
    const void* q;
    const void* k;
    const int32_t* pos;
    const float* angles;
    void* q_out;
    uint8_t* k_codes;
    uint16_t* k_scales;
    const int64_t* slot_mapping;
    float* q_dbg;
    float* k_dbg;
    float* s_dbg;
    const void* v;       // NULL: no V rows
    uint8_t* v_codes;
    uint16_t* v_scales;
    float* v_dbg;
    float* vs_dbg;
    int64_t n_tokens;
    int64_t n_slots;
    int32_t hq;       // Q heads in the tensor layout
    int32_t hq_rows;  // Q rows processed per token (0 when Q is skipped)
    int32_t hk;
    int32_t support_b;
    int32_t group;
    int32_t angle_sets;  // 1: one set shared by all heads; n_kv_heads: one per key head
    int32_t split;       // waves per token (set by the launcher; > 1 for small batches)
    float q_set_scale;   // angle sets / Hq: query head h uses set floor((h + 1/2) * q_set_scale)
    double rsqrt_b;
    double rsqrt_v;  // 1 / sqrt(head_dim)
    float inv_freq[kMaxPairs];
};

// dtype: 0 fp32, 1 bf16; layout: 0 half-split, 1 interleaved.
hipError_t launch_rotate_quantize(const RotateArgs& a, int dtype, int head_dim, int layout, hipStream_t st);
// The small-batch family (n_tokens x row passes per token <= 4096), called by
// launch_rotate_quantize.
hipError_t launch_rotate_quantize_split(const RotateArgs& a, int dtype, int head_dim, int layout, hipStream_t st);

}  // namespace rrp
