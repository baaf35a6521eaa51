// rrp_kernels.hpp -- kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rrp {

constexpr int kMaxPairs = 64;        // head_dim <= 128
constexpr int kMaxCalibBlocks = 4096;  // block partials of the calibration pass
constexpr int kMaxStatsBlocks = 4096;  // block partials of the diagnostic pass

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
    double rsqrt_b;
    double rsqrt_v;  // 1 / sqrt(head_dim)
    float inv_freq[kMaxPairs];
};

struct CalibArgs {
    const void* q;
    const void* k;
    const int32_t* pos;
    double* partials;  // [P * 5][n_blocks]
    int64_t n_tokens;
    int32_t hq;
    int32_t hk;
    int32_t nbq;  // blocks accumulating the Q stream (first nbq blocks)
    int32_t nbk;  // blocks accumulating the K stream
    float inv_freq[kMaxPairs];
};

struct CalibFinalArgs {
    const double* partials;
    double* moments;  // [P][2][6]
    float* angles_out;
    double n_rows_q;  // rows added to the Q stream by this call
    double n_rows_k;
    int32_t nbq;
    int32_t nbk;
    int32_t n_pairs;
    int32_t estimator;
};

struct StatsArgs {
    const void* k;
    const int32_t* pos;
    const float* angles;
    double* partials;  // [5][n_blocks]
    int64_t n_tokens;
    int32_t hk;
    int32_t support_b;
    int32_t group;
    double rsqrt_b;
    float inv_freq[kMaxPairs];
};

struct StatsFinalArgs {
    const double* partials;
    double* stats_out;
    int32_t n_blocks;
    double n_groups;
    double n_rows;
};

// dtype: 0 fp32, 1 bf16; layout: 0 half-split, 1 interleaved.
hipError_t launch_rotate_quantize(const RotateArgs& a, int dtype, int head_dim, int layout, hipStream_t st);

int calib_blocks(int64_t n_tokens, bool with_q, int hq, int hk, int* nbq, int* nbk);
hipError_t launch_calibrate(const CalibArgs& a, int dtype, int head_dim, int layout, hipStream_t st);
hipError_t launch_calibrate_final(const CalibFinalArgs& a, hipStream_t st);

int stats_blocks(int64_t n_tokens);
hipError_t launch_stats(const StatsArgs& a, int n_blocks, int dtype, int head_dim, int layout, hipStream_t st);
hipError_t launch_stats_final(const StatsFinalArgs& a, hipStream_t st);

}  // namespace rrp
