// rrp_kernels.hpp -- kernel argument blocks and launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rrp_rotate.hpp"

namespace rrp {

constexpr int kMaxCalibBlocks = 4096;  // block partials of the calibration pass
constexpr int kMaxStatsBlocks = 8192;  // block partials of the diagnostic pass

struct CalibArgs {
    const void* q;
    const void* k;
    const int32_t* pos;
    double* partials;  // [P * 5][n_blocks]
    int64_t n_tokens;
    int32_t hq;
    int32_t hk;
    int32_t nbq;     // blocks per angle set accumulating the Q stream
    int32_t nbk;     // blocks per angle set accumulating the K stream
    int32_t n_sets;  // angle sets (1: all heads pooled; n_kv_heads: per key head)
    float inv_freq[kMaxPairs];
};

struct CalibFinalArgs {
    const double* partials;
    double* moments;  // [n_sets][P][2][6]
    float* angles_out;  // [n_sets][P]
    double n_rows_q;  // rows added to each set's Q stream by this call
    double n_rows_k;
    int32_t nbq;      // blocks per set (as in CalibArgs)
    int32_t nbk;
    int32_t n_pairs;  // P
    int32_t n_sets;
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
    int32_t angle_sets;  // 1: shared angle set; n_kv_heads: one per key head
    int32_t bin;         // single support: channels of a group held by one lane (set by the launcher)
    int32_t xmask;       // single support: lane position bits shared by a group (set by the launcher)
    double wgt;          // single support: 1 / lanes sharing a group (set by the launcher)
    double rsqrt_b;
    float inv_freq[kMaxPairs];
};

struct StatsFinalArgs {
    const double* partials;  // [n_sets * 5][n_blocks]
    double* stats_out;       // [n_sets][8]
    int32_t n_blocks;
    int32_t n_sets;          // supports reduced (1, or log2(head_dim) + 1 for the sweep)
    int32_t sweep;           // write the support 2^set into column 7
    double n_groups;
    double n_rows;
};

struct DecodeArgs {
    const void* q;             // [n_seqs][hq][head_dim] rotated queries
    const uint8_t* k_codes;    // [n_slots][hk][head_dim / 2]
    const uint16_t* k_scales;  // [n_slots][hk][head_dim / group] fp16 bits
    const int64_t* seq_start;  // [n_seqs] slot of key 0
    const int32_t* seq_len;    // [n_seqs] keys per sequence
    float* scores;             // [n_seqs][hq][max_len]
    int64_t n_seqs;            // sequences in the batch (in a launch: one past its last sequence)
    int64_t n_slots;
    int64_t n_chunks;          // key chunks per sequence (one wave each)
    int32_t hq;
    int32_t hk;
    int32_t group_heads;       // hq / hk query heads per key head
    int32_t max_len;
    int32_t vec_store;         // scores rows are 16-byte aligned: store 4 logits at once
    int32_t grid3d;            // grid (hk / 4, n_chunks, sequences) instead of one dimension (set by the launcher)
    int64_t seq_base;          // first sequence of this launch (the launcher splits long batches)
};


int calib_blocks(int64_t n_tokens, bool with_q, int hq, int hk, int head_dim, int n_sets, int* nbq, int* nbk);
hipError_t launch_calibrate(const CalibArgs& a, int dtype, int head_dim, int layout, hipStream_t st);
hipError_t launch_calibrate_final(const CalibFinalArgs& a, hipStream_t st);

int stats_blocks(int64_t n_tokens, bool sweep);
hipError_t launch_stats(const StatsArgs& a, int n_blocks, int dtype, int head_dim, int layout, bool sweep,
                        hipStream_t st);
hipError_t launch_stats_final(const StatsFinalArgs& a, hipStream_t st);

int64_t decode_chunks(int max_len);
int64_t decode_launches(int64_t n_seqs, int64_t n_chunks, int hk);  // 0: one sequence's waves overfill a grid
int decode_chunk_keys();  // keys per wave
hipError_t launch_decode_scores(const DecodeArgs& a, int dtype, int head_dim, int group, hipStream_t st);

}  // namespace rrp
