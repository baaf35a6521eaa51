// rrp_abi.hip -- the C-ABI entry points (include/rrp.h): host-side validation,
// RoPE frequency table, workspace sizing and kernel dispatch.
//
// Every check runs before anything is enqueued, so an error return leaves the
// stream untouched.  The RoPE frequencies are evaluated here on the host in
// fp64 (libm pow) and rounded once to fp32; they travel to the kernels inside
// the kernel argument block.  The library allocates no memory: the block
// partial sums of calibration and diagnostics live in a workspace the caller
// passes in (its size comes from the *_workspace_size queries).
#include <math.h>
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "rrp.h"
#include "rrp_kernels.hpp"

#define RRP_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int check_shape(const rrp_shape* s, int32_t dtype) {
    if (s == nullptr) return RRP_ERR_INVALID_ARG;
    if (dtype != RRP_F32 && dtype != RRP_BF16) return RRP_ERR_INVALID_ARG;
    if (s->n_q_heads < 0 || s->n_kv_heads < 1) return RRP_ERR_INVALID_ARG;
    if (s->rope_layout != RRP_ROPE_HALF_SPLIT && s->rope_layout != RRP_ROPE_INTERLEAVED) return RRP_ERR_INVALID_ARG;
    if (!(s->rope_theta > 0.0) || !isfinite(s->rope_theta)) return RRP_ERR_INVALID_ARG;
    if (s->head_dim < 2 || (s->head_dim & 1)) return RRP_ERR_INVALID_ARG;
    if (s->head_dim != 64 && s->head_dim != 128) return RRP_ERR_UNSUPPORTED;
    if (s->angle_heads < 0 || (s->angle_heads > 1 && s->angle_heads != s->n_kv_heads)) return RRP_ERR_INVALID_ARG;
    if (s->angle_heads > 1 && s->n_q_heads % s->n_kv_heads != 0) return RRP_ERR_INVALID_ARG;
    if (s->angle_heads > rrp::kMaxAngleSets) return RRP_ERR_UNSUPPORTED;  // per-set tables held in LDS
    return RRP_OK;
}

// Angle sets of the layer: 1 (shared by all heads) or n_kv_heads (one per key head).
int angle_sets(const rrp_shape* s) { return s->angle_heads > 1 ? s->angle_heads : 1; }

int check_b_g(const rrp_shape* s, int32_t support_b, int32_t group) {
    if (!is_pow2(support_b) || support_b > s->head_dim) return RRP_ERR_INVALID_ARG;
    if (!is_pow2(group) || group < 2 || group > s->head_dim) return RRP_ERR_INVALID_ARG;
    return RRP_OK;
}

void fill_inv_freq(const rrp_shape* s, float* out) {
    for (int k = 0; k < rrp::kMaxPairs; ++k)
        out[k] = k < s->head_dim / 2 ? (float)pow(s->rope_theta, -2.0 * (double)k / (double)s->head_dim) : 0.0f;
}

// Workspace bytes of one calibration call: the block partials [P * 5][blocks]
// (0 when there are no tokens).  with_q: the Q stream is accumulated.
size_t calib_workspace_bytes(const rrp_shape* s, int64_t n_tokens, bool with_q) {
    if (n_tokens <= 0) return 0;
    int nbq = 0, nbk = 0;
    const int nb = rrp::calib_blocks(n_tokens, with_q && s->n_q_heads > 0, s->n_q_heads, s->n_kv_heads,
                                     s->head_dim, angle_sets(s), &nbq, &nbk);
    return (size_t)nb * (size_t)(s->head_dim / 2) * 5 * sizeof(double);
}

// Supports reduced by the diagnostics: 1, or every b = 1, 2, ..., head_dim (sweep).
int stats_supports(const rrp_shape* s, bool sweep) {
    int n = 1;
    if (sweep)
        for (int b = 1; b < s->head_dim; b <<= 1) ++n;
    return n;
}

// Workspace bytes of one diagnostics call: the block partials [supports * 5][blocks].
size_t stats_workspace_bytes(const rrp_shape* s, int64_t n_tokens, bool sweep) {
    if (n_tokens <= 0) return 0;
    return (size_t)rrp::stats_blocks(n_tokens, sweep) * (size_t)stats_supports(s, sweep) * 5 * sizeof(double);
}

// A workspace of `have` bytes at `p` for a call needing `need` bytes.
int check_workspace(const void* p, size_t have, size_t need) {
    if (need == 0) return RRP_OK;
    if (p == nullptr || have < need) return RRP_ERR_INVALID_ARG;
    return aligned(p, 8) ? RRP_OK : RRP_ERR_MISALIGNED;
}

}  // namespace

RRP_EXPORT int rrp_version(void) { return kVersion; }

RRP_EXPORT const char* rrp_status_string(int status) {
    switch (status) {
        case RRP_OK: return "ok";
        case RRP_ERR_INVALID_ARG: return "invalid argument";
        case RRP_ERR_MISALIGNED: return "misaligned pointer";
        case RRP_ERR_UNSUPPORTED: return "unsupported configuration";
        case RRP_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

namespace {

// Shared body of the Q/K and Q/K/V entry points (v == nullptr: no V rows).
int rotate_quantize(const rrp_shape* shape, int32_t dtype, const void* q, const void* k, const void* v,
                    const int32_t* pos, int64_t n_tokens, const float* angles, int32_t support_b, int32_t group,
                    void* q_out, uint8_t* k_codes, uint16_t* k_scales, uint8_t* v_codes, uint16_t* v_scales,
                    const int64_t* slot_mapping, int64_t n_slots, float* q_rot_f32, float* k_rot_f32,
                    float* k_scale_f32, float* v_rot_f32, float* v_scale_f32, void* stream) {
    int st = check_shape(shape, dtype);
    if (st != RRP_OK) return st;
    if ((st = check_b_g(shape, support_b, group)) != RRP_OK) return st;
    if (n_tokens < 0 || n_slots < 0) return RRP_ERR_INVALID_ARG;
    if (n_tokens == 0) return RRP_OK;  // nothing is read or written; empty arrays may be NULL
    if (k == nullptr || pos == nullptr || k_codes == nullptr || k_scales == nullptr) return RRP_ERR_INVALID_ARG;
    if ((q_out != nullptr || q_rot_f32 != nullptr) && q == nullptr) return RRP_ERR_INVALID_ARG;
    if (slot_mapping == nullptr && n_slots < n_tokens) return RRP_ERR_INVALID_ARG;
    const uintptr_t code_align = dtype == RRP_F32 ? 2 : 4;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_out, 16) || !aligned(q_rot_f32, 16) ||
        !aligned(k_rot_f32, 16) || !aligned(k_scale_f32, 4) || !aligned(pos, 4) || !aligned(angles, 4) ||
        !aligned(k_codes, code_align) || !aligned(k_scales, 2) || !aligned(slot_mapping, 8) ||
        !aligned(v, 16) || !aligned(v_codes, code_align) || !aligned(v_scales, 2) || !aligned(v_rot_f32, 16) ||
        !aligned(v_scale_f32, 4))
        return RRP_ERR_MISALIGNED;

    rrp::RotateArgs a{};
    a.q = q;
    a.k = k;
    a.pos = pos;
    a.angles = angles;
    a.q_out = q_out;
    a.k_codes = k_codes;
    a.k_scales = k_scales;
    a.slot_mapping = slot_mapping;
    a.q_dbg = q_rot_f32;
    a.k_dbg = k_rot_f32;
    a.s_dbg = k_scale_f32;
    a.v = v;
    a.v_codes = v_codes;
    a.v_scales = v_scales;
    a.v_dbg = v_rot_f32;
    a.vs_dbg = v_scale_f32;
    a.n_tokens = n_tokens;
    a.n_slots = n_slots;
    a.hq = shape->n_q_heads;
    a.hq_rows = (q != nullptr && (q_out != nullptr || q_rot_f32 != nullptr)) ? shape->n_q_heads : 0;
    a.hk = shape->n_kv_heads;
    a.support_b = support_b;
    a.group = group;
    a.angle_sets = angles != nullptr ? angle_sets(shape) : 1;
    a.q_set_scale = shape->n_q_heads > 0 ? (float)a.angle_sets / (float)shape->n_q_heads : 0.0f;
    a.rsqrt_b = 1.0 / sqrt((double)support_b);
    a.rsqrt_v = 1.0 / sqrt((double)shape->head_dim);
    fill_inv_freq(shape, a.inv_freq);
    hipError_t e = rrp::launch_rotate_quantize(a, dtype, shape->head_dim, shape->rope_layout, (hipStream_t)stream);
    return e == hipSuccess ? RRP_OK : RRP_ERR_HIP;
}

}  // namespace

RRP_EXPORT int rrp_rotate_quantize_qk(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                                      const int32_t* pos, int64_t n_tokens, const float* angles,
                                      int32_t support_b, int32_t group, void* q_out, uint8_t* k_codes,
                                      uint16_t* k_scales, const int64_t* slot_mapping, int64_t n_slots,
                                      float* q_rot_f32, float* k_rot_f32, float* k_scale_f32, void* stream) {
    return rotate_quantize(shape, dtype, q, k, nullptr, pos, n_tokens, angles, support_b, group, q_out, k_codes,
                           k_scales, nullptr, nullptr, slot_mapping, n_slots, q_rot_f32, k_rot_f32, k_scale_f32,
                           nullptr, nullptr, stream);
}

RRP_EXPORT int rrp_rotate_quantize_qkv(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                                       const void* v, const int32_t* pos, int64_t n_tokens, const float* angles,
                                       int32_t support_b, int32_t group, void* q_out, uint8_t* k_codes,
                                       uint16_t* k_scales, uint8_t* v_codes, uint16_t* v_scales,
                                       const int64_t* slot_mapping, int64_t n_slots, float* q_rot_f32,
                                       float* k_rot_f32, float* k_scale_f32, float* v_rot_f32, float* v_scale_f32,
                                       void* stream) {
    if (v == nullptr || v_codes == nullptr || v_scales == nullptr) return RRP_ERR_INVALID_ARG;
    return rotate_quantize(shape, dtype, q, k, v, pos, n_tokens, angles, support_b, group, q_out, k_codes,
                           k_scales, v_codes, v_scales, slot_mapping, n_slots, q_rot_f32, k_rot_f32, k_scale_f32,
                           v_rot_f32, v_scale_f32, stream);
}

RRP_EXPORT int rrp_calibrate_angles_workspace_size(const rrp_shape* shape, int64_t n_tokens, int32_t with_q,
                                                   size_t* bytes) {
    const int st = check_shape(shape, RRP_BF16);
    if (st != RRP_OK) return st;
    if (n_tokens < 0 || bytes == nullptr) return RRP_ERR_INVALID_ARG;
    *bytes = calib_workspace_bytes(shape, n_tokens, with_q != 0);
    return RRP_OK;
}

namespace {

// Body of rrp_calibrate_angles, with the block partials in `partials`
// (calib_workspace_bytes of them; checked by the caller).
int calibrate(const rrp_shape* shape, int32_t dtype, const void* q, const void* k, const int32_t* pos,
              int64_t n_tokens, int32_t estimator, double* moments, float* angles_out, double* partials,
              hipStream_t s) {
    const int P = shape->head_dim / 2;
    rrp::CalibFinalArgs f{};
    f.moments = moments;
    f.angles_out = angles_out;
    f.n_pairs = P;
    f.n_sets = angle_sets(shape);
    f.estimator = estimator;
    if (n_tokens > 0) {
        int nbq = 0, nbk = 0;
        const bool with_q = q != nullptr && shape->n_q_heads > 0;
        rrp::calib_blocks(n_tokens, with_q, shape->n_q_heads, shape->n_kv_heads, shape->head_dim, f.n_sets, &nbq,
                          &nbk);
        rrp::CalibArgs a{};
        a.q = q;
        a.k = k;
        a.pos = pos;
        a.partials = partials;
        a.n_tokens = n_tokens;
        a.hq = shape->n_q_heads;
        a.hk = shape->n_kv_heads;
        a.nbq = nbq;
        a.nbk = nbk;
        a.n_sets = f.n_sets;
        fill_inv_freq(shape, a.inv_freq);
        if (rrp::launch_calibrate(a, dtype, shape->head_dim, shape->rope_layout, s) != hipSuccess) return RRP_ERR_HIP;
        f.partials = a.partials;
        f.nbq = nbq;
        f.nbk = nbk;
        f.n_rows_q = (double)n_tokens * (shape->n_q_heads / f.n_sets);  // rows per set
        f.n_rows_k = (double)n_tokens * (shape->n_kv_heads / f.n_sets);
    } else if (angles_out == nullptr) {
        return RRP_OK;
    }
    return rrp::launch_calibrate_final(f, s) == hipSuccess ? RRP_OK : RRP_ERR_HIP;
}

// Argument checks of rrp_calibrate_angles (everything but the workspace).
int check_calibrate(const rrp_shape* shape, int32_t dtype, const void* q, const void* k, const int32_t* pos,
                    int64_t n_tokens, int32_t estimator, const double* moments, const float* angles_out) {
    int st = check_shape(shape, dtype);
    if (st != RRP_OK) return st;
    if (estimator < RRP_EST_DEFAULT || estimator > RRP_EST_STREAM_BALANCED) return RRP_ERR_INVALID_ARG;
    if (n_tokens < 0 || moments == nullptr) return RRP_ERR_INVALID_ARG;
    if (n_tokens > 0 && (k == nullptr || pos == nullptr)) return RRP_ERR_INVALID_ARG;
    if (q == nullptr && estimator != RRP_EST_K_ONLY && n_tokens > 0) return RRP_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(pos, 4) || !aligned(moments, 8) || !aligned(angles_out, 4))
        return RRP_ERR_MISALIGNED;
    return RRP_OK;
}

}  // namespace

RRP_EXPORT int rrp_calibrate_angles(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                                    const int32_t* pos, int64_t n_tokens, int32_t estimator,
                                    double* moments, float* angles_out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    int st = check_calibrate(shape, dtype, q, k, pos, n_tokens, estimator, moments, angles_out);
    if (st != RRP_OK) return st;
    st = check_workspace(workspace, workspace_bytes, calib_workspace_bytes(shape, n_tokens, q != nullptr));
    if (st != RRP_OK) return st;
    return calibrate(shape, dtype, q, k, pos, n_tokens, estimator, moments, angles_out,
                     static_cast<double*>(workspace), (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// rrp_calibrate_angles_noalloc: the calibration with its block partials in a
// static device array of this library instead of a caller workspace, for
// callers that cannot allocate.  The array is sized for the largest workspace
// of any accepted shape (kMaxCalibBlocks partial columns of 64 pairs x 5 sums:
// 10 MiB), so no accepted call exceeds it.  Every partial a call reads is
// written earlier by the same call, so nothing needs clearing between calls.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kStaticScratchDoubles = (size_t)rrp::kMaxCalibBlocks * rrp::kMaxPairs * 5;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) double scratch[kStaticScratchDoubles];

namespace {

std::mutex g_scratch_mutex;
double* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (null until looked up)

// The device address of `scratch` on `device`: looked up once per device, with
// that device current (each device holds its own copy of the array).
hipError_t static_scratch(int device, double** out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[device] == nullptr) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = static_cast<double*>(p);
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

}  // namespace

RRP_EXPORT int rrp_calibrate_angles_noalloc(const rrp_shape* shape, int32_t dtype, const void* q, const void* k,
                                            const int32_t* pos, int64_t n_tokens, int32_t estimator,
                                            double* moments, float* angles_out, void* stream) {
    int st = check_calibrate(shape, dtype, q, k, pos, n_tokens, estimator, moments, angles_out);
    if (st != RRP_OK) return st;
    const size_t need = calib_workspace_bytes(shape, n_tokens, q != nullptr);
    if (need > sizeof(scratch)) return RRP_ERR_UNSUPPORTED;  // beyond the static scratch (no accepted shape)
    double* partials = nullptr;
    if (need > 0) {
        int device = -1;
        hipError_t e = stream != nullptr ? hipStreamGetDevice((hipStream_t)stream, &device) : hipGetDevice(&device);
        if (e == hipSuccess) e = static_scratch(device, &partials);
        if (e != hipSuccess) return RRP_ERR_HIP;
    }
    return calibrate(shape, dtype, q, k, pos, n_tokens, estimator, moments, angles_out, partials,
                     (hipStream_t)stream);
}

namespace {

// Shared body of the single-support and sweep diagnostics (support_b is ignored
// by the sweep, which covers b = 1, 2, 4, ..., head_dim).
int quant_error(const rrp_shape* shape, int32_t dtype, const void* k, const int32_t* pos, int64_t n_tokens,
                const float* angles, int32_t support_b, int32_t group, bool sweep, double* stats_out,
                void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_shape(shape, dtype);
    if (st != RRP_OK) return st;
    if ((st = check_b_g(shape, sweep ? 1 : support_b, group)) != RRP_OK) return st;
    if (n_tokens < 0 || stats_out == nullptr) return RRP_ERR_INVALID_ARG;
    if (n_tokens > 0 && (k == nullptr || pos == nullptr)) return RRP_ERR_INVALID_ARG;
    if (!aligned(k, 16) || !aligned(pos, 4) || !aligned(angles, 4) || !aligned(stats_out, 8))
        return RRP_ERR_MISALIGNED;
    if ((st = check_workspace(workspace, workspace_bytes, stats_workspace_bytes(shape, n_tokens, sweep))) != RRP_OK)
        return st;
    const hipStream_t s = (hipStream_t)stream;
    const int n_sets = stats_supports(shape, sweep);
    rrp::StatsFinalArgs f{};
    f.stats_out = stats_out;
    f.n_sets = n_sets;
    f.sweep = sweep ? 1 : 0;
    f.n_rows = (double)n_tokens * shape->n_kv_heads;
    f.n_groups = f.n_rows * (shape->head_dim / group);
    if (n_tokens > 0) {
        const int nb = rrp::stats_blocks(n_tokens, sweep);
        rrp::StatsArgs a{};
        a.k = k;
        a.pos = pos;
        a.angles = angles;
        a.partials = static_cast<double*>(workspace);
        a.n_tokens = n_tokens;
        a.hk = shape->n_kv_heads;
        a.support_b = sweep ? 1 : support_b;
        a.group = group;
        a.angle_sets = angles != nullptr ? angle_sets(shape) : 1;
        a.rsqrt_b = 1.0 / sqrt((double)a.support_b);
        fill_inv_freq(shape, a.inv_freq);
        if (rrp::launch_stats(a, nb, dtype, shape->head_dim, shape->rope_layout, sweep, s) != hipSuccess)
            return RRP_ERR_HIP;
        f.partials = a.partials;
        f.n_blocks = nb;
    }
    return rrp::launch_stats_final(f, s) == hipSuccess ? RRP_OK : RRP_ERR_HIP;
}

}  // namespace

RRP_EXPORT int rrp_quant_error_stats_workspace_size(const rrp_shape* shape, int64_t n_tokens, size_t* bytes) {
    const int st = check_shape(shape, RRP_BF16);
    if (st != RRP_OK) return st;
    if (n_tokens < 0 || bytes == nullptr) return RRP_ERR_INVALID_ARG;
    *bytes = stats_workspace_bytes(shape, n_tokens, false);
    return RRP_OK;
}

RRP_EXPORT int rrp_quant_error_sweep_workspace_size(const rrp_shape* shape, int64_t n_tokens, size_t* bytes) {
    const int st = check_shape(shape, RRP_BF16);
    if (st != RRP_OK) return st;
    if (n_tokens < 0 || bytes == nullptr) return RRP_ERR_INVALID_ARG;
    *bytes = stats_workspace_bytes(shape, n_tokens, true);
    return RRP_OK;
}

RRP_EXPORT int rrp_quant_error_stats(const rrp_shape* shape, int32_t dtype, const void* k, const int32_t* pos,
                                     int64_t n_tokens, const float* angles, int32_t support_b, int32_t group,
                                     double* stats_out, void* workspace, size_t workspace_bytes, void* stream) {
    return quant_error(shape, dtype, k, pos, n_tokens, angles, support_b, group, false, stats_out, workspace,
                       workspace_bytes, stream);
}

RRP_EXPORT int rrp_quant_error_sweep(const rrp_shape* shape, int32_t dtype, const void* k, const int32_t* pos,
                                     int64_t n_tokens, const float* angles, int32_t group, double* stats_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return quant_error(shape, dtype, k, pos, n_tokens, angles, 1, group, true, stats_out, workspace,
                       workspace_bytes, stream);
}

RRP_EXPORT int rrp_decode_scores(const rrp_shape* shape, int32_t dtype, const void* q, int64_t n_seqs,
                                 const uint8_t* k_codes, const uint16_t* k_scales, int32_t group, int64_t n_slots,
                                 const int64_t* seq_start, const int32_t* seq_len, int32_t max_len, float* scores,
                                 void* stream) {
    int st = check_shape(shape, dtype);
    if (st != RRP_OK) return st;
    const int hq = shape->n_q_heads, hk = shape->n_kv_heads, d = shape->head_dim;
    if (hq < 1 || hq % hk != 0) return RRP_ERR_INVALID_ARG;
    if (hq / hk > 16) return RRP_ERR_UNSUPPORTED;  // one MFMA column per query head of a key head
    // A wave's chunk of keys is addressed by 32-bit offsets from its first row.
    // The stated bounds hold for a band of 256 keys, which covers the chunk.
    const int64_t band = rrp::decode_chunk_keys() > 256 ? rrp::decode_chunk_keys() : 256;
    if (band * hk * (d / 2) >= ((int64_t)1 << 31)) return RRP_ERR_UNSUPPORTED;
    if (!is_pow2(group) || group < 2 || group > d) return RRP_ERR_INVALID_ARG;
    if (n_seqs < 0 || n_slots < 0 || max_len < 0) return RRP_ERR_INVALID_ARG;
    if (n_seqs == 0 || max_len == 0) return RRP_OK;
    if (n_slots == 0) return RRP_ERR_INVALID_ARG;  // an empty cache holds no key to read
    // key indices are 32-bit: a chunk's end plus one tile stays below 2^31
    if (max_len > INT32_MAX - 2 * band) return RRP_ERR_UNSUPPORTED;
    if (q == nullptr || k_codes == nullptr || k_scales == nullptr || seq_start == nullptr || seq_len == nullptr ||
        scores == nullptr)
        return RRP_ERR_INVALID_ARG;
    const uintptr_t scale_align = 2 * (d / group) < 8 ? 2 * (d / group) : 8;
    if (!aligned(q, 16) || !aligned(k_codes, d / 8) || !aligned(k_scales, scale_align) || !aligned(seq_start, 8) ||
        !aligned(seq_len, 4) || !aligned(scores, 4))
        return RRP_ERR_MISALIGNED;
    rrp::DecodeArgs a{};
    a.q = q;
    a.k_codes = k_codes;
    a.k_scales = k_scales;
    a.seq_start = seq_start;
    a.seq_len = seq_len;
    a.scores = scores;
    a.n_seqs = n_seqs;
    a.n_slots = n_slots;
    a.n_chunks = rrp::decode_chunks(max_len);
    a.hq = hq;
    a.hk = hk;
    a.group_heads = hq / hk;
    a.max_len = max_len;
    a.vec_store = (max_len % 4 == 0 && aligned(scores, 16)) ? 1 : 0;
    if (rrp::decode_launches(n_seqs, a.n_chunks, hk) < 1) return RRP_ERR_UNSUPPORTED;  // one sequence overfills a grid
    const hipError_t e = rrp::launch_decode_scores(a, dtype, d, group, (hipStream_t)stream);
    return e == hipSuccess ? RRP_OK : RRP_ERR_HIP;
}
