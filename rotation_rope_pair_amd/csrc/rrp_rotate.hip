// rrp_rotate.hip -- fused RoPE + pair rotation + block FWHT + INT4 KV4 quantisation.
//
// Each wavefront walks tokens with a grid stride (for batches small enough that
// every row pass of every token can have a wave of its own, the passes are
// split over that many waves instead, so a decode batch is not serialised on
// one wave per token).  For
// one token it issues the 128-bit loads of its Q rows and K rows first (R rows
// per pass, each row's two 16-byte chunks per lane), evaluates the token's rotation table once (one
// pair per lane, shared by every head of the token through LDS), then runs
// the Q passes and the K passes: RoPE + R_phi as one complex multiply per pair
// (with the half-head butterfly folded in when b = head_dim), the remaining
// Walsh-Hadamard butterflies in registers and across lanes (one fused DPP
// multiply-add per value), and either the Q store (bf16 nearest-even / fp32)
// or the K group quantisation with nibble-packed codes and fp16 scales written
// at the token's cache slot.  Q rows are computed in fp32, K rows in fp64 (the
// group scales and codes then follow the definition for any group size).
// Every input byte is read once and every output byte written once, with
// streaming (non-temporal) hints: the kernel is bound by HBM bandwidth and by
// the vector ALU.
#include "rrp_rotate_kernel.hpp"

namespace rrp {

// The split family runs a batch only when each of its row passes gets a wave of
// its own (n_tokens x passes per token <= kSmallBatchWaves).  Where waves would
// have to take unequal shares of a token, one wave per token measured faster
// (2048 tokens of 32/8 heads at d 64: 7.8 against 9.1 us; 1024 tokens at
// d 128: 8.5 against 9.3 us); below the bound the split family is faster
// (512 tokens at d 128: 5.7 against 7.8 us).
hipError_t launch_rotate_quantize(const RotateArgs& a, int dtype, int head_dim, int layout, hipStream_t st) {
    if (a.n_tokens > 0 && head_dim > 0) {
        const int rows = 2048 / (head_dim * (dtype == 1 ? 2 : 4));  // rows per wave pass (Geo<E, D>::R)
        const int64_t nq = (a.hq_rows + rows - 1) / rows, nk = (a.hk + rows - 1) / rows;
        const int64_t npass = nq + (a.v != nullptr ? 2 : 1) * nk;
        if (a.n_tokens * npass <= kSmallBatchWaves) return launch_rotate_quantize_split(a, dtype, head_dim, layout, st);
    }
    return dispatch<false>(a, dtype, head_dim, layout, st);
}

}  // namespace rrp
