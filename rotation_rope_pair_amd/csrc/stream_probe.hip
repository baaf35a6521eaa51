// stream_probe.hip -- the practical HBM streaming rates of the GPU, measured
// by plain kernels of known traffic (a measurement aid for the benchmark, not
// part of the rrp C-ABI; built into its own library, libstream_probe.so).
//
//   stream_probe_copy   reads n bytes and writes n bytes
//   stream_probe_read   reads n bytes (xor-folded; one store per thread, only
//                       when the fold hits a value no real input produces, so
//                       the loads cannot be dropped)
//   stream_probe_write  writes n bytes
//
// Each thread makes one 16-byte non-temporal access (copy: one load and one
// store) and the grid covers the buffer once, with no loop.  Waves are then
// dispatched in address order and the running ones stay in one narrow band
// of memory.  Measured on MI355X, 1 GiB buffers: this pattern reached the
// highest rates of the patterns tried.  The alternatives were grid-stride
// loops with 1-16 accesses in flight per thread, per-block contiguous chunks
// of 1-16 accesses per thread, and 8-byte loads.  Copy 6.5 TB/s against
// 5.2-6.0, write 6.7 against 4.4-6.0, read 7.1 against 6.2-7.3.
// n must be a multiple of 16 and the pointers 16-byte aligned (checked).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define PROBE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        size_t n) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                        unsigned* __restrict__ sink) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const unsigned v = a.x ^ a.y ^ a.z ^ a.w;
        if (v == 0x9E3779B9u) sink[0] = v;  // keeps the load; practically never taken
    }
}

__global__ __launch_bounds__(kThreads) void write_kernel(u32x4* __restrict__ dst, size_t n) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) __builtin_nontemporal_store(u32x4{(unsigned)i, 1u, 2u, 3u}, dst + i);
}

// One thread per 16 bytes; 0 for a size no grid can cover.
unsigned blocks_for(size_t n16) {
    const size_t b = (n16 + kThreads - 1) / kThreads;
    return b >= 1 && b <= 0x7FFFFFFFu ? (unsigned)b : 0u;
}

bool ok(const void* p, size_t bytes) { return p != nullptr && ((uintptr_t)p & 15) == 0 && (bytes & 15) == 0; }

}  // namespace

// Each returns 0 when enqueued (or for an empty buffer), 1 for a bad argument,
// 2 for a failed launch.
PROBE_EXPORT int stream_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!ok(src, bytes) || !ok(dst, bytes)) return 1;
    const size_t n = bytes / 16;
    if (n == 0) return 0;
    const unsigned blocks = blocks_for(n);
    if (blocks == 0) return 1;
    hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

PROBE_EXPORT int stream_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
    if (!ok(src, bytes) || sink == nullptr) return 1;
    const size_t n = bytes / 16;
    if (n == 0) return 0;
    const unsigned blocks = blocks_for(n);
    if (blocks == 0) return 1;
    hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const u32x4*>(src), n, static_cast<unsigned*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

PROBE_EXPORT int stream_probe_write(void* dst, size_t bytes, void* stream) {
    if (!ok(dst, bytes)) return 1;
    const size_t n = bytes / 16;
    if (n == 0) return 0;
    const unsigned blocks = blocks_for(n);
    if (blocks == 0) return 1;
    hipLaunchKernelGGL(write_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<u32x4*>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
