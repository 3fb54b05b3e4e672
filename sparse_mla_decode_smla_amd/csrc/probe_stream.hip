// Stream-read probe used by the benchmark as a measured bandwidth reference
// next to the 8 TB/s peak: one pass over a buffer with 16-byte non-temporal
// loads, four in flight per lane, spread over a grid that fills the chip.
// Each lane folds what it read into one word and stores it, so the loads
// cannot be dropped; the stores are 4 bytes per lane, negligible next to the
// bytes read.  Not part of the decode library.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                          unsigned* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 acc = u32x4{0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        const u32x4 b = __builtin_nontemporal_load(p + i + stride);
        const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

// buf: device buffer of `bytes` bytes (16-byte aligned, bytes a multiple of
// 16); sink: device buffer of grid * 256 unsigned words.  Returns 0 on a
// successful launch on `stream`, -1 on bad arguments, else the HIP error.
extern "C" int smla_probe_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, void* stream) {
    if (!buf || !sink || grid <= 0 || (bytes & 15) || ((uintptr_t)buf & 15)) return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf,
                       bytes / 16, sink);
    return (int)hipGetLastError();
}
