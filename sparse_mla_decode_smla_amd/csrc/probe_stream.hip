// Measurement probes used by the benchmark (not part of the decode library).
//
// Stream read: a measured bandwidth reference next to the 8 TB/s peak: one
// pass over a buffer with 16-byte non-temporal loads, four in flight per
// lane, spread over a grid that fills the chip.  Each lane folds what it read
// into one word and stores it, so the loads cannot be dropped; the stores are
// 4 bytes per lane, negligible next to the bytes read.
//
// Row gather: random 1152-byte rows moved into LDS by 16-byte LDS-DMA
// (global_load_lds_dwordx4), as the decode kernel gathers latent rows, with
// different spreads of one instruction's 64 lanes over rows.  Four issuing
// waves per workgroup, each taking 8 rows per tile into its own ring of 4
// stages with 3 tiles in flight, no compute; the workgroup's row numbers are
// first copied into LDS (as the decode kernel holds its row table), so that
// no global load of a row number waits behind the gathers in flight.  Modes (the 64 lanes of one
// 1 KB instruction): 0 = 8 rows x 128 bytes, 8 consecutive lanes per row (the
// kernel's band-major gather); 1 = 1 row x 1024 bytes (row-major; a ninth
// instruction takes the 8 rows' last 128 bytes); 2 = the same 8 rows x 128
// bytes as 0, lanes ordered by half band (lane l takes bytes
// 64 (l / 32) + 16 (l % 4) of row (l / 4) % 8); 3 = the same bytes, lanes
// interleaved by row (lane l takes chunk l / 8 of row l % 8); 4 = mode 0 with
// the loads marked non-temporal (the nt bit).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* src, unsigned lds_base) {
    if (NT)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src),
                     "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
                     "s"(__builtin_amdgcn_readfirstlane(lds_base))
                     : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

constexpr int kRow = 1152, kTileRows = 32, kStages = 4, kWaveStage = 8 * kRow;  // 9216 bytes
constexpr int kRowTab = 4 * kStages * kWaveStage;  // LDS offset of the row numbers
constexpr int kMaxTiles = 64;                      // row numbers held: kMaxTiles * kTileRows

template <int MODE>
__global__ __launch_bounds__(256) void gather_kernel(const unsigned char* __restrict__ buf,
                                                     const int* __restrict__ rows, int ntiles,
                                                     unsigned* __restrict__ sink) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const unsigned base = (unsigned)(uintptr_t)lds + (unsigned)(w * kStages * kWaveStage);
    int* tab = (int*)(lds + kRowTab);
    for (int i = threadIdx.x; i < ntiles * kTileRows; i += blockDim.x)
        tab[i] = rows[(size_t)blockIdx.x * ntiles * kTileRows + i];
    __syncthreads();
    const int* my = tab + 8 * w;
    for (int t = 0; t < ntiles; ++t) {
        const unsigned st = base + (unsigned)((t % kStages) * kWaveStage);
        if (MODE == 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) dma16(buf + (size_t)my[t * kTileRows + j] * kRow + lane * 16, st + j * 1024);
            dma16(buf + (size_t)my[t * kTileRows + (lane >> 3)] * kRow + 1024 + (lane & 7) * 16, st + 8 * 1024);
        } else {
            int r, off;
            if (MODE == 0 || MODE == 4) { r = lane >> 3; off = (lane & 7) * 16; }
            else if (MODE == 2) { r = (lane >> 2) & 7; off = (lane >> 5) * 64 + (lane & 3) * 16; }
            else { r = lane & 7; off = (lane >> 3) * 16; }
            const unsigned char* src = buf + (size_t)my[t * kTileRows + r] * kRow + off;
#pragma unroll
            for (int b = 0; b < 9; ++b) dma16<MODE == 4>(src + b * 128, st + b * 1024);
        }
        if (t >= kStages - 1) wait_vm<9 * (kStages - 1)>();
    }
    wait_vm<0>();
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = *(volatile unsigned*)lds;
}

// Launch floor: a kernel that does almost nothing (thread 0 of each
// workgroup stores one word), for timing a graph of back-to-back launches.
__global__ void empty_kernel(unsigned* __restrict__ sink, unsigned v) {
    if (threadIdx.x == 0) sink[blockIdx.x] = v;
}

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

// buf: nrows rows of 1152 bytes; rows: int32 [grid, ntiles, 32] row numbers, each in [0, nrows), ntiles <= 64;
// sink: grid words.  One launch of `grid` workgroups of 256 threads with 155,648 bytes of LDS.  Returns 0 on a
// successful launch, -1 on bad arguments, else the HIP error.
extern "C" int smla_probe_gather(const void* buf, const int* rows, int ntiles, int mode, unsigned* sink, int grid,
                                 void* stream) {
    if (!buf || !rows || !sink || grid <= 0 || ntiles <= 0 || ntiles > kMaxTiles || mode < 0 || mode > 4) return -1;
    const size_t lds = kRowTab + 4 * kMaxTiles * kTileRows;
    const void* fns[5] = {(const void*)gather_kernel<0>, (const void*)gather_kernel<1>, (const void*)gather_kernel<2>,
                          (const void*)gather_kernel<3>, (const void*)gather_kernel<4>};
    hipError_t e = hipFuncSetAttribute(fns[mode], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    const unsigned char* b = (const unsigned char*)buf;
    hipStream_t st = (hipStream_t)stream;
    switch (mode) {
        case 0: hipLaunchKernelGGL(gather_kernel<0>, dim3(grid), dim3(256), lds, st, b, rows, ntiles, sink); break;
        case 1: hipLaunchKernelGGL(gather_kernel<1>, dim3(grid), dim3(256), lds, st, b, rows, ntiles, sink); break;
        case 2: hipLaunchKernelGGL(gather_kernel<2>, dim3(grid), dim3(256), lds, st, b, rows, ntiles, sink); break;
        case 4: hipLaunchKernelGGL(gather_kernel<4>, dim3(grid), dim3(256), lds, st, b, rows, ntiles, sink); break;
        default: hipLaunchKernelGGL(gather_kernel<3>, dim3(grid), dim3(256), lds, st, b, rows, ntiles, sink); break;
    }
    return (int)hipGetLastError();
}

// buf: device buffer of `bytes` bytes (16-byte aligned, bytes a multiple of
// 16); sink: device buffer of grid * 256 unsigned words.  Returns 0 on a
// successful launch on `stream`, -1 on bad arguments, else the HIP error.
extern "C" int smla_probe_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, void* stream) {
    if (!buf || !sink || grid <= 0 || (bytes & 15) || ((uintptr_t)buf & 15)) return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf,
                       bytes / 16, sink);
    return (int)hipGetLastError();
}

// sink: device buffer of at least grid unsigned words; 1 <= threads <= 1024.  Enqueues one launch of
// `grid` workgroups of `threads` threads on `stream`.  Returns 0, -1 on bad arguments, else the HIP error.
extern "C" int smla_probe_empty(unsigned* sink, int grid, int threads, unsigned value, void* stream) {
    if (!sink || grid <= 0 || threads <= 0 || threads > 1024) return -1;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(threads), 0, (hipStream_t)stream, sink, value);
    return (int)hipGetLastError();
}
