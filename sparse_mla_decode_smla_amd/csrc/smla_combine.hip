// Log-sum-exp combine of split-K partial results, and the smla_combine entry
// point ("The Moment of Truth: Analyzing a Custom MMA Kernel's Performance on
// Blackwell GPUs", "The Split-K Solution: Reasoning About the Fix": partial
// results over chunks of the top-k list are reduced by a separate combine
// kernel).
//
// For each (row, head) pair and each 4-wide slice of the value dims:
//   M = max_i lse_i;  lse = M + ln sum_i exp(lse_i - M);
//   out = sum_i exp(lse_i - lse) * part_out_i  (parts with lse_i = -inf skipped),
// accumulated in fp32 and rounded to bf16 at the store.  A pair whose parts
// are all empty gets out = 0 and lse = -inf.  Memory bound: every partial
// byte is read once with 16-byte loads, consecutive threads on consecutive
// slices of the same pair.
#include <hip/hip_runtime.h>

#include <cmath>

#include "smla.h"
#include "smla_internal.h"

namespace smla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ part_out,
                                                                  const float* __restrict__ part_lse,
                                                                  int num_splits, int64_t pairs, int d_v,
                                                                  uint16_t* __restrict__ out,
                                                                  float* __restrict__ lse) {
    const int slices = d_v / 4;
    const int64_t items = pairs * slices;
    for (int64_t it = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x; it < items;
         it += (int64_t)gridDim.x * kCombineThreads) {
        const int64_t pair = it / slices;
        const int c = (int)(it - pair * slices);
        float M = -INFINITY;
        for (int s = 0; s < num_splits; ++s) M = fmaxf(M, part_lse[(int64_t)s * pairs + pair]);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        float total = -INFINITY;
        if (M != -INFINITY) {
            float z = 0.f;
            for (int s = 0; s < num_splits; ++s) {
                const float l = part_lse[(int64_t)s * pairs + pair];
                if (l != -INFINITY) z += expf(l - M);
            }
            total = M + logf(z);
            for (int s = 0; s < num_splits; ++s) {
                const float l = part_lse[(int64_t)s * pairs + pair];
                if (l == -INFINITY) continue;
                const f32x4 v = *(const f32x4*)(part_out + ((int64_t)s * pairs + pair) * d_v + 4 * c);
                acc += expf(l - total) * v;
            }
        }
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (__bf16)acc[j];
        *(bf16x4*)(out + pair * d_v + 4 * c) = o;
        if (c == 0) lse[pair] = total;
    }
}

}  // namespace

smla_status_t launch_combine(const float* part_out, const float* part_lse, int num_splits, int64_t pairs,
                             int d_v, void* out, float* lse, hipStream_t stream) {
    const int64_t items = pairs * (d_v / 4);
    if (items == 0) return SMLA_OK;
    int64_t blocks = (items + kCombineThreads - 1) / kCombineThreads;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream, part_out,
                       part_lse, num_splits, pairs, d_v, (uint16_t*)out, lse);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace smla

extern "C" smla_status_t smla_combine(const float* part_out, const float* part_lse, int32_t num_splits,
                                      int32_t rows, int32_t num_heads, int32_t d_v, void* out, float* lse,
                                      void* stream) {
    if (num_splits < 1 || rows < 0 || num_heads < 0 || d_v <= 0) return SMLA_ERR_INVALID_ARG;
    if (d_v % 4 != 0) return SMLA_ERR_UNSUPPORTED;
    const int64_t pairs = (int64_t)rows * num_heads;
    if (pairs == 0) return SMLA_OK;
    if (!part_out || !part_lse || !out || !lse) return SMLA_ERR_INVALID_ARG;
    if (((uintptr_t)part_out & 15) != 0 || ((uintptr_t)out & 7) != 0) return SMLA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return smla::launch_combine(part_out, part_lse, num_splits, pairs, d_v, out, lse, (hipStream_t)stream);
}
