// Log-sum-exp combine of split-K partial results, and the smla_combine entry
// point ("The Moment of Truth: Analyzing a Custom MMA Kernel's Performance on
// Blackwell GPUs", "The Split-K Solution: Reasoning About the Fix": partial
// results over chunks of the top-k list are reduced by a separate combine
// kernel).
//
// For each (row, head) pair:
//   M = max_i lse_i;  lse = M + ln sum_i exp(lse_i - M);
//   out = sum_i exp(lse_i - lse) * part_out_i  (parts with lse_i = -inf are
//   ignored, whatever their part_out holds),
// (part_out in bf16) accumulated in fp32 and rounded to bf16 at the store.  A pair whose parts
// are all empty gets out = 0 and lse = -inf.
//
// One to four waves per pair.  The weights of all parts are computed with
// lane i holding part i (then i + 64, ...) and wave-wide max / sum reductions;
// with at most 64 parts each lane reads its part's lse once, and that value
// serves the max, the sum and the weight (a dependent re-read of the lse costs
// about 0.5 us per call).  The output loop then streams the parts' bf16 rows with 16-byte loads, lane
// l owning 8 consecutive value dims, in batches of 16, 8, 4 or 1 parts
// (fitting S exactly) whose loads are all issued before any is consumed, so a
// pair costs about S / 16 memory round trips rather than S.
#include <hip/hip_runtime.h>

#include <cmath>

#include "smla.h"
#include "smla_internal.h"

namespace smla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Adds parts s_first .. s_first + NB - 1 (weights in lanes w_lane .. w_lane + NB - 1
// of `w`) to the accumulators; all NB loads are issued before any is used (as
// non-temporal loads when NT: the parts were streamed out and are read once).
template <int NB, bool NT>
__device__ __forceinline__ void add_parts(const uint16_t* base, int64_t part_stride, int s_first, int w_lane, float w,
                                          f32x4& acc0, f32x4& acc1) {
    bf16x8 v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const bf16x8* src = (const bf16x8*)(base + (int64_t)(s_first + j) * part_stride);
        v[j] = NT ? __builtin_nontemporal_load(src) : *src;
    }
    // (the scheduler would otherwise interleave loads and uses of a 16-part
    // batch, one round trip per part, to keep the kernel under 64 VGPRs)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), w_lane + j));
        // a select, not a branch, so the loads stay batched; an ignored part
        // (weight 0) adds nothing, not even a NaN
        const bool use = wj != 0.f;
        f32x4 x0, x1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x0[e] = use ? (float)v[j][e] : 0.f;
            x1[e] = use ? (float)v[j][4 + e] : 0.f;
        }
        acc0 += wj * x0;
        acc1 += wj * x1;
    }
}

// d_v == 512: lane l owns dims [8l, 8l + 8).  Grid: one workgroup of NW waves
// per pair; wave w adds the parts of the w-th of NW contiguous ranges and
// waves 1..NW-1 hand their sums to wave 0 through LDS.  Several waves per pair
// put more loads in flight when there are few pairs (small batch).
template <int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void combine_kernel(const uint16_t* __restrict__ part_out,
                                                          const float* __restrict__ part_lse, int num_splits,
                                                          int64_t pairs, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
    __shared__ f32x4 red[NW > 1 ? NW - 1 : 1][2][64];
    // (row, head) pairs are dealt to workgroup ids as the partial kernel deals
    // its (row, part) items: consecutive ids go round-robin over the 8 XCDs, and
    // the pairs of XCD x are the x-th eighth of all pairs, so a row's pairs run
    // on the XCD (and read from the L2) where the partial kernel wrote that
    // row's parts whenever the rows divide evenly over the XCDs.  (A bijection
    // of [0, pairs).)
    const int64_t xcd = blockIdx.x & 7, within = blockIdx.x >> 3;
    const int64_t pair = xcd * (pairs >> 3) + min(xcd, pairs & 7) + within;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const int per_w = (num_splits + NW - 1) / NW;
    const int lo = min(num_splits, w * per_w), hi = min(num_splits, lo + per_w);
    const uint16_t* base = part_out + pair * kDv + 8 * lane;
    const int64_t part_stride = pairs * kDv;
    f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    float total = -INFINITY;
    if (num_splits <= 64) {
        // ---- lane s holds part s's lse: one read serves M, the sum and the weights
        const float l = lane < num_splits ? part_lse[(int64_t)lane * pairs + pair] : -INFINITY;
        const float M = wave_max(l);
        if (M != -INFINITY) {
            total = M + logf(wave_sum(l == -INFINITY ? 0.f : expf(l - M)));
            const float wt = l == -INFINITY ? 0.f : expf(l - total);  // weight of part `lane`
            const int n = hi - lo;
            int j0 = 0;
            for (; j0 + 16 <= n; j0 += 16) add_parts<16, NT>(base, part_stride, lo + j0, lo + j0, wt, acc0, acc1);
            if (j0 + 8 <= n) { add_parts<8, NT>(base, part_stride, lo + j0, lo + j0, wt, acc0, acc1); j0 += 8; }
            if (j0 + 4 <= n) { add_parts<4, NT>(base, part_stride, lo + j0, lo + j0, wt, acc0, acc1); j0 += 4; }
            for (; j0 < n; ++j0) add_parts<1, NT>(base, part_stride, lo + j0, lo + j0, wt, acc0, acc1);
        }
    } else {
        // ---- weights: M, z and lse over all parts (lane i holds parts i, i+64, ...), in every wave
        float M = -INFINITY;
        for (int s = lane; s < num_splits; s += 64) M = fmaxf(M, part_lse[(int64_t)s * pairs + pair]);
        M = wave_max(M);
        if (M != -INFINITY) {
            float z = 0.f;
            for (int s = lane; s < num_splits; s += 64) {
                const float l = part_lse[(int64_t)s * pairs + pair];
                z += l == -INFINITY ? 0.f : expf(l - M);
            }
            total = M + logf(wave_sum(z));
        }
        if (total != -INFINITY) {
            for (int s0 = lo; s0 < hi; s0 += 64) {
                // weight of part s0 + lane (0 for an empty part or past the range)
                float wt = 0.f;
                if (s0 + lane < hi) {
                    const float l = part_lse[(int64_t)(s0 + lane) * pairs + pair];
                    wt = l == -INFINITY ? 0.f : expf(l - total);
                }
                const int n = min(64, hi - s0);
                int j0 = 0;
                for (; j0 + 16 <= n; j0 += 16) add_parts<16, NT>(base, part_stride, s0 + j0, j0, wt, acc0, acc1);
                if (j0 + 8 <= n) { add_parts<8, NT>(base, part_stride, s0 + j0, j0, wt, acc0, acc1); j0 += 8; }
                if (j0 + 4 <= n) { add_parts<4, NT>(base, part_stride, s0 + j0, j0, wt, acc0, acc1); j0 += 4; }
                for (; j0 < n; ++j0) add_parts<1, NT>(base, part_stride, s0 + j0, j0, wt, acc0, acc1);
            }
        }
    }
    if (NW > 1) {
        if (w > 0) {
            red[w - 1][0][lane] = acc0;
            red[w - 1][1][lane] = acc1;
        }
        __syncthreads();
        if (w > 0) return;
#pragma unroll
        for (int i = 0; i < NW - 1; ++i) {
            acc0 += red[i][0][lane];
            acc1 += red[i][1][lane];
        }
    }
    bf16x8 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[j] = (__bf16)acc0[j];
        o[4 + j] = (__bf16)acc1[j];
    }
    *(bf16x8*)(out + pair * kDv + 8 * lane) = o;
    if (lane == 0) lse[pair] = total;
}

}  // namespace

template <bool NT>
void launch_combine_nt(const uint16_t* part_out, const float* part_lse, int num_splits, int64_t pairs, void* out,
                       float* lse, hipStream_t stream) {
    // few pairs (small batch): four waves per pair so that more part loads are in flight
    if (pairs <= 512)
        hipLaunchKernelGGL((combine_kernel<4, NT>), dim3((unsigned)pairs), dim3(256), 0, stream, part_out, part_lse,
                           num_splits, pairs, (uint16_t*)out, lse);
    else
        hipLaunchKernelGGL((combine_kernel<1, NT>), dim3((unsigned)pairs), dim3(64), 0, stream, part_out, part_lse,
                           num_splits, pairs, (uint16_t*)out, lse);
}

// stream_parts: the parts were written with non-temporal stores (they are
// then read with non-temporal loads too).
smla_status_t launch_combine(const uint16_t* part_out, const float* part_lse, int num_splits, int64_t pairs,
                             void* out, float* lse, hipStream_t stream, bool stream_parts) {
    if (pairs == 0) return SMLA_OK;
    if (stream_parts)
        launch_combine_nt<true>(part_out, part_lse, num_splits, pairs, out, lse, stream);
    else
        launch_combine_nt<false>(part_out, part_lse, num_splits, pairs, out, lse, stream);
    return hipGetLastError() == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

}  // namespace smla

extern "C" smla_status_t smla_combine(const void* part_out, const float* part_lse, int32_t num_splits,
                                      int32_t rows, int32_t num_heads, int32_t d_v, void* out, float* lse,
                                      void* stream) {
    if (num_splits < 1 || rows < 0 || num_heads < 0 || d_v <= 0) return SMLA_ERR_INVALID_ARG;
    if (d_v != smla::kDv) return SMLA_ERR_UNSUPPORTED;
    const int64_t pairs = (int64_t)rows * num_heads;
    if (pairs == 0) return SMLA_OK;
    if (pairs > 0x7fffffffLL) return SMLA_ERR_UNSUPPORTED;
    if (!part_out || !part_lse || !out || !lse) return SMLA_ERR_INVALID_ARG;
    if (((uintptr_t)part_out & 15) != 0 || ((uintptr_t)out & 15) != 0) return SMLA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    return smla::launch_combine((const uint16_t*)part_out, part_lse, num_splits, pairs, out, lse, (hipStream_t)stream,
                                false);
}
