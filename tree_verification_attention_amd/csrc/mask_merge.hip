// Tree-mask construction and the log-sum-exp merge of partial attention results.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ancestors.h"
#include "launch.h"

namespace ta {

// ------------------------------------------------------------------------------------------
// tree_mask_build: one workgroup per tree. Output mask[b][i][w], W = ceil(T / 64) words per row.

__global__ __launch_bounds__(256) void mask_kernel(const int32_t *parent, int T, uint64_t *mask,
                                                   int32_t *err) {
    __shared__ AncestorLds s;
    const int b = blockIdx.x;
    const int cur = build_ancestor_masks(parent + (int64_t)b * T, T, s, err, threadIdx.x, 256);
    const int W = (T + 63) >> 6;
    uint64_t *out = mask + (int64_t)b * T * W;
    for (int e = threadIdx.x; e < T * W; e += 256) out[e] = s.m[cur][e / W][e % W];
}

hipError_t launch_mask(const int32_t *parent, int B, int T, uint64_t *mask, int32_t *err,
                       hipStream_t s) {
    hipLaunchKernelGGL(mask_kernel, dim3(B), dim3(256), 0, s, parent, T, mask, err);
    return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Merge. For one output row with parts p = 1..n carrying (o_p, LSE_p), the aggregation of the
// LongSpec page ("Fast tree attention", aggregation equations) extended to n parts is
//     LSE = M + ln sum_p exp(LSE_p - M),   O = sum_p exp(LSE_p - LSE) o_p,   M = max_p LSE_p.
// One wavefront per row: lanes read the parts' LSEs and reduce them across the wavefront, then
// every lane accumulates its slice of the D output columns over the parts.

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <int D, typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs m) {
    constexpr int PER_LANE = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= m.rows) return;
    const int n0 = m.seq_parts ? m.seq_parts[row / m.seq_rows] : m.n0;
    const int n = n0 + (m.o1 ? 1 : 0);

    auto part_lse = [&](int p) -> float {
        return p < n0 ? m.lse0[p * m.sl0 + row] : m.lse1[row];
    };
    auto part_o = [&](int p) -> const float * {
        return p < n0 ? m.o0 + p * m.so0 + row * D : m.o1 + row * D;
    };

    float mx = -INFINITY;
    for (int c = 0; c < n; c += 64)
        if (c + lane < n) mx = fmaxf(mx, part_lse(c + lane));
    mx = wave_max(mx);

    float acc[PER_LANE];
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) acc[e] = 0.f;
    float total = 0.f;
    if (mx != -INFINITY) {
        for (int c = 0; c < n; c += 64) {
            const float w = (c + lane < n) ? expf(part_lse(c + lane) - mx) : 0.f;
            total += w;
            const int cn = min(64, n - c);
            for (int k = 0; k < cn; ++k) {
                const float wk = __shfl(w, k);
                if (wk == 0.f) continue;  // empty part (LSE = -inf): its O is never read
                const float *op = part_o(c + k) + lane * PER_LANE;
                if constexpr (PER_LANE == 2) {
                    const float2 v = *reinterpret_cast<const float2 *>(op);
                    acc[0] += wk * v.x;
                    acc[1] += wk * v.y;
                } else {
                    acc[0] += wk * op[0];
                }
            }
        }
        total = wave_sum(total);
    }
    const float inv = total > 0.f ? 1.f / total : 0.f;
    OutT *o = reinterpret_cast<OutT *>(m.o) + row * D + lane * PER_LANE;
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) o[e] = (OutT)(acc[e] * inv);
    if (lane == 0) m.lse[row] = total > 0.f ? mx + logf(total) : -INFINITY;
}

hipError_t launch_merge(const MergeArgs &m, bool out_bf16, hipStream_t s) {
    if (m.rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((m.rows + 3) / 4)), block(256);
    if (m.D == 128) {
        if (out_bf16)
            hipLaunchKernelGGL((merge_kernel<128, __bf16>), grid, block, 0, s, m);
        else
            hipLaunchKernelGGL((merge_kernel<128, float>), grid, block, 0, s, m);
    } else {
        if (out_bf16)
            hipLaunchKernelGGL((merge_kernel<64, __bf16>), grid, block, 0, s, m);
        else
            hipLaunchKernelGGL((merge_kernel<64, float>), grid, block, 0, s, m);
    }
    return hipGetLastError();
}

}  // namespace ta
