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
// A row's parts are merged by a group of D / 4 lanes (16 bytes of the row per lane, so a
// wavefront takes 64 / (D / 4) rows): the lanes read the parts' LSEs and reduce them across the
// group, then every lane accumulates its four output columns over the parts, in part order.
template <int D, typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs m) {
    constexpr int LPR = D / 4;           // lanes per row
    constexpr int RPW = 64 / LPR;        // rows per wavefront
    const int lane = threadIdx.x & 63, gl = lane % LPR, gbase = lane - gl;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
    const bool live = row < m.rows;
    const int64_t rr = live ? row : 0;   // rows past the end follow row 0 and store nothing
    const int n0 = m.seq_parts ? m.seq_parts[rr / m.seq_rows] : m.n0;
    const int n = n0 + (m.o1 ? 1 : 0);
    auto part_lse = [&](int p) -> float { return p < n0 ? m.lse0[p * m.sl0 + rr] : m.lse1[rr]; };
    auto part_o = [&](int p) -> const float * {
        return p < n0 ? m.o0 + p * m.so0 + rr * D : m.o1 + rr * D;
    };
    // the parts of the rows of one wavefront may differ in number: every group loops to the
    // largest count, the others' lanes idle
    int nmax = n;
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) nmax = max(nmax, __shfl_xor(nmax, o));

    float mx = -INFINITY;
    for (int c = 0; c < nmax; c += LPR)
        if (c + gl < n) mx = fmaxf(mx, part_lse(c + gl));
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float total = 0.f;
    const bool any = mx != -INFINITY;
    for (int c = 0; c < nmax; c += LPR) {
        const float w = (any && c + gl < n) ? expf(part_lse(c + gl) - mx) : 0.f;
        total += w;
        const int cn = min(LPR, nmax - c);
        for (int k = 0; k < cn; ++k) {
            const float wk = __shfl(w, gbase + k);
            if (wk == 0.f) continue;  // empty part (LSE = -inf), or past this row's parts
            const float4 v = *reinterpret_cast<const float4 *>(part_o(c + k) + gl * 4);
            acc.x += wk * v.x;
            acc.y += wk * v.y;
            acc.z += wk * v.z;
            acc.w += wk * v.w;
        }
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) total += __shfl_xor(total, o);
    if (!live) return;
    const float inv = total > 0.f ? 1.f / total : 0.f;
    OutT *o = reinterpret_cast<OutT *>(m.o) + row * D + gl * 4;
    o[0] = (OutT)(acc.x * inv);
    o[1] = (OutT)(acc.y * inv);
    o[2] = (OutT)(acc.z * inv);
    o[3] = (OutT)(acc.w * inv);
    if (gl == 0) m.lse[row] = total > 0.f ? mx + logf(total) : -INFINITY;
}

hipError_t launch_merge(const MergeArgs &m, bool out_bf16, hipStream_t s) {
    if (m.rows == 0) return hipSuccess;
    const int rpw = 64 / (m.D / 4);  // rows per wavefront
    const dim3 grid((unsigned)((m.rows + 4 * rpw - 1) / (4 * rpw))), block(256);
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
