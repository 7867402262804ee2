// fp32 attention parts for tree verification (the fp32-input path).
//
// Same partial outputs as the bf16 kernel -- one (O, LSE) per (part, row) for a prefix chunk,
// plus the masked tree keys in the last part -- computed with plain fp32 vector arithmetic: there is no fp32 MFMA
// shape worth using at these sizes. One wavefront per (row, part); every lane walks its own
// subset of keys with an online softmax, then the 64 lane partials are merged through LDS by the
// log-sum-exp identity.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace ta {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
    __shared__ float qs[D];
    __shared__ float red[64][D + 1];
    __shared__ float lm[64], ll[64];
    __shared__ uint32_t anc[TA_MAX_TREE / 32];

    const int lane = threadIdx.x;
    const int64_t row = blockIdx.x;  // (b * T + node) * Hq + h
    const int part = blockIdx.y;
    const int h = (int)(row % a.Hq);
    const int node = (int)((row / a.Hq) % a.T);
    const int b = (int)(row / ((int64_t)a.Hq * a.T));
    const int g = h / a.G;
    const bool has_tree = a.with_tree && part == a.n_splits - 1;
    if (a.seq_parts && a.with_prefix && row == 0 && part == 0)
        for (int i = lane; i < a.B; i += 64) a.seq_parts[i] = a.n_splits;

    const float *q = reinterpret_cast<const float *>(a.q) + b * a.q_sb + node * a.q_st + h * a.q_sh;
    for (int d = lane; d < D; d += 64) qs[d] = q[d];

    // prefix keys [pb, pe) of this part
    int pb = 0, pe = 0;
    if (a.with_prefix) {
        int L = a.seq_lens[b];
        if (L < 0 || L > a.capacity) {
            if (a.err && lane == 0) atomicOr(a.err, (int32_t)TA_DEV_BAD_LEN);
            L = L < 0 ? 0 : a.capacity;
        }
        pb = part * a.chunk;
        pe = min(pb + a.chunk, L);
        if (pe < pb) pe = pb;
    }
    // ancestor-or-self bitmap of `node`, walked upwards from the node itself
    for (int w = lane; w < TA_MAX_TREE / 32; w += 64) anc[w] = 0u;
    __syncthreads();
    if (has_tree && lane == 0) {
        const int32_t *par = a.parent + (int64_t)b * a.T;
        int j = node;
        while (j >= 0) {
            anc[j >> 5] |= 1u << (j & 31);
            const int p = par[j];
            if (p < -1 || p >= j) {
                if (a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_PARENT);
                break;
            }
            j = p;
        }
    }
    __syncthreads();

    float m = -INFINITY, l = 0.f, acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = 0.f;
    const int n_keys = (pe - pb) + (has_tree ? a.T : 0);
    for (int k = lane; k < n_keys; k += 64) {
        const float *kp, *vp;
        if (k >= pe - pb) {
            const int j = k - (pe - pb);
            if (!((anc[j >> 5] >> (j & 31)) & 1u)) continue;
            const int64_t off = b * a.kt_sb + j * a.kt_st + g * a.kt_sh;
            kp = reinterpret_cast<const float *>(a.kt) + off;
            vp = reinterpret_cast<const float *>(a.vt) + off;
        } else {
            const int j = pb + k;
            int64_t off;
            if (a.block_table) {
                const int pg = a.block_table[(int64_t)b * a.max_blocks + (j >> a.page_shift)];
                if ((unsigned)pg >= (unsigned)a.num_pages) {
                    if (a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_PAGE);
                    continue;
                }
                off = pg * a.kv_s0 + (j & a.page_mask) * a.kv_s1 + g * a.kv_s2;
            } else {
                off = b * a.kv_s0 + j * a.kv_s1 + g * a.kv_s2;
            }
            kp = reinterpret_cast<const float *>(a.kc) + off;
            vp = reinterpret_cast<const float *>(a.vc) + off;
        }
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(kp + d);
            s = fmaf(qs[d], k4.x, s);
            s = fmaf(qs[d + 1], k4.y, s);
            s = fmaf(qs[d + 2], k4.z, s);
            s = fmaf(qs[d + 3], k4.w, s);
        }
        s *= a.scale;
        if (s > m) {
            const float alpha = m == -INFINITY ? 0.f : expf(m - s);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] *= alpha;
            m = s;
        }
        const float p = expf(s - m);
        l += p;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
            const float4 v4 = *reinterpret_cast<const float4 *>(vp + d);
            acc[d] = fmaf(p, v4.x, acc[d]);
            acc[d + 1] = fmaf(p, v4.y, acc[d + 1]);
            acc[d + 2] = fmaf(p, v4.z, acc[d + 2]);
            acc[d + 3] = fmaf(p, v4.w, acc[d + 3]);
        }
    }

    // merge the 64 lane partials
    lm[lane] = m;
    __syncthreads();
    float mx = -INFINITY;
    for (int i = 0; i < 64; ++i) mx = fmaxf(mx, lm[i]);
    const float f = (m == -INFINITY) ? 0.f : expf(m - mx);
    ll[lane] = l * f;
#pragma unroll
    for (int d = 0; d < D; ++d) red[lane][d] = acc[d] * f;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < 64; ++i) tot += ll[i];
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    float *op = a.out_o + part * a.part_so + row * D;
    for (int d = lane; d < D; d += 64) {
        float s = 0.f;
        for (int i = 0; i < 64; ++i) s += red[i][d];
        op[d] = s * inv;
    }
    if (lane == 0) a.out_lse[part * a.part_sl + row] = tot > 0.f ? mx + logf(tot) : -INFINITY;
}

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s) {
    const int parts = a.n_splits;
    const int64_t rows = (int64_t)a.B * a.T * a.Hq;
    if (parts == 0 || rows == 0) return hipSuccess;
    const dim3 grid((unsigned)rows, parts);
    if (a.D == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace ta
