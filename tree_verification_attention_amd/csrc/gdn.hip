// Tree verification of gated-delta-net layers on gfx950 (DFlash-TfM summary page,
// "Rollback-free tree verification for GDN").
//
// A GDN layer updates a d_k x d_v state per token as S_t = a_t (I - b_t k_t k_t^T) S_{t-1} +
// b_t k_t v_t^T (a_t = e^{g_t}); on a draft tree every node continues its parent's state (a
// root-attached node continues the committed state S_0) and emits o_t = scale * S_t^T q_t.
// Unrolling the recurrence along a node's root path (the chunked form of a linear recurrence)
// gives, with G_t = sum of g over t and its ancestors,
//
//   S_t = e^{G_t} S_0 + sum_{j in path(t)} e^{G_t - G_j} k_j u_j^T,
//   u_t + sum_{j strict ancestor of t} b_t e^{G_t - G_j} (k_t . k_j) u_j = b_t (v_t - e^{G_t} S_0^T k_t),
//   o_t = scale * (e^{G_t} S_0^T q_t + sum_{j ancestor or self} e^{G_t - G_j} (q_t . k_j) u_j):
//
// the page's (I + X) U = beta V with X the strictly-ancestral interaction matrix (and the S_0
// term on the right), Y the ancestral-or-self one for the output. The matrix is lower triangular
// in topological order; it is solved level by level of the tree (all nodes of one depth at once,
// their ancestors being done), so no state is ever updated and nothing needs rolling back.
//
// gdn_verify_kernel: one 256-thread workgroup per (value-column block of 32, value head,
//   sequence): K of the head and the S_0 column block in LDS, the pseudo-values U of the block
//   in LDS (sized for 128 or 256 nodes); each thread owns (node, 16 columns) items. All
//   arithmetic fp32 (bf16 inputs widened).
// gdn_commit_kernel: the deferred commit. Once the accepted path is known the committed state
//   becomes the last accepted node's state, obtained by applying the path's updates to S_0 in
//   place.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace ta {

namespace {

constexpr int kGdnThreads = 256;
constexpr int kColBlock = 32;   // value columns per workgroup
constexpr int kItemCols = 16;   // columns per (node, half) item

__device__ inline float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Dot product of two bf16 rows of length DK held in LDS (16-byte aligned).
template <int DK>
__device__ inline float dot_lds(const uint16_t *x, const uint16_t *y) {
    float s = 0.f;
#pragma unroll 4
    for (int d = 0; d < DK; d += 8) {
        const uint4 a = *reinterpret_cast<const uint4 *>(x + d);
        const uint4 b = *reinterpret_cast<const uint4 *>(y + d);
        const uint32_t au[4] = {a.x, a.y, a.z, a.w}, bu[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s = fmaf(__uint_as_float(au[e] << 16), __uint_as_float(bu[e] << 16), s);
            s = fmaf(__uint_as_float(au[e] & 0xffff0000u), __uint_as_float(bu[e] & 0xffff0000u), s);
        }
    }
    return s;
}

// Entry d of a bf16 row held packed in registers (two entries per 32-bit word).
__device__ inline float unpack(const uint32_t *x, int d) {
    return __uint_as_float((d & 1) ? (x[d >> 1] & 0xffff0000u) : (x[d >> 1] << 16));
}

// Dot product of a packed register row (bf16, DK) with a bf16 row in LDS.
template <int DK>
__device__ inline float dot_reg_lds(const uint32_t *x, const uint16_t *y) {
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < DK; d += 8) {
        const uint4 b = *reinterpret_cast<const uint4 *>(y + d);
        const uint32_t bu[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s = fmaf(unpack(x, d + 2 * e), __uint_as_float(bu[e] << 16), s);
            s = fmaf(unpack(x, d + 2 * e + 1), __uint_as_float(bu[e] & 0xffff0000u), s);
        }
    }
    return s;
}

// Per-tree quantities by pointer jumping in LDS: depth (1 for a root-attached node) and the
// cumulative log-decay G over the node and its ancestors. Invalid parents count as -1.
struct TreeLds {
    int32_t par[TA_MAX_TREE];
    int32_t jmp[2][TA_MAX_TREE];
    int32_t dep[2][TA_MAX_TREE];
    float gs[2][TA_MAX_TREE];
    float beta[TA_MAX_TREE];
    int32_t max_depth;
};

__device__ inline int tree_levels(const int32_t *parent, const float *g, const float *beta,
                                  int64_t gstride, int T, TreeLds &s, int32_t *err) {
    const int tid = threadIdx.x;
    if (tid == 0) s.max_depth = 0;
    for (int i = tid; i < T; i += kGdnThreads) {
        int p = parent[i];
        if (p < -1 || p >= i) {
            if (err) atomicOr(err, (int32_t)TA_DEV_BAD_PARENT);
            p = -1;
        }
        s.par[i] = p;
        s.jmp[0][i] = p;
        s.dep[0][i] = 1;
        s.gs[0][i] = g[i * gstride];
        s.beta[i] = beta[i * gstride];
    }
    __syncthreads();
    int cur = 0;
    for (int span = 1; span < T; span <<= 1) {
        for (int i = tid; i < T; i += kGdnThreads) {
            const int j = s.jmp[cur][i];
            s.dep[cur ^ 1][i] = s.dep[cur][i] + (j >= 0 ? s.dep[cur][j] : 0);
            s.gs[cur ^ 1][i] = s.gs[cur][i] + (j >= 0 ? s.gs[cur][j] : 0.f);
            s.jmp[cur ^ 1][i] = j >= 0 ? s.jmp[cur][j] : -1;
        }
        __syncthreads();
        cur ^= 1;
    }
    for (int i = tid; i < T; i += kGdnThreads) atomicMax(&s.max_depth, s.dep[cur][i]);
    __syncthreads();
    return cur;
}

template <int DK, int TMAX>
__global__ __launch_bounds__(kGdnThreads) void gdn_verify_kernel(GdnArgs a) {
    __shared__ __align__(16) float S0b[DK * kColBlock];     // S_0 column block [DK][32]
    __shared__ __align__(16) float U[TMAX * kColBlock];     // pseudo-values [T][32]
    __shared__ __align__(16) uint16_t Ks[TMAX * DK];        // keys of the head [T][DK], bf16
    __shared__ TreeLds tr;
    const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int T = a.T, hk = h / (a.Hv / a.Hk);
    const int c0 = cb * kColBlock;
    const int lv = tree_levels(a.parent + (int64_t)b * T, a.g + (int64_t)b * T * a.Hv + h,
                               a.beta + (int64_t)b * T * a.Hv + h, a.Hv, T, tr, a.err);
    const int32_t *dep = tr.dep[lv];
    const float *G = tr.gs[lv];
    // K rows of this key head and the S_0 column block
    {
        const uint16_t *kg = static_cast<const uint16_t *>(a.k);
        for (int idx = tid; idx < T * (DK / 8); idx += kGdnThreads) {
            const int t = idx / (DK / 8), d8 = idx % (DK / 8);
            *reinterpret_cast<uint4 *>(Ks + t * DK + d8 * 8) = *reinterpret_cast<const uint4 *>(
                kg + (((int64_t)b * T + t) * a.Hk + hk) * DK + d8 * 8);
        }
        const float *s0 = a.S0 + ((int64_t)b * a.Hv + h) * DK * a.dv;
        for (int idx = tid; idx < DK * (kColBlock / 4); idx += kGdnThreads) {
            const int d = idx / (kColBlock / 4), c4 = idx % (kColBlock / 4);
            *reinterpret_cast<float4 *>(S0b + d * kColBlock + c4 * 4) =
                *reinterpret_cast<const float4 *>(s0 + (int64_t)d * a.dv + c0 + c4 * 4);
        }
    }
    __syncthreads();
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);
    // right-hand side: w_t = beta_t (v_t - e^{G_t} S_0^T k_t), into U
    for (int it = tid; it < 2 * T; it += kGdnThreads) {
        const int t = it >> 1, cc = (it & 1) * kItemCols;
        float acc[kItemCols];
#pragma unroll
        for (int c = 0; c < kItemCols; ++c) acc[c] = 0.f;
        for (int d = 0; d < DK; ++d) {
            const float kd = bf(Ks[t * DK + d]);
            const float4 *row = reinterpret_cast<const float4 *>(S0b + d * kColBlock + cc);
#pragma unroll
            for (int c4 = 0; c4 < kItemCols / 4; ++c4) {
                const float4 s = row[c4];
                acc[4 * c4 + 0] = fmaf(kd, s.x, acc[4 * c4 + 0]);
                acc[4 * c4 + 1] = fmaf(kd, s.y, acc[4 * c4 + 1]);
                acc[4 * c4 + 2] = fmaf(kd, s.z, acc[4 * c4 + 2]);
                acc[4 * c4 + 3] = fmaf(kd, s.w, acc[4 * c4 + 3]);
            }
        }
        const float eg = __expf(G[t]), bt = tr.beta[t];
        const uint16_t *vr = vg + (((int64_t)b * T + t) * a.Hv + h) * a.dv + c0 + cc;
#pragma unroll
        for (int c = 0; c < kItemCols; ++c) U[t * kColBlock + cc + c] = bt * (bf(vr[c]) - eg * acc[c]);
    }
    __syncthreads();
    // forward substitution, one tree level at a time: u_t -= b_t e^{G_t - G_j} (k_t . k_j) u_j
    // over the strict ancestors j (all of shallower levels, hence final)
    for (int level = 2; level <= tr.max_depth; ++level) {
        for (int it = tid; it < 2 * T; it += kGdnThreads) {
            const int t = it >> 1, cc = (it & 1) * kItemCols;
            if (dep[t] != level) continue;
            float u[kItemCols];
#pragma unroll
            for (int c = 0; c < kItemCols; ++c) u[c] = U[t * kColBlock + cc + c];
            const float bt = tr.beta[t], gt = G[t];
            for (int j = tr.par[t]; j >= 0; j = tr.par[j]) {
                const float x = bt * __expf(gt - G[j]) * dot_lds<DK>(Ks + t * DK, Ks + j * DK);
#pragma unroll
                for (int c = 0; c < kItemCols; ++c) u[c] = fmaf(-x, U[j * kColBlock + cc + c], u[c]);
            }
#pragma unroll
            for (int c = 0; c < kItemCols; ++c) U[t * kColBlock + cc + c] = u[c];
        }
        __syncthreads();
    }
    // output: o_t = scale (e^{G_t} S_0^T q_t + sum_{j ancestor or self} e^{G_t - G_j} (q_t . k_j) u_j)
    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    for (int it = tid; it < 2 * T; it += kGdnThreads) {
        const int t = it >> 1, cc = (it & 1) * kItemCols;
        uint32_t qp[DK / 2];  // q_t, bf16 packed in pairs
        const uint16_t *qr = qg + (((int64_t)b * T + t) * a.Hk + hk) * DK;
#pragma unroll
        for (int d = 0; d < DK; d += 8) {
            const uint4 w = *reinterpret_cast<const uint4 *>(qr + d);
            qp[d / 2] = w.x;
            qp[d / 2 + 1] = w.y;
            qp[d / 2 + 2] = w.z;
            qp[d / 2 + 3] = w.w;
        }
        float acc[kItemCols];
#pragma unroll
        for (int c = 0; c < kItemCols; ++c) acc[c] = 0.f;
#pragma unroll
        for (int d = 0; d < DK; ++d) {
            const float qd = unpack(qp, d);
            const float4 *row = reinterpret_cast<const float4 *>(S0b + d * kColBlock + cc);
#pragma unroll
            for (int c4 = 0; c4 < kItemCols / 4; ++c4) {
                const float4 s = row[c4];
                acc[4 * c4 + 0] = fmaf(qd, s.x, acc[4 * c4 + 0]);
                acc[4 * c4 + 1] = fmaf(qd, s.y, acc[4 * c4 + 1]);
                acc[4 * c4 + 2] = fmaf(qd, s.z, acc[4 * c4 + 2]);
                acc[4 * c4 + 3] = fmaf(qd, s.w, acc[4 * c4 + 3]);
            }
        }
        const float gt = G[t], eg = __expf(gt);
#pragma unroll
        for (int c = 0; c < kItemCols; ++c) acc[c] *= eg;
        for (int j = t; j >= 0; j = tr.par[j]) {
            const float y = __expf(gt - G[j]) * dot_reg_lds<DK>(qp, Ks + j * DK);
#pragma unroll
            for (int c = 0; c < kItemCols; ++c) acc[c] = fmaf(y, U[j * kColBlock + cc + c], acc[c]);
        }
        float *orow = a.o + (((int64_t)b * T + t) * a.Hv + h) * a.dv + c0 + cc;
#pragma unroll
        for (int c4 = 0; c4 < kItemCols / 4; ++c4)
            reinterpret_cast<float4 *>(orow)[c4] =
                make_float4(a.scale * acc[4 * c4], a.scale * acc[4 * c4 + 1],
                            a.scale * acc[4 * c4 + 2], a.scale * acc[4 * c4 + 3]);
    }
}

// Deferred commit: S <- the state after the updates of path[b][0 .. n-1] (root first), for one
// (32-column block, value head, sequence). Thread (d, c-group) owns S[d][4 c-group .. +3].
template <int DK>
__global__ __launch_bounds__(kGdnThreads) void gdn_commit_kernel(GdnCommitArgs a) {
    const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int hk = h / (a.Hv / a.Hk), c0 = cb * kColBlock;
    constexpr int kRowsPerPass = kGdnThreads / (kColBlock / 4);  // 32 rows of S per pass
    constexpr int kPasses = DK / kRowsPerPass;
    const int cg = tid % (kColBlock / 4), r0 = tid / (kColBlock / 4);
    __shared__ float kt[DK];
    __shared__ float part[kRowsPerPass][kColBlock];
    __shared__ float ktS[kColBlock];
    const int n = a.accept_len[b];
    if (n < 0 || n > a.T) {
        if (tid == 0 && a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_COMMIT);
        return;
    }
    float *Sg = a.S + ((int64_t)b * a.Hv + h) * DK * a.dv;
    float4 S[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        S[p] = *reinterpret_cast<const float4 *>(Sg + (int64_t)(r0 + p * kRowsPerPass) * a.dv + c0 +
                                                 4 * cg);
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);
    for (int s = 0; s < n; ++s) {
        const int t = a.path[(int64_t)b * a.T + s];
        if (t < 0 || t >= a.T) {
            if (tid == 0 && a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_COMMIT);
            break;  // uniform: every thread reads the same entry
        }
        for (int d = tid; d < DK; d += kGdnThreads)
            kt[d] = bf(kg[(((int64_t)b * a.T + t) * a.Hk + hk) * DK + d]);
        __syncthreads();
        // k^T S for this column block
        float4 acc = make_float4(0, 0, 0, 0);
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const float kd = kt[r0 + p * kRowsPerPass];
            acc.x = fmaf(kd, S[p].x, acc.x);
            acc.y = fmaf(kd, S[p].y, acc.y);
            acc.z = fmaf(kd, S[p].z, acc.z);
            acc.w = fmaf(kd, S[p].w, acc.w);
        }
        *reinterpret_cast<float4 *>(&part[r0][4 * cg]) = acc;
        __syncthreads();
        if (tid < kColBlock) {
            float sum = 0.f;
            for (int r = 0; r < kRowsPerPass; ++r) sum += part[r][tid];
            ktS[tid] = sum;
        }
        __syncthreads();
        const float al = __expf(a.g[((int64_t)b * a.T + t) * a.Hv + h]);
        const float bt = a.beta[((int64_t)b * a.T + t) * a.Hv + h];
        const uint16_t *vr = vg + (((int64_t)b * a.T + t) * a.Hv + h) * a.dv + c0 + 4 * cg;
        const float v0 = bf(vr[0]), v1 = bf(vr[1]), v2 = bf(vr[2]), v3 = bf(vr[3]);
        const float4 ks = *reinterpret_cast<const float4 *>(&ktS[4 * cg]);
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const float kd = kt[r0 + p * kRowsPerPass];
            // S = a (S - b k (k^T S)) + b k v^T
            S[p].x = al * (S[p].x - bt * kd * ks.x) + bt * kd * v0;
            S[p].y = al * (S[p].y - bt * kd * ks.y) + bt * kd * v1;
            S[p].z = al * (S[p].z - bt * kd * ks.z) + bt * kd * v2;
            S[p].w = al * (S[p].w - bt * kd * ks.w) + bt * kd * v3;
        }
        __syncthreads();  // kt / part / ktS are rewritten by the next step
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        *reinterpret_cast<float4 *>(Sg + (int64_t)(r0 + p * kRowsPerPass) * a.dv + c0 + 4 * cg) = S[p];
}

}  // namespace

hipError_t launch_gdn_verify(const GdnArgs &a, hipStream_t s) {
    // trees of up to 128 nodes take the smaller LDS footprint (two workgroups per CU)
    const dim3 grid(a.dv / kColBlock, a.Hv, a.B);
    if (a.dk == 128) {
        if (a.T <= 128) hipLaunchKernelGGL((gdn_verify_kernel<128, 128>), grid, dim3(kGdnThreads), 0, s, a);
        else hipLaunchKernelGGL((gdn_verify_kernel<128, 256>), grid, dim3(kGdnThreads), 0, s, a);
    } else {
        if (a.T <= 128) hipLaunchKernelGGL((gdn_verify_kernel<64, 128>), grid, dim3(kGdnThreads), 0, s, a);
        else hipLaunchKernelGGL((gdn_verify_kernel<64, 256>), grid, dim3(kGdnThreads), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gdn_commit(const GdnCommitArgs &a, hipStream_t s) {
    const dim3 grid(a.dv / kColBlock, a.Hv, a.B);
    if (a.dk == 128)
        hipLaunchKernelGGL(gdn_commit_kernel<128>, grid, dim3(kGdnThreads), 0, s, a);
    else
        hipLaunchKernelGGL(gdn_commit_kernel<64>, grid, dim3(kGdnThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ta
