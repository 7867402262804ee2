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
// gdn_verify_kernel: one workgroup per (value-column block, value head, sequence): 64 columns and
//   512 threads when that still gives every CU two workgroups' worth of columns (the tree work --
//   depths, ancestor tables, path coefficients -- is then done once per 64 columns, and the
//   grid fits the CUs in one round), else 32 columns and 256 threads. K S_0 and Q S_0 for all nodes run on bf16 MFMA with S_0 split into a high and a
//   low bf16 part (fp32 accumulation; the split leaves about 2^-16 of S_0's relative precision);
//   the key dot products of ancestor pairs use the two-term bf16 dot instruction, everything
//   else is fp32 VALU. K of the head and the pseudo-values U live in LDS (sized for 128 or 256
//   nodes); in the solve and the output each thread owns (node, 16 columns) items.
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

constexpr int kGdnThreads = 256;  // the commit kernel's workgroup
constexpr int kColBlock = 32;    // value columns per commit workgroup
constexpr int kItemCols = 16;    // columns per (node, column group) item

__device__ inline float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Dot product of a packed register row (bf16 pairs, DK entries) with a bf16 row in LDS, on the
// two-term bf16 dot instruction with fp32 accumulation.
template <int DK>
__device__ inline float dot_reg_lds(const uint32_t *x, const uint16_t *y) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
    for (int d = 0; d < DK; d += 8) {
        const uint4 b = *reinterpret_cast<const uint4 *>(y + d);
        const uint32_t bu[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            s[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[d / 2 + e]),
                                                   __builtin_bit_cast(bf16x2, bu[e]), s[e], false);
    }
    return (s[0] + s[1]) + (s[2] + s[3]);
}

template <int DK>
__device__ inline void load_row(uint32_t *x, const uint16_t *src) {
#pragma unroll
    for (int d = 0; d < DK; d += 8) {
        const uint4 w = *reinterpret_cast<const uint4 *>(src + d);
        x[d / 2] = w.x;
        x[d / 2 + 1] = w.y;
        x[d / 2 + 2] = w.z;
        x[d / 2 + 3] = w.w;
    }
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

// Thread i's node (T <= the workgroup's threads): its parent, log-decay and write strength.
struct NodeIn {
    int p;
    float g, beta;
};

__device__ inline NodeIn node_in(const int32_t *parent, const float *g, const float *beta,
                                 int64_t gstride, int T) {
    const int i = threadIdx.x;
    if (i >= T) return NodeIn{-1, 0.f, 0.f};
    return NodeIn{parent[i], g[i * gstride], beta[i * gstride]};
}

template <int NT>
__device__ inline int tree_levels(NodeIn in, int T, TreeLds &s, int32_t *err) {
    static_assert(TA_MAX_TREE <= NT, "one node per thread");
    const int tid = threadIdx.x;
    if (tid == 0) s.max_depth = 0;
    if (tid < T) {
        int p = in.p;
        if (p < -1 || p >= tid) {
            if (err) atomicOr(err, (int32_t)TA_DEV_BAD_PARENT);
            p = -1;
        }
        s.par[tid] = p;
        s.jmp[0][tid] = p;
        s.dep[0][tid] = 1;
        s.gs[0][tid] = in.g;
        s.beta[tid] = in.beta;
    }
    __syncthreads();
    int cur = 0;
    for (int span = 1; span < T; span <<= 1) {
        // done once every jump pointer has passed the root
        bool more = false;
        for (int i = tid; i < T; i += NT) more |= s.jmp[cur][i] >= 0;
        if (!__syncthreads_or(more)) break;
        for (int i = tid; i < T; i += NT) {
            const int j = s.jmp[cur][i];
            s.dep[cur ^ 1][i] = s.dep[cur][i] + (j >= 0 ? s.dep[cur][j] : 0);
            s.gs[cur ^ 1][i] = s.gs[cur][i] + (j >= 0 ? s.gs[cur][j] : 0.f);
            s.jmp[cur ^ 1][i] = j >= 0 ? s.jmp[cur][j] : -1;
        }
        __syncthreads();
        cur ^= 1;
    }
    // the tree's depth: a wavefront maximum, then one LDS atomic per wavefront
    int md = 0;
    for (int i = tid; i < T; i += NT) md = max(md, s.dep[cur][i]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) md = max(md, __shfl_xor(md, m));
    if ((tid & 63) == 0) atomicMax(&s.max_depth, md);
    __syncthreads();
    return cur;
}

template <int DK, int TMAX, int CB>
__global__ __launch_bounds__(CB * 8) void gdn_verify_kernel(GdnArgs a) {
    constexpr int NT = CB * 8;            // threads: 256 for 32 columns, 512 for 64
    constexpr int kGroups = CB / kItemCols;  // column groups of a node (solve and output items)
    // keys of the head [T][DK] bf16 and the S_0 column block split into bf16 high and low parts
    // (S0 = hi + lo to about 2^-16 relative), transposed [32][DK]; rows padded by 16 bytes so
    // that lanes reading different rows hit different banks
    constexpr int KS = DK + 8;
    __shared__ __align__(16) uint16_t Ks[TMAX * KS];
    __shared__ __align__(16) float U[TMAX * CB];    // pseudo-values [T][32]
    // coefficients along every node's root path, position m (0 = the node itself, m = its m-th
    // ancestor j_m): XA = b_t e^{G_t - G_j} (k_t . k_j) for m >= 1, YA = e^{G_t - G_j} (q_t . k_j);
    // positions past kAncCap are computed where they are used. XA / YA reuse the S_0 halves'
    // LDS, which is dead once the K S_0 / Q S_0 products are done.
    constexpr int kAncCap = TMAX <= 128 ? 16 : 8;
    constexpr int kS0Bytes = 2 * CB * KS * 2, kCoefBytes = 2 * TMAX * kAncCap * 4;
    __shared__ __align__(16) unsigned char s0buf[kS0Bytes > kCoefBytes ? kS0Bytes : kCoefBytes];
    uint16_t *S0hi = reinterpret_cast<uint16_t *>(s0buf);
    uint16_t *S0lo = S0hi + CB * KS;
    float *XA = reinterpret_cast<float *>(s0buf);
    float *YA = XA + TMAX * kAncCap;
    __shared__ int16_t anc[TMAX * kAncCap];  // j_m of every node, -1 past the root
    __shared__ TreeLds tr;
    const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, hf = lane >> 5;
    const int T = a.T, hk = h / (a.Hv / a.Hk);
    const int c0 = cb * CB;
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    // every load of a thread is issued before any LDS store, so their latencies overlap
    constexpr int KV = TMAX * (DK / 8) / NT;  // 16-byte key chunks per thread
    uint4 kc[KV];
#pragma unroll
    for (int r = 0; r < KV; ++r) {
        const int idx = tid + r * NT, t = min(idx / (DK / 8), T - 1);
        kc[r] = *reinterpret_cast<const uint4 *>(
            kg + (((int64_t)b * T + t) * a.Hk + hk) * DK + (idx % (DK / 8)) * 8);
    }
    // S_0 entries (d, c) and (d + 1, c) per thread and step, so that one 32-bit LDS store
    // takes both of their bf16 parts
    constexpr int SV = DK * CB / (2 * NT);
    const float *s0 = a.S0 + ((int64_t)b * a.Hv + h) * DK * a.dv;
    float sx[SV][2];
#pragma unroll
    for (int r = 0; r < SV; ++r) {
        const int idx = tid + r * NT, d = 2 * (idx / CB), c = idx % CB;
        sx[r][0] = s0[(int64_t)d * a.dv + c0 + c];
        sx[r][1] = s0[(int64_t)(d + 1) * a.dv + c0 + c];
    }
    const NodeIn nin = node_in(a.parent + (int64_t)b * T, a.g + (int64_t)b * T * a.Hv + h,
                               a.beta + (int64_t)b * T * a.Hv + h, a.Hv, T);
    // keys and S_0 halves into LDS (the loads above are all in flight by now)
#pragma unroll
    for (int r = 0; r < KV; ++r) {
        const int idx = tid + r * NT;
        if (idx / (DK / 8) < T)
            *reinterpret_cast<uint4 *>(Ks + (idx / (DK / 8)) * KS + (idx % (DK / 8)) * 8) = kc[r];
    }
#pragma unroll
    for (int r = 0; r < SV; ++r) {
        const int idx = tid + r * NT, d = 2 * (idx / CB), c = idx % CB;
        const __bf16 h0 = (__bf16)sx[r][0], h1 = (__bf16)sx[r][1];
        const __bf16 l0 = (__bf16)(sx[r][0] - (float)h0), l1 = (__bf16)(sx[r][1] - (float)h1);
        *reinterpret_cast<bf16x2 *>(S0hi + c * KS + d) = bf16x2{h0, h1};
        *reinterpret_cast<bf16x2 *>(S0lo + c * KS + d) = bf16x2{l0, l1};
    }
    const int lv = tree_levels<NT>(nin, T, tr, a.err);
    const int32_t *dep = tr.dep[lv];
    const float *G = tr.gs[lv];
    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);
    for (int t = tid; t < T; t += NT) {
        int j = t;
        for (int m = 0; m < kAncCap; ++m) {
            anc[t * kAncCap + m] = (int16_t)j;
            j = j >= 0 ? tr.par[j] : -1;
        }
    }
    __syncthreads();
    // K S_0 and Q S_0 on v_mfma_f32_32x32x16_bf16, one (32-node tile, 32-column tile) per
    // wavefront at a time: lane (l32, hf) supplies node row l32 (A) and value column col
    // (B) over k = 16 ks + 8 hf .. + 7; register r of the result is node 8 (r / 4) + 4 hf + r % 4
    constexpr int kColTiles = CB / 32;
    for (int pt = wave; pt < ((T + 31) / 32) * kColTiles; pt += NT / 64) {
        const int nt = pt / kColTiles, col = (pt % kColTiles) * 32 + l32;
        // rows past the tree read its last row; their results are dropped below
        const int row = min(nt * 32 + l32, T - 1);
        const uint16_t *qrow = qg + (((int64_t)b * T + row) * a.Hk + hk) * DK;
        bf16x8 aq[DK / 16], ak[DK / 16];
        float vv[16];
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks)
            aq[ks] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * ks + 8 * hf);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = min(nt * 32 + 8 * (r / 4) + 4 * hf + r % 4, T - 1);
            vv[r] = bf(vg[(((int64_t)b * T + t) * a.Hv + h) * a.dv + c0 + col]);
        }
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks)
            ak[ks] = *reinterpret_cast<const bf16x8 *>(Ks + row * KS + 16 * ks + 8 * hf);
        f32x16 accK, accQ;
#pragma unroll
        for (int r = 0; r < 16; ++r) accK[r] = accQ[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < DK / 16; ++ks) {
            const int d0 = 16 * ks + 8 * hf;
            const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(S0hi + col * KS + d0);
            const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(S0lo + col * KS + d0);
            accK = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[ks], bh, accK, 0, 0, 0);
            accK = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[ks], bl, accK, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[ks], bh, accQ, 0, 0, 0);
            accQ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[ks], bl, accQ, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = nt * 32 + 8 * (r / 4) + 4 * hf + r % 4;
            if (t < T) {
                const float eg = __expf(G[t]);
                // right-hand side w_t = beta_t (v_t - e^{G_t} S_0^T k_t), into U
                U[t * CB + col] = tr.beta[t] * (vv[r] - eg * accK[r]);
                // e^{G_t} S_0^T q_t goes to the output, which the last phase completes
                a.o[(((int64_t)b * T + t) * a.Hv + h) * a.dv + c0 + col] = eg * accQ[r];
            }
        }
    }
    __syncthreads();  // the S_0 halves are dead from here on: their LDS takes XA / YA
    // path coefficients: item (t, part) takes the positions part, part + kGroups, ... of t's
    // root path
    for (int it = tid; it < kGroups * T; it += NT) {
        const int t = it / kGroups, half = it % kGroups;
        if (half >= dep[t]) continue;
        uint32_t kp[DK / 2], qp[DK / 2];
        load_row<DK>(qp, qg + (((int64_t)b * T + t) * a.Hk + hk) * DK);
        load_row<DK>(kp, Ks + t * KS);
        const float bt = tr.beta[t], gt = G[t];
        for (int m = half; m < kAncCap; m += kGroups) {
            const int j = anc[t * kAncCap + m];
            if (j < 0) break;
            const float e = __expf(gt - G[j]);
            YA[t * kAncCap + m] = e * dot_reg_lds<DK>(qp, Ks + j * KS);
            if (m > 0) XA[t * kAncCap + m] = bt * e * dot_reg_lds<DK>(kp, Ks + j * KS);
        }
    }
    __syncthreads();
    // forward substitution, one tree level at a time: u_t -= b_t e^{G_t - G_j} (k_t . k_j) u_j
    // over the strict ancestors j (all of shallower levels, hence final)
    for (int level = 2; level <= tr.max_depth; ++level) {
        for (int it = tid; it < kGroups * T; it += NT) {
            const int t = it / kGroups, cc = (it % kGroups) * kItemCols;
            if (dep[t] != level) continue;
            float u[kItemCols];
#pragma unroll
            for (int c = 0; c < kItemCols; ++c) u[c] = U[t * CB + cc + c];
            // ancestors at path positions 1 .. nd from the tables, four at a time so that their
            // loads overlap; deeper ones (past the tables) one by one with the coefficient on the
            // spot
            const int nd = min(dep[t] - 1, kAncCap - 1);
            for (int m0 = 1; m0 <= nd; m0 += 4) {
                float x[4];
                float4 uj[4][kItemCols / 4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = m0 + i <= nd;
                    const int j = ok ? anc[t * kAncCap + m0 + i] : t;
                    x[i] = ok ? XA[t * kAncCap + m0 + i] : 0.f;
#pragma unroll
                    for (int c4 = 0; c4 < kItemCols / 4; ++c4)
                        uj[i][c4] = *reinterpret_cast<const float4 *>(U + j * CB + cc + 4 * c4);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int c4 = 0; c4 < kItemCols / 4; ++c4) {
                        u[4 * c4 + 0] = fmaf(-x[i], uj[i][c4].x, u[4 * c4 + 0]);
                        u[4 * c4 + 1] = fmaf(-x[i], uj[i][c4].y, u[4 * c4 + 1]);
                        u[4 * c4 + 2] = fmaf(-x[i], uj[i][c4].z, u[4 * c4 + 2]);
                        u[4 * c4 + 3] = fmaf(-x[i], uj[i][c4].w, u[4 * c4 + 3]);
                    }
            }
            if (dep[t] > kAncCap) {
                const float bt = tr.beta[t], gt = G[t];
                uint32_t kp[DK / 2];
                load_row<DK>(kp, Ks + t * KS);
                for (int j = tr.par[anc[t * kAncCap + kAncCap - 1]]; j >= 0; j = tr.par[j]) {
                    const float x = bt * __expf(gt - G[j]) * dot_reg_lds<DK>(kp, Ks + j * KS);
#pragma unroll
                    for (int c = 0; c < kItemCols; ++c)
                        u[c] = fmaf(-x, U[j * CB + cc + c], u[c]);
                }
            }
#pragma unroll
            for (int c = 0; c < kItemCols; ++c) U[t * CB + cc + c] = u[c];
        }
        __syncthreads();
    }
    // output: o_t = scale (e^{G_t} S_0^T q_t + sum_{j ancestor or self} e^{G_t - G_j} (q_t . k_j) u_j)
    for (int it = tid; it < kGroups * T; it += NT) {
        const int t = it / kGroups, cc = (it % kGroups) * kItemCols;
        float *orow = a.o + (((int64_t)b * T + t) * a.Hv + h) * a.dv + c0 + cc;
        float acc[kItemCols];
#pragma unroll
        for (int c4 = 0; c4 < kItemCols / 4; ++c4) {
            const float4 w = reinterpret_cast<const float4 *>(orow)[c4];
            acc[4 * c4] = w.x;
            acc[4 * c4 + 1] = w.y;
            acc[4 * c4 + 2] = w.z;
            acc[4 * c4 + 3] = w.w;
        }
        // path positions 0 .. nd from the tables, four at a time; deeper ones one by one
        const int nd = min(dep[t] - 1, kAncCap - 1);
        for (int m0 = 0; m0 <= nd; m0 += 4) {
            float y[4];
            float4 uj[4][kItemCols / 4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = m0 + i <= nd;
                const int j = ok ? anc[t * kAncCap + m0 + i] : t;
                y[i] = ok ? YA[t * kAncCap + m0 + i] : 0.f;
#pragma unroll
                for (int c4 = 0; c4 < kItemCols / 4; ++c4)
                    uj[i][c4] = *reinterpret_cast<const float4 *>(U + j * CB + cc + 4 * c4);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c4 = 0; c4 < kItemCols / 4; ++c4) {
                    acc[4 * c4 + 0] = fmaf(y[i], uj[i][c4].x, acc[4 * c4 + 0]);
                    acc[4 * c4 + 1] = fmaf(y[i], uj[i][c4].y, acc[4 * c4 + 1]);
                    acc[4 * c4 + 2] = fmaf(y[i], uj[i][c4].z, acc[4 * c4 + 2]);
                    acc[4 * c4 + 3] = fmaf(y[i], uj[i][c4].w, acc[4 * c4 + 3]);
                }
        }
        if (dep[t] > kAncCap) {
            const float gt = G[t];
            uint32_t qp[DK / 2];
            load_row<DK>(qp, qg + (((int64_t)b * T + t) * a.Hk + hk) * DK);
            for (int j = tr.par[anc[t * kAncCap + kAncCap - 1]]; j >= 0; j = tr.par[j]) {
                const float y = __expf(gt - G[j]) * dot_reg_lds<DK>(qp, Ks + j * KS);
#pragma unroll
                for (int c = 0; c < kItemCols; ++c) acc[c] = fmaf(y, U[j * CB + cc + c], acc[c]);
            }
        }
#pragma unroll
        for (int c4 = 0; c4 < kItemCols / 4; ++c4)
            reinterpret_cast<float4 *>(orow)[c4] =
                make_float4(a.scale * acc[4 * c4], a.scale * acc[4 * c4 + 1],
                            a.scale * acc[4 * c4 + 2], a.scale * acc[4 * c4 + 3]);
    }
}

// Deferred commit: S <- the state after the updates of path[b][0 .. n-1] (root first), for one
// (32-column block, value head, sequence). Thread (d, c-group) owns S[d][4 c-group .. +3]. The
// path is taken kCommitStage steps at a time: the steps' key rows, value columns, decays and
// betas are first staged in LDS together (one round trip to memory for all of them), then the
// updates run back to back with one barrier each.
constexpr int kCommitStage = 32;

template <int DK>
__global__ __launch_bounds__(kGdnThreads) void gdn_commit_kernel(GdnCommitArgs a) {
    const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int hk = h / (a.Hv / a.Hk), c0 = cb * kColBlock;
    constexpr int kRowsPerPass = kGdnThreads / (kColBlock / 4);  // 32 rows of S per pass
    constexpr int kPasses = DK / kRowsPerPass;
    constexpr int KCH = DK / 8;                                  // 16-byte chunks of a key row
    const int cg = tid % (kColBlock / 4), r0 = tid / (kColBlock / 4);
    __shared__ __attribute__((aligned(16))) uint16_t kst[kCommitStage][DK];
    __shared__ __attribute__((aligned(16))) float vst[kCommitStage][kColBlock];
    __shared__ float alst[kCommitStage], btst[kCommitStage];
    __shared__ int32_t tst[kCommitStage];
    __shared__ int32_t n_ok;
    // per-wavefront k^T S partial sums, double-buffered so that one barrier per step suffices
    constexpr int kWaves = kGdnThreads / 64;
    __shared__ __attribute__((aligned(16))) float part[2][kWaves][kColBlock];
    // the accepted length, the state and the first path entries are loaded together
    const int n = a.accept_len[b];
    float *Sg = a.S + ((int64_t)b * a.Hv + h) * DK * a.dv;
    float4 S[kPasses];
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        S[p] = *reinterpret_cast<const float4 *>(Sg + (int64_t)(r0 + p * kRowsPerPass) * a.dv + c0 +
                                                 4 * cg);
    const int t_first = tid < min(kCommitStage, a.T) ? a.path[(int64_t)b * a.T + tid] : 0;
    if (n < 0 || n > a.T) {
        if (tid == 0 && a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_COMMIT);
        return;
    }
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);
    int step = 0;
    for (int s0 = 0; s0 < n; s0 += kCommitStage) {
        const int m = min(kCommitStage, n - s0);
        if (tid == 0) n_ok = m;
        __syncthreads();  // n_ok set; the previous chunk's staged operands are no longer read
        if (tid < m) {
            const int t = s0 == 0 ? t_first : a.path[(int64_t)b * a.T + s0 + tid];
            const bool ok = t >= 0 && t < a.T;
            if (!ok) atomicMin(&n_ok, tid);
            tst[tid] = ok ? t : 0;
        }
        __syncthreads();
        const int mg = n_ok;  // the chunk's steps before its first invalid entry
        for (int e = tid; e < mg * KCH; e += kGdnThreads) {
            const int st = e / KCH, c = e % KCH;
            *reinterpret_cast<uint4 *>(&kst[st][8 * c]) = *reinterpret_cast<const uint4 *>(
                kg + (((int64_t)b * a.T + tst[st]) * a.Hk + hk) * DK + 8 * c);
        }
        for (int e = tid; e < mg * (kColBlock / 4); e += kGdnThreads) {
            const int st = e / (kColBlock / 4), c = e % (kColBlock / 4);
            const uint2 w = *reinterpret_cast<const uint2 *>(
                vg + (((int64_t)b * a.T + tst[st]) * a.Hv + h) * a.dv + c0 + 4 * c);
            *reinterpret_cast<float4 *>(&vst[st][4 * c]) =
                make_float4(bf((uint16_t)w.x), bf((uint16_t)(w.x >> 16)), bf((uint16_t)w.y),
                            bf((uint16_t)(w.y >> 16)));
        }
        if (tid < mg) {
            const int64_t gi = ((int64_t)b * a.T + tst[tid]) * a.Hv + h;
            alst[tid] = __expf(a.g[gi]);
            btst[tid] = a.beta[gi];
        }
        __syncthreads();
        for (int st = 0; st < mg; ++st, ++step) {
            float(*pt)[kColBlock] = part[step & 1];
            float kd[kPasses];
#pragma unroll
            for (int p = 0; p < kPasses; ++p) kd[p] = bf(kst[st][r0 + p * kRowsPerPass]);
            // k^T S for this column block
            float4 acc = make_float4(0, 0, 0, 0);
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                acc.x = fmaf(kd[p], S[p].x, acc.x);
                acc.y = fmaf(kd[p], S[p].y, acc.y);
                acc.z = fmaf(kd[p], S[p].z, acc.z);
                acc.w = fmaf(kd[p], S[p].w, acc.w);
            }
            // over the wavefront's 8 row groups (lanes cg, cg + 8, ..., cg + 56), then over the
            // wavefronts
#pragma unroll
            for (int o = 8; o < 64; o <<= 1) {
                acc.x += __shfl_xor(acc.x, o);
                acc.y += __shfl_xor(acc.y, o);
                acc.z += __shfl_xor(acc.z, o);
                acc.w += __shfl_xor(acc.w, o);
            }
            if ((tid & 63) < kColBlock / 4) *reinterpret_cast<float4 *>(&pt[tid >> 6][4 * cg]) = acc;
            __syncthreads();
            float4 ks = make_float4(0, 0, 0, 0);
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float4 x = *reinterpret_cast<const float4 *>(&pt[w][4 * cg]);
                ks.x += x.x;
                ks.y += x.y;
                ks.z += x.z;
                ks.w += x.w;
            }
            const float al = alst[st], bt = btst[st];
            const float4 v = *reinterpret_cast<const float4 *>(&vst[st][4 * cg]);
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                // S = a (S - b k (k^T S)) + b k v^T
                S[p].x = al * (S[p].x - bt * kd[p] * ks.x) + bt * kd[p] * v.x;
                S[p].y = al * (S[p].y - bt * kd[p] * ks.y) + bt * kd[p] * v.y;
                S[p].z = al * (S[p].z - bt * kd[p] * ks.z) + bt * kd[p] * v.z;
                S[p].w = al * (S[p].w - bt * kd[p] * ks.w) + bt * kd[p] * v.w;
            }
        }
        if (mg < m) {
            if (tid == 0 && a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_COMMIT);
            break;  // uniform: every thread read the same n_ok
        }
    }
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
        *reinterpret_cast<float4 *>(Sg + (int64_t)(r0 + p * kRowsPerPass) * a.dv + c0 + 4 * cg) = S[p];
}

}  // namespace

hipError_t launch_gdn_verify(const GdnArgs &a, int cus, hipStream_t s) {
    // 64-column workgroups (one per CU at most; trees of up to 128 nodes) when 32-column ones
    // would need two rounds of the CUs or more; otherwise 32 columns, trees of up to 128 nodes
    // taking the smaller LDS footprint (two workgroups per CU)
    const bool wide = a.T <= 128 && a.dv % 64 == 0 &&
                      (int64_t)a.B * a.Hv * (a.dv / 32) >= 2 * (int64_t)cus;
#define TA_GDN(DK, TM, CBW) \
    hipLaunchKernelGGL((gdn_verify_kernel<DK, TM, CBW>), dim3(a.dv / CBW, a.Hv, a.B), dim3(CBW * 8), 0, s, a)
    if (a.dk == 128) {
        if (wide) TA_GDN(128, 128, 64);
        else if (a.T <= 128) TA_GDN(128, 128, 32);
        else TA_GDN(128, 256, 32);
    } else {
        if (wide) TA_GDN(64, 128, 64);
        else if (a.T <= 128) TA_GDN(64, 128, 32);
        else TA_GDN(64, 256, 32);
    }
#undef TA_GDN
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
