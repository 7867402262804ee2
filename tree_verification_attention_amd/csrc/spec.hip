// Tree speculative sampling on gfx950 (textbook page, "Faster decoding", section on modified
// rejection sampling keeping the target distribution).
//
// At one position a candidate x drawn from the candidate distribution q is accepted with
// probability min(1, p(x) / q(x)); a rejection emits a token from the residual [p - q]_+ / Z. On a
// tree, the children of a position are candidates drawn independently from that position's q and
// are tried in index order; after a rejection the residual takes the place of p for the next
// child; with every child rejected the correction token comes from the last residual, and an
// accepted node without children ends the path with a bonus token from its row's p.
//
// Unnormalised form used here: with R_1 = p, N_1 = 1, C_0 = 0 and C_k = C_{k-1} + N_k, the
// residual after k rejections is r_{k+1} = R_{k+1} / N_{k+1} with R_{k+1} = [p - C_k q]_+ (since
// [[a]_+ - b]_+ = [a - b]_+ for b >= 0) and N_{k+1} = sum_v R_{k+1}(v). Trial k accepts x iff
// N_{k+1} == 0 (no rejection possible) or u * N_k * q(x) < R_k(x), which is u < min(1, r_k/q) for
// q(x) > 0. Every sum runs in fp64 over the fp32 inputs.
//
// spec_mass_kernel (data-parallel, HBM-bound): per (row, 4096-entry chunk), the chunk's sum of
//   [p - q]_+ when the row's position has children (N_2's parts: a first rejection there needs
//   it), else of p (the bonus token's weights).
// spec_walk_kernel: one workgroup per sequence. The per-node values p(x), q(x) are gathered up
//   front, so the walk itself reads LDS only; a second trial at one position needs N_{k+1} for
//   k >= 2, which the workgroup computes with a pass over that row; the final token is located
//   chunk by chunk from the chunk sums, then inside its chunk by a block prefix sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace ta {

namespace {

constexpr int kMassThreads = 256;
constexpr int kWalkThreads = 1024;
constexpr int kChunk = 4096;              // entries per chunk (1024 float4)
constexpr int kChunkVec = kChunk / 4;

__device__ inline double entry(float p, float q, double C, bool use_q) {
    // R(v) = [p - C q]_+, or p itself for the bonus weights
    return use_q ? fmax(0.0, (double)p - C * (double)q) : (double)p;
}

// Sum of R over a float4 pair.
__device__ inline double entry4(float4 p, float4 q, double C, bool use_q) {
    return entry(p.x, q.x, C, use_q) + entry(p.y, q.y, C, use_q) + entry(p.z, q.z, C, use_q) +
           entry(p.w, q.w, C, use_q);
}

__device__ inline double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// Row r of sequence b is position r - 1; does that position have a child? (invalid parents count
// as -1, as everywhere else)
__device__ inline bool position_has_child(const int32_t *parent, int T, int pos) {
    bool kid = false;
    for (int i = threadIdx.x; i < T; i += blockDim.x) {
        int pa = parent[i];
        if (pa < -1 || pa >= i) pa = -1;
        kid |= pa == pos;
    }
    return __syncthreads_or(kid);
}

__global__ __launch_bounds__(kMassThreads) void spec_mass_kernel(const float *p, const float *q,
                                                                 int64_t row_stride, int T, int V,
                                                                 int nch, const int32_t *parent,
                                                                 double *sums) {
    const int chunk = blockIdx.x;
    const int row_id = blockIdx.y;  // b * (T + 1) + row
    const int b = row_id / (T + 1), row = row_id % (T + 1);
    const bool use_q = position_has_child(parent + (int64_t)b * T, T, row - 1);
    const float *pr = p + (int64_t)row_id * row_stride;
    const float *qr = q + (int64_t)row_id * row_stride;
    const int nvec = V / 4;
    const int v0 = chunk * kChunkVec + threadIdx.x;
    float4 pv[4], qv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int v = v0 + k * kMassThreads;
        pv[k] = v < nvec ? reinterpret_cast<const float4 *>(pr)[v] : make_float4(0, 0, 0, 0);
        qv[k] = use_q && v < nvec ? reinterpret_cast<const float4 *>(qr)[v]
                                  : make_float4(0, 0, 0, 0);
    }
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) s += entry4(pv[k], qv[k], 1.0, use_q);
    if (chunk == nch - 1)
        for (int e = nvec * 4 + threadIdx.x; e < V; e += kMassThreads)
            s += entry(pr[e], use_q ? qr[e] : 0.f, 1.0, use_q);
    s = wave_sum(s);
    __shared__ double ws[kMassThreads / 64];
    if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = ws[0];
        for (int w = 1; w < kMassThreads / 64; ++w) t += ws[w];
        sums[(int64_t)row_id * nch + chunk] = t;
    }
}

struct WalkShared {
    int32_t par[TA_MAX_TREE];
    int32_t first_child[TA_MAX_TREE + 1];
    int32_t next_sib[TA_MAX_TREE];
    float pv[TA_MAX_TREE];             // p(x) and q(x) of every node's draft token at its row
    float qv[TA_MAX_TREE];
    double n2[TA_MAX_TREE + 1];        // N_2 of every row with children
    double cs[TA_MAX_VOCAB / kChunk];  // chunk sums of the residual of the last row pass
    double red[kWalkThreads / 64];
    int32_t path[TA_MAX_TREE];
    // walk state (written by thread 0)
    int32_t pos, child, k, n_path, have_pass, done, bonus, found;
    double Cprev, Nk, pass_C, pass_N, theta, base;
    int32_t pass_row, chunk_hit;
};

// Sum of R over chunk ch of one row, by one wavefront (result in every lane).
__device__ inline double chunk_sum_wave(const float *pr, const float *qr, double C, bool use_q,
                                        int ch, int nch, int V) {
    const int lane = threadIdx.x & 63;
    const int nvec = V / 4;
    double s = 0.0;
#pragma unroll 4
    for (int k = 0; k < kChunkVec / 64; ++k) {
        const int v = ch * kChunkVec + k * 64 + lane;
        if (v < nvec)
            s += entry4(reinterpret_cast<const float4 *>(pr)[v],
                        use_q ? reinterpret_cast<const float4 *>(qr)[v] : make_float4(0, 0, 0, 0),
                        C, use_q);
    }
    if (ch == nch - 1)
        for (int e = nvec * 4 + lane; e < V; e += 64) s += entry(pr[e], use_q ? qr[e] : 0.f, C, use_q);
    return wave_sum(s);
}

__global__ __launch_bounds__(kWalkThreads) void spec_walk_kernel(
    const float *p, const float *q, int64_t row_stride, int T, int V, int nch,
    const int32_t *draft, const int32_t *parent, const double *u_accept, const double *u_sample,
    const double *sums, int32_t *accept_len, int32_t *path, int32_t *next_token, int32_t *err) {
    __shared__ WalkShared sh;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row0 = (int64_t)b * (T + 1);
    for (int r = tid; r <= T; r += kWalkThreads) sh.first_child[r] = INT32_MAX;
    if (tid < T) {
        int pa = parent[(int64_t)b * T + tid];
        if (pa < -1 || pa >= tid) {
            if (err) atomicOr(err, (int32_t)TA_DEV_BAD_PARENT);
            pa = -1;
        }
        sh.par[tid] = pa;
    }
    __syncthreads();
    if (tid < T) {
        const int pa = sh.par[tid];
        atomicMin(&sh.first_child[pa + 1], tid);
        int nx = -1;
        for (int j = tid + 1; j < T; ++j)
            if (sh.par[j] == pa) {
                nx = j;
                break;
            }
        sh.next_sib[tid] = nx;
        // p(x) and q(x) of the node's draft token, at its parent's row
        const int x = draft[(int64_t)b * T + tid];
        const int64_t ro = (row0 + pa + 1) * row_stride;
        if (x >= 0 && x < V) {
            sh.pv[tid] = p[ro + x];
            sh.qv[tid] = q[ro + x];
        } else {
            // a token outside the vocabulary has no target mass: it is always rejected
            if (err) atomicOr(err, (int32_t)TA_DEV_BAD_TOKEN);
            sh.pv[tid] = 0.f;
            sh.qv[tid] = 1.f;
        }
    }
    __syncthreads();
    if (tid <= T) {
        const bool has_child = sh.first_child[tid] != INT32_MAX;
        if (!has_child) sh.first_child[tid] = -1;
        double n = 0.0;  // N_2 of the row, summed over its chunks in order
        if (has_child) {
            const double *sr = sums + (row0 + tid) * nch;
            for (int c = 0; c < nch; ++c) n += sr[c];
        }
        sh.n2[tid] = n;
    }
    if (tid == 0) {
        sh.pos = -1;
        sh.child = -2;
        sh.n_path = 0;
        sh.have_pass = 0;
        sh.done = 0;
    }
    __syncthreads();
    // -------- the walk: thread 0 advances it; the block makes the row passes it asks for -------
    for (;;) {
        if (tid == 0) {
            for (;;) {
                const int row = sh.pos + 1;
                if (sh.child == -2) {  // entering a position
                    sh.child = sh.first_child[row];
                    sh.k = 1;
                    sh.Cprev = 0.0;
                    sh.Nk = 1.0;
                    sh.have_pass = 0;
                }
                const int c = sh.child;
                if (c < 0) {  // no children: bonus token from this row's p
                    sh.bonus = 1;
                    sh.done = 1;
                    break;
                }
                double n_next;
                if (sh.k == 1) {
                    n_next = sh.n2[row];
                } else if (sh.have_pass) {
                    n_next = sh.pass_N;
                } else {  // N_{k+1} = sum [p - C_k q]_+ : ask the block for a pass over the row
                    sh.pass_row = row;
                    sh.pass_C = sh.Cprev + sh.Nk;
                    break;
                }
                const double R = fmax(0.0, (double)sh.pv[c] - sh.Cprev * (double)sh.qv[c]);
                const bool accept =
                    n_next == 0.0 || u_accept[(int64_t)b * T + c] * sh.Nk * (double)sh.qv[c] < R;
                if (accept) {
                    sh.path[sh.n_path++] = c;
                    sh.pos = c;
                    sh.child = -2;
                    continue;
                }
                sh.Cprev += sh.Nk;
                sh.Nk = n_next;
                sh.k += 1;
                sh.have_pass = 0;
                sh.child = sh.next_sib[c];
                if (sh.child < 0) {  // every child rejected: correction from R_k = [p - Cprev q]_+
                    sh.bonus = 0;
                    sh.done = 1;
                    break;
                }
            }
        }
        __syncthreads();
        if (sh.done) break;
        // row pass: chunk sums of [p - pass_C q]_+ into cs, their total into pass_N
        {
            const int64_t ro = (row0 + sh.pass_row) * row_stride;
            const double C = sh.pass_C;
            for (int ch = wave; ch < nch; ch += kWalkThreads / 64) {
                const double s = chunk_sum_wave(p + ro, q + ro, C, true, ch, nch, V);
                if (lane == 0) sh.cs[ch] = s;
            }
            __syncthreads();
            if (tid == 0) {
                double n = 0.0;
                for (int c = 0; c < nch; ++c) n += sh.cs[c];
                sh.pass_N = n;
                sh.have_pass = 1;
            }
            __syncthreads();
        }
    }
    // -------- the emitted token --------
    const int row = sh.pos + 1;
    const int64_t ro = (row0 + row) * row_stride;
    const bool use_q = !sh.bonus;
    const double C = sh.Cprev;
    // chunk sums of the final weights: the mass kernel's (bonus: p; correction after one trial:
    // [p - q]_+), else the last row pass's
    const bool from_pass = !sh.bonus && sh.k > 2;
    if (!from_pass)
        for (int c = tid; c < nch; c += kWalkThreads) sh.cs[c] = sums[(row0 + row) * nch + c];
    __syncthreads();
    if (tid == 0) {
        double w = 0.0;
        for (int c = 0; c < nch; ++c) w += sh.cs[c];
        sh.theta = u_sample[b] * w;
        // the first chunk whose running sum passes theta
        double cum = 0.0;
        int hit = -1, last_pos = -1;
        for (int c = 0; c < nch; ++c) {
            if (sh.cs[c] > 0.0) last_pos = c;
            if (hit < 0 && cum + sh.cs[c] > sh.theta) {
                hit = c;
                sh.base = cum;
            }
            cum += sh.cs[c];
        }
        if (hit < 0) {  // rounding left theta past the total: the last chunk with mass
            hit = last_pos < 0 ? 0 : last_pos;
            sh.base = -INFINITY;  // no entry passes: take the chunk's last positive entry
        }
        sh.chunk_hit = hit;
        sh.found = INT32_MAX;
    }
    __syncthreads();
    {
        const int e0 = sh.chunk_hit * kChunk + 4 * tid;  // this thread's 4 entries
        double w[4], t = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + j;
            w[j] = e < V ? entry(p[ro + e], use_q ? q[ro + e] : 0.f, C, use_q) : 0.0;
            t += w[j];
        }
        // block exclusive prefix of the per-thread totals
        double incl = t;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const double o = __shfl_up(incl, m);
            if (lane >= m) incl += o;
        }
        if (lane == 63) sh.red[wave] = incl;
        __syncthreads();
        double before = 0.0;
        for (int w2 = 0; w2 < wave; ++w2) before += sh.red[w2];
        double run = sh.base + before + incl - t;
        int hit = INT32_MAX, lastp = -1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            run += w[j];
            if (hit == INT32_MAX && run > sh.theta) hit = e0 + j;
            if (w[j] > 0.0) lastp = e0 + j;
        }
        // smallest passing index; failing that (rounding), the chunk's last entry with weight
        int key = hit;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) key = min(key, __shfl_xor(key, m));
        int lkey = lastp;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) lkey = max(lkey, __shfl_xor(lkey, m));
        __syncthreads();
        __shared__ int s_min[kWalkThreads / 64], s_last[kWalkThreads / 64];
        if (lane == 0) {
            s_min[wave] = key;
            s_last[wave] = lkey;
        }
        __syncthreads();
        if (tid == 0) {
            int k2 = INT32_MAX, l2 = -1;
            for (int w2 = 0; w2 < kWalkThreads / 64; ++w2) {
                k2 = min(k2, s_min[w2]);
                l2 = max(l2, s_last[w2]);
            }
            next_token[b] = k2 != INT32_MAX ? k2 : (l2 >= 0 ? l2 : 0);
            accept_len[b] = sh.n_path;
        }
    }
    for (int j = tid; j < T; j += kWalkThreads) path[(int64_t)b * T + j] = j < sh.n_path ? sh.path[j] : -1;
}

}  // namespace

int spec_sample_chunks(int V) { return (V + kChunk - 1) / kChunk; }

hipError_t launch_spec_sample(const SpecArgs &a, hipStream_t s) {
    const int nch = spec_sample_chunks(a.V);
    hipLaunchKernelGGL(spec_mass_kernel, dim3(nch, a.B * (a.T + 1)), dim3(kMassThreads), 0, s, a.p,
                       a.q, a.row_stride, a.T, a.V, nch, a.parent, a.sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(spec_walk_kernel, dim3(a.B), dim3(kWalkThreads), 0, s, a.p, a.q,
                       a.row_stride, a.T, a.V, nch, a.draft, a.parent, a.u_accept, a.u_sample,
                       a.sums, a.accept_len, a.path, a.next_token, a.err);
    return hipGetLastError();
}

}  // namespace ta
