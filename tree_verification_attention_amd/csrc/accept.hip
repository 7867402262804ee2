// Greedy tree acceptance and accepted-path KV commit on gfx950: the two data-parallel steps that
// follow the verify step's attention.
//
// Greedy verification (textbook page, "Faster decoding", greedy verification contract): the
// target's greedy token at a position is the argmax of its logits; on a draft tree a node is
// accepted when its draft token equals the greedy token of its parent's row (the root row for a
// root-attached node) and its parent is accepted; the deepest accepted node ends the committed
// path, and the greedy token of its row is emitted as the correction token.
//
// argmax_kernel: one workgroup per logits row, 16-byte loads (vocabularies of 1e5+ entries make
// this the HBM-bound part); each thread scans its entries in increasing index order keeping the
// first maximum, and the partial winners merge by (larger value, then smaller index). NaN never
// wins; a row of NaN only gives 0.
// accept_kernel: one wavefront per sequence walks the tree in topological order (T <= 256).
//
// Commit (same page, reserve / execute / commit: only the accepted prefix's target KV is
// committed): commit_kernel copies the path's tree K/V rows to cache positions L, L + 1, ... of
// the sequence (contiguous or paged); lens_kernel then advances the lengths. A commit that would
// pass the cache capacity writes nothing and keeps the length.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace ta {

namespace {

constexpr int kArgmaxThreads = 512;

struct Best {
    float v;
    int i;  // INT32_MAX: nothing seen but NaN
};

__device__ inline Best better(Best a, Best b) {
    if (a.i == INT32_MAX) return b;
    if (b.i == INT32_MAX) return a;
    if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
    return a;
}

__device__ inline void take(Best &best, float v, int i) {
    // visited in increasing index order: strict > keeps the first maximum; NaN never compares
    if (v == v && (best.i == INT32_MAX || v > best.v)) {
        best.v = v;
        best.i = i;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(const void *logits, int64_t row_stride,
                                                                int V, int32_t *greedy) {
    constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
    const int64_t row = blockIdx.x;
    const char *base = static_cast<const char *>(logits) + row * row_stride * (BF16 ? 2 : 4);
    const int nvec = V / EPV;
    Best best{0.f, INT32_MAX};
    auto scan = [&](uint4 w, int i0) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
        if (BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                take(best, __uint_as_float(u[k] << 16), i0 + 2 * k);
                take(best, __uint_as_float(u[k] & 0xffff0000u), i0 + 2 * k + 1);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) take(best, __uint_as_float(u[k]), i0 + k);
        }
    };
    const uint4 *vp = reinterpret_cast<const uint4 *>(base);
    int v = threadIdx.x;
    // four loads in flight per thread
    for (; v + 3 * kArgmaxThreads < nvec; v += 4 * kArgmaxThreads) {
        const uint4 w0 = vp[v], w1 = vp[v + kArgmaxThreads], w2 = vp[v + 2 * kArgmaxThreads],
                    w3 = vp[v + 3 * kArgmaxThreads];
        scan(w0, v * EPV);
        scan(w1, (v + kArgmaxThreads) * EPV);
        scan(w2, (v + 2 * kArgmaxThreads) * EPV);
        scan(w3, (v + 3 * kArgmaxThreads) * EPV);
    }
    for (; v < nvec; v += kArgmaxThreads) scan(vp[v], v * EPV);
    // the entries past the last full vector
    for (int i = nvec * EPV + threadIdx.x; i < V; i += kArgmaxThreads) {
        float x;
        if (BF16) x = __uint_as_float((uint32_t) reinterpret_cast<const uint16_t *>(base)[i] << 16);
        else x = reinterpret_cast<const float *>(base)[i];
        take(best, x, i);
    }
    // merge: wavefront butterflies, then the wavefronts through LDS
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Best o{__shfl_xor(best.v, m), __shfl_xor(best.i, m)};
        best = better(best, o);
    }
    __shared__ float sv[kArgmaxThreads / 64];
    __shared__ int si[kArgmaxThreads / 64];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sv[wave] = best.v;
        si[wave] = best.i;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        Best r{sv[0], si[0]};
        for (int w = 1; w < kArgmaxThreads / 64; ++w) r = better(r, Best{sv[w], si[w]});
        greedy[row] = r.i == INT32_MAX ? 0 : r.i;
    }
}

// One wavefront per sequence; lane 0 walks the nodes in order, the lanes then fill the path.
__global__ __launch_bounds__(64) void accept_kernel(const int32_t *greedy, const int32_t *draft,
                                                    const int32_t *parent, int T, int32_t *accept_len,
                                                    int32_t *path, int32_t *next_token, int32_t *err) {
    __shared__ int32_t par[TA_MAX_TREE], depth[TA_MAX_TREE];
    __shared__ int32_t chain_len, last;
    const int b = blockIdx.x, lane = threadIdx.x;
    const int32_t *g = greedy + (int64_t)b * (T + 1);
    for (int i = lane; i < T; i += 64) {
        int p = parent[(int64_t)b * T + i];
        if (p < -1 || p >= i) {
            if (err) atomicOr(err, (int32_t)TA_DEV_BAD_PARENT);
            p = -1;
        }
        par[i] = p;
    }
    __syncthreads();
    if (lane == 0) {
        int best = -1;
        for (int i = 0; i < T; ++i) {
            const int p = par[i];
            const bool ok = draft[(int64_t)b * T + i] == g[p + 1] && (p < 0 || depth[p] > 0);
            depth[i] = ok ? (p < 0 ? 1 : depth[p] + 1) : 0;
            if (ok && (best < 0 || depth[i] > depth[best])) best = i;
        }
        chain_len = best < 0 ? 0 : depth[best];
        last = best;
        accept_len[b] = chain_len;
        next_token[b] = g[best + 1];
    }
    __syncthreads();
    const int n = chain_len;
    int32_t *out = path + (int64_t)b * T;
    for (int k = n + lane; k < T; k += 64) out[k] = -1;
    if (lane == 0) {
        int j = last;
        for (int k = n - 1; k >= 0; --k) {
            out[k] = j;
            j = par[j];
        }
    }
}

// Block (slot j, kv-head g, sequence b): copies tree K/V row path[b][j] to cache position
// seq_lens[b] + j, 16 bytes per thread.
__global__ __launch_bounds__(64) void commit_kernel(CommitArgs c) {
    const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int n = c.accept_len[b];
    const int L = c.seq_lens[b];
    if (j >= n) return;
    if (L < 0 || L > c.capacity) {
        if (c.err && threadIdx.x == 0) atomicOr(c.err, (int32_t)TA_DEV_BAD_LEN);
        return;
    }
    if (n > c.T || L + n > c.capacity) {
        if (c.err && threadIdx.x == 0 && j == 0) atomicOr(c.err, (int32_t)TA_DEV_BAD_COMMIT);
        return;
    }
    const int node = c.path[(int64_t)b * c.T + j];
    if (node < 0 || node >= c.T) {
        if (c.err && threadIdx.x == 0) atomicOr(c.err, (int32_t)TA_DEV_BAD_COMMIT);
        return;
    }
    const int pos = L + j;
    int64_t dst;
    if (c.block_table) {
        const int pg = c.block_table[(int64_t)b * c.max_blocks + (pos >> c.page_shift)];
        if ((unsigned)pg >= (unsigned)c.num_pages) {
            if (c.err && threadIdx.x == 0) atomicOr(c.err, (int32_t)TA_DEV_BAD_PAGE);
            return;
        }
        dst = pg * c.kv_s0 + (pos & c.page_mask) * c.kv_s1 + g * c.kv_s2;
    } else {
        dst = b * c.kv_s0 + (int64_t)pos * c.kv_s1 + g * c.kv_s2;
    }
    const int64_t src = b * c.kt_sb + (int64_t)node * c.kt_st + g * c.kt_sh;
    const int chunks = c.row_bytes / 16;
    for (int t = threadIdx.x; t < 2 * chunks; t += 64) {
        const bool v = t >= chunks;
        const int q = v ? t - chunks : t;
        const char *s = static_cast<const char *>(v ? c.vt : c.kt) + src * c.es + 16 * q;
        char *d = static_cast<char *>(v ? c.vc : c.kc) + dst * c.es + 16 * q;
        *reinterpret_cast<uint4 *>(d) = *reinterpret_cast<const uint4 *>(s);
    }
}

__global__ void lens_kernel(const int32_t *seq_lens, const int32_t *accept_len, int B, int T,
                            int capacity, int32_t *new_lens) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int L = seq_lens[b], n = accept_len[b];
    const bool ok = L >= 0 && L <= capacity && n >= 0 && n <= T && L + n <= capacity;
    new_lens[b] = ok ? L + n : L;
}

}  // namespace

hipError_t launch_greedy_accept(const void *logits, bool bf16, int64_t row_stride, int B, int T,
                                int V, const int32_t *draft, const int32_t *parent, int32_t *greedy,
                                int32_t *accept_len, int32_t *path, int32_t *next_token,
                                int32_t *err, hipStream_t s) {
    const unsigned rows = (unsigned)B * (unsigned)(T + 1);
    if (bf16)
        hipLaunchKernelGGL(argmax_kernel<true>, dim3(rows), dim3(kArgmaxThreads), 0, s, logits,
                           row_stride, V, greedy);
    else
        hipLaunchKernelGGL(argmax_kernel<false>, dim3(rows), dim3(kArgmaxThreads), 0, s, logits,
                           row_stride, V, greedy);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, s, greedy, draft, parent, T,
                       accept_len, path, next_token, err);
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs &c, int B, int Hkv, int32_t *new_lens, hipStream_t s) {
    hipLaunchKernelGGL(commit_kernel, dim3(c.T, Hkv, B), dim3(64), 0, s, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lens_kernel, dim3((B + 255) / 256), dim3(256), 0, s, c.seq_lens,
                       c.accept_len, B, c.T, c.capacity, new_lens);
    return hipGetLastError();
}

}  // namespace ta
