// Greedy tree acceptance and accepted-path KV commit on gfx950: the two data-parallel steps that
// follow the verify step's attention.
//
// Greedy verification (textbook page, "Faster decoding", greedy verification contract): the
// target's greedy token at a position is the argmax of its logits; on a draft tree a node is
// accepted when its draft token equals the greedy token of its parent's row (the root row for a
// root-attached node) and its parent is accepted; the deepest accepted node ends the committed
// path, and the greedy token of its row is emitted as the correction token.
//
// argmax_kernel: every logits row is cut into chunks of 32 KB, one workgroup each, every thread
// holding 8 16-byte loads in flight (vocabularies of 1e5+ entries make this the HBM-bound part).
// Each thread scans its entries in increasing index order keeping the first maximum; winners
// merge by (larger value, then smaller index) and each chunk's winner goes to the workspace. NaN
// never wins; a row of NaN only gives 0.
// accept_kernel: one workgroup per sequence merges its rows' chunk winners into the greedy
// tokens and resolves the tree in log2(T) pointer-jumping rounds (T <= 256).
//
// Commit (same page, reserve / execute / commit: only the accepted prefix's target KV is
// committed): commit_kernel copies the path's tree K/V rows to cache positions L, L + 1, ... of
// the sequence (contiguous or paged) and advances its length, one workgroup per sequence in one
// launch. A commit that would pass the cache capacity writes nothing and keeps the length.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace ta {

namespace {

constexpr int kArgmaxThreads = 256;
constexpr int kVecPerThread = 8;                                  // loads in flight per thread
constexpr int kChunkVecs = kArgmaxThreads * kVecPerThread;       // 16-byte vectors per chunk
constexpr int kJumps = 8;                                         // 2^kJumps >= deepest tree
static_assert((1 << kJumps) >= TA_MAX_TREE, "pointer jumping must reach the root");

struct Best {
    float v;
    int i;  // -1: nothing seen but NaN
};

__device__ inline Best better(Best a, Best b) {
    if (a.i < 0) return b;
    if (b.i < 0) return a;
    if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
    return a;
}

__device__ inline Best block_best(Best best) {
    // wavefront butterflies, then the wavefronts through LDS
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) best = better(best, Best{__shfl_xor(best.v, m), __shfl_xor(best.i, m)});
    __shared__ float sv[kArgmaxThreads / 64];
    __shared__ int si[kArgmaxThreads / 64];
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // a previous call's readers are done
    if ((threadIdx.x & 63) == 0) {
        sv[wave] = best.v;
        si[wave] = best.i;
    }
    __syncthreads();
    Best r{sv[0], si[0]};
#pragma unroll
    for (int q = 1; q < kArgmaxThreads / 64; ++q) r = better(r, Best{sv[q], si[q]});
    return r;
}

template <bool BF16>
__device__ inline uint32_t word(const uint4 &w, int j) {
    const int q = BF16 ? j / 2 : j;
    return q == 0 ? w.x : q == 1 ? w.y : q == 2 ? w.z : w.w;
}

// Entry j of a 16-byte vector: its bit pattern as a signed integer (bf16: 16 bits) and its value.
template <bool BF16>
__device__ inline int bits(const uint4 &w, int j) {
    const uint32_t u = word<BF16>(w, j);
    return BF16 ? (int)(int16_t)((j & 1) ? (u >> 16) : (u & 0xffffu)) : (int)u;
}

template <bool BF16>
__device__ inline float elem(const uint4 &w, int j) {
    const uint32_t u = word<BF16>(w, j);
    if (!BF16) return __uint_as_float(u);
    return __uint_as_float((j & 1) ? (u & 0xffff0000u) : (u << 16));
}

template <bool BF16>
__device__ inline float tail_elem(const char *base, int i) {
    if (BF16) return __uint_as_float((uint32_t) reinterpret_cast<const uint16_t *>(base)[i] << 16);
    return reinterpret_cast<const float *>(base)[i];
}

template <bool BF16>
__device__ inline int tail_bits(const char *base, int i) {
    if (BF16) return (int)reinterpret_cast<const int16_t *>(base)[i];
    return reinterpret_cast<const int32_t *>(base)[i];
}

template <bool MAX>
__device__ inline int block_reduce(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const int o = __shfl_xor(v, m);
        v = MAX ? max(v, o) : min(v, o);
    }
    __shared__ int sr[kArgmaxThreads / 64];
    __syncthreads();  // a previous call's readers are done
    if ((threadIdx.x & 63) == 0) sr[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = sr[0];
#pragma unroll
    for (int q = 1; q < kArgmaxThreads / 64; ++q) r = MAX ? max(r, sr[q]) : min(r, sr[q]);
    return r;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Workgroup (row, chunk): vectors [chunk * kChunkVecs, (chunk + 1) * kChunkVecs) of the row,
// thread t taking vectors t, t + 256, ...; all of a thread's loads are issued before any is
// scanned. Past the row's last full vector the index is clamped to it: such a copy repeats an
// entry at a larger index and so never wins against the original. The last chunk also takes the
// entries past the last full vector.
//
// Fast path: read as signed integers, the bit patterns of non-negative floats order like their
// values and every negative float (sign bit set) sorts below them, so a plain integer maximum of
// the raw patterns (two bf16 per packed 16-bit max) finds the largest value whenever that value
// is positive and not NaN (pattern in (0, +inf]); the first entry holding that exact pattern is
// then the first maximum. Any other chunk (maximum <= +0, where -0 and +0 tie, or a positive NaN
// present) takes the exact path: a strict greater-than in increasing index order, which keeps the
// first maximum and skips NaN, then the first -inf if nothing is above -inf.
template <bool BF16>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_kernel(const void *logits, int64_t row_stride,
                                                                int V, int S, int2 *part) {
    constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
    constexpr int kPosInf = BF16 ? 0x7f80 : 0x7f800000;
    const int64_t row = blockIdx.x / S;
    const int chunk = blockIdx.x % S;
    const char *base = static_cast<const char *>(logits) + row * row_stride * (BF16 ? 2 : 4);
    const int nvec = V / EPV;
    const uint4 *vp = reinterpret_cast<const uint4 *>(base);
    const int c0 = chunk * kChunkVecs + threadIdx.x;
    const bool tail = chunk == S - 1;
    auto slot_index = [&](int sl) { return (c0 + (sl / EPV) * kArgmaxThreads) * EPV + sl % EPV; };
    uint4 w[kVecPerThread];
    int tmax = INT32_MIN;
    if (nvec > 0) {
#pragma unroll
        for (int k = 0; k < kVecPerThread; ++k) w[k] = vp[min(c0 + k * kArgmaxThreads, nvec - 1)];
        if (BF16) {
            s16x2 mx = {(short)-32768, (short)-32768};
#pragma unroll
            for (int k = 0; k < kVecPerThread; ++k) {
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(s16x2, w[k].x));
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(s16x2, w[k].y));
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(s16x2, w[k].z));
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(s16x2, w[k].w));
            }
            tmax = max((int)mx.x, (int)mx.y);
        } else {
#pragma unroll
            for (int k = 0; k < kVecPerThread; ++k)
                tmax = max(max(tmax, (int)w[k].x), max(max((int)w[k].y, (int)w[k].z), (int)w[k].w));
        }
    }
    for (int i = nvec * EPV + threadIdx.x; tail && i < V; i += kArgmaxThreads)
        tmax = max(tmax, tail_bits<BF16>(base, i));
    const int M = block_reduce<true>(tmax);
    Best r;
    if (M > 0 && M <= kPosInf) {
        int first = INT32_MAX;
        if (tmax == M) {
            if (nvec > 0) {
                int sl = -1;
#pragma unroll
                for (int k = kVecPerThread - 1; k >= 0; --k)
#pragma unroll
                    for (int j = EPV - 1; j >= 0; --j)
                        if (bits<BF16>(w[k], j) == M) sl = k * EPV + j;
                if (sl >= 0) first = slot_index(sl);
            }
            for (int i = nvec * EPV + threadIdx.x; tail && first == INT32_MAX && i < V;
                 i += kArgmaxThreads)
                if (tail_bits<BF16>(base, i) == M) first = i;
        }
        r.i = block_reduce<false>(first);
        r.v = BF16 ? __uint_as_float((uint32_t)M << 16) : __int_as_float(M);
    } else {
        float bv = -INFINITY;
        int bs = -1;  // slot of the best entry so far
        if (nvec > 0) {
#pragma unroll
            for (int k = 0; k < kVecPerThread; ++k)
#pragma unroll
                for (int j = 0; j < EPV; ++j) {
                    const float x = elem<BF16>(w[k], j);
                    if (x > bv) {
                        bv = x;
                        bs = k * EPV + j;
                    }
                }
        }
        Best best{bv, bs < 0 ? -1 : slot_index(bs)};
        for (int i = nvec * EPV + threadIdx.x; tail && i < V; i += kArgmaxThreads) {
            const float x = tail_elem<BF16>(base, i);
            if (x > best.v) best = Best{x, i};
        }
        r = block_best(best);
        if (r.i < 0) {
            // every entry of the chunk is -inf or NaN: the first -inf, if any
            int first = INT32_MAX;
            if (nvec > 0) {
                int sl = -1;
#pragma unroll
                for (int k = kVecPerThread - 1; k >= 0; --k)
#pragma unroll
                    for (int j = EPV - 1; j >= 0; --j)
                        if (elem<BF16>(w[k], j) == -INFINITY) sl = k * EPV + j;
                if (sl >= 0) first = slot_index(sl);
            }
            for (int i = nvec * EPV + threadIdx.x; tail && first == INT32_MAX && i < V;
                 i += kArgmaxThreads)
                if (tail_elem<BF16>(base, i) == -INFINITY) first = i;
            first = block_reduce<false>(first);
            r = Best{-INFINITY, first == INT32_MAX ? -1 : first};
        }
    }
    if (threadIdx.x == 0) part[blockIdx.x] = make_int2(__float_as_int(r.v), r.i);
}

// One workgroup per sequence, thread i = tree node i. The chunk winners of every row merge into
// the greedy tokens; every node then checks its own agreement, and pointer jumping (round k
// joins each node with its ancestor 2^k levels up) gives every node its depth and whether all
// of its root path agrees, keeping the ancestor tables jump[k]. A block maximum over
// (depth, -index) picks the path's last node, and slot j of the path is that node's ancestor
// n - 1 - j levels up, read from the tables.
__global__ __launch_bounds__(TA_MAX_TREE) void accept_kernel(const int2 *part, int S,
                                                             const int32_t *draft,
                                                             const int32_t *parent, int T,
                                                             int32_t *greedy, int32_t *accept_len,
                                                             int32_t *path, int32_t *next_token,
                                                             int32_t *err) {
    __shared__ int32_t jump[kJumps][TA_MAX_TREE];  // ancestor 2^k levels up, -1 past the root
    __shared__ int32_t st[2][TA_MAX_TREE];         // (levels covered << 1) | all of them agree
    __shared__ int32_t g[TA_MAX_TREE + 1];
    __shared__ int32_t red[TA_MAX_TREE / 64];
    const int b = blockIdx.x, i = threadIdx.x;
    const bool node = i < T;
    int anc = -1, tok = 0;
    if (node) {  // loads issued ahead of the chunk winners'
        anc = parent[(int64_t)b * T + i];
        tok = draft[(int64_t)b * T + i];
    }
    for (int r = i; r <= T; r += TA_MAX_TREE) {
        const int2 *pr = part + ((int64_t)b * (T + 1) + r) * S;
        Best w{__int_as_float(pr[0].x), pr[0].y};
#pragma unroll 4
        for (int c = 1; c < S; ++c) w = better(w, Best{__int_as_float(pr[c].x), pr[c].y});
        g[r] = w.i < 0 ? 0 : w.i;
        greedy[(int64_t)b * (T + 1) + r] = g[r];
    }
    if (node) {
        if (anc < -1 || anc >= i) {
            if (err) atomicOr(err, (int32_t)TA_DEV_BAD_PARENT);
            anc = -1;
        }
        jump[0][i] = anc;
    }
    __syncthreads();
    int ok = node && tok == g[anc + 1];
    int levels = 1;
    if (node) st[0][i] = (levels << 1) | ok;
    for (int k = 0; k < kJumps; ++k) {
        // also the barrier after the previous round's writes
        if (!__syncthreads_or(node && anc >= 0)) break;
        if (node && anc >= 0) {
            const int up = st[k & 1][anc];
            ok &= up & 1;
            levels += up >> 1;
            anc = jump[k][anc];
        }
        if (node) {
            if (k + 1 < kJumps) jump[k + 1][i] = anc;
            st[(k + 1) & 1][i] = (levels << 1) | ok;
        }
    }
    // the deepest accepted node, the smallest index among equally deep ones
    int key = node && ok ? (levels << 9) | (511 - i) : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) key = max(key, __shfl_xor(key, m));
    if ((i & 63) == 0) red[i >> 6] = key;
    __syncthreads();
    key = red[0];
#pragma unroll
    for (int q = 1; q < TA_MAX_TREE / 64; ++q) key = max(key, red[q]);
    const int n = key >> 9;
    const int last = key ? 511 - (key & 511) : -1;
    if (i == 0) {
        accept_len[b] = n;
        next_token[b] = g[last + 1];
    }
    if (node) {
        int v = -1;
        if (i < n) {
            const int up = n - 1 - i;
            v = last;
            for (int k = 0; k < kJumps; ++k)
                if ((up >> k) & 1) v = jump[k][v];
        }
        path[(int64_t)b * T + i] = v;
    }
}

// One workgroup per sequence b: copies the tree K/V rows path[b][0 .. n-1] of every KV head to
// cache positions seq_lens[b] .. seq_lens[b] + n - 1, then writes the new length. Each thread
// moves up to kCommitVec 16-byte pieces per round, all loads issued before any store (a typical
// commit -- a few rows of a few KV heads -- is one round). The workgroup is the only reader of
// seq_lens[b] and writes new_lens[b] after a barrier that follows its read, so new_lens may alias
// seq_lens in the same launch.
constexpr int kCommitThreads = 512;
constexpr int kCommitVec = 4;

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitArgs c, int Hkv,
                                                                int32_t *new_lens) {
    const int b = blockIdx.x;
    const int n = c.accept_len[b];
    const int L = c.seq_lens[b];
    __syncthreads();  // every thread has read the old length before it is overwritten below
    const bool len_ok = L >= 0 && L <= c.capacity;
    const bool fits = n >= 0 && n <= c.T && L + n <= c.capacity;
    if (threadIdx.x == 0 && c.err && n > 0) {
        if (!len_ok) atomicOr(c.err, (int32_t)TA_DEV_BAD_LEN);
        else if (!fits) atomicOr(c.err, (int32_t)TA_DEV_BAD_COMMIT);
    }
    if (len_ok && fits) {
        const int chunks = c.row_bytes / 16;            // 16-byte pieces of one K (or V) row
        const int per_slot = Hkv * 2 * chunks;          // every KV head, K then V
        const int total = n * per_slot;
        for (int base = 0; base < total; base += kCommitThreads * kCommitVec) {
            uint4 val[kCommitVec];
            char *dst_p[kCommitVec];
#pragma unroll
            for (int u = 0; u < kCommitVec; ++u) {
                dst_p[u] = nullptr;
                const int t = base + u * kCommitThreads + threadIdx.x;
                if (t >= total) continue;
                const int j = t / per_slot;
                int r = t - j * per_slot;
                const int g = r / (2 * chunks);
                r -= g * 2 * chunks;
                const bool v = r >= chunks;
                const int q = v ? r - chunks : r;
                const int node = c.path[(int64_t)b * c.T + j];
                if (node < 0 || node >= c.T) {
                    if (c.err && q == 0 && !v) atomicOr(c.err, (int32_t)TA_DEV_BAD_COMMIT);
                    continue;
                }
                const int pos = L + j;
                int64_t dst;
                if (c.block_table) {
                    const int pg = c.block_table[(int64_t)b * c.max_blocks + (pos >> c.page_shift)];
                    if ((unsigned)pg >= (unsigned)c.num_pages) {
                        if (c.err && q == 0 && !v) atomicOr(c.err, (int32_t)TA_DEV_BAD_PAGE);
                        continue;
                    }
                    dst = pg * c.kv_s0 + (pos & c.page_mask) * c.kv_s1 + g * c.kv_s2;
                } else {
                    dst = b * c.kv_s0 + (int64_t)pos * c.kv_s1 + g * c.kv_s2;
                }
                const int64_t src = b * c.kt_sb + (int64_t)node * c.kt_st + g * c.kt_sh;
                val[u] = *reinterpret_cast<const uint4 *>(
                    static_cast<const char *>(v ? c.vt : c.kt) + src * c.es + 16 * q);
                dst_p[u] = static_cast<char *>(v ? c.vc : c.kc) + dst * c.es + 16 * q;
            }
#pragma unroll
            for (int u = 0; u < kCommitVec; ++u)
                if (dst_p[u]) *reinterpret_cast<uint4 *>(dst_p[u]) = val[u];
        }
    }
    if (threadIdx.x == 0) new_lens[b] = len_ok && fits ? L + n : L;
}

}  // namespace

int greedy_accept_chunks(int V, bool bf16) {
    const int nvec = V / (bf16 ? 8 : 4);
    return nvec > kChunkVecs ? (nvec + kChunkVecs - 1) / kChunkVecs : 1;
}

hipError_t launch_greedy_accept(const void *logits, bool bf16, int64_t row_stride, int B, int T,
                                int V, int S, const int32_t *draft, const int32_t *parent,
                                int2 *part, int32_t *greedy, int32_t *accept_len, int32_t *path,
                                int32_t *next_token, int32_t *err, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)B * (T + 1) * S));
    if (bf16)
        hipLaunchKernelGGL(argmax_kernel<true>, grid, dim3(kArgmaxThreads), 0, s, logits,
                           row_stride, V, S, part);
    else
        hipLaunchKernelGGL(argmax_kernel<false>, grid, dim3(kArgmaxThreads), 0, s, logits,
                           row_stride, V, S, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(TA_MAX_TREE), 0, s, part, S, draft, parent, T,
                       greedy, accept_len, path, next_token, err);
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs &c, int B, int Hkv, int32_t *new_lens, hipStream_t s) {
    hipLaunchKernelGGL(commit_kernel, dim3(B), dim3(kCommitThreads), 0, s, c, Hkv, new_lens);
    return hipGetLastError();
}

}  // namespace ta
