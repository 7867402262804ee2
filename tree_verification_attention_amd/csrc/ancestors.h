// Ancestor-or-self bit masks of a draft tree, built cooperatively by one workgroup in LDS.
//
// The tree mask lets every node attend only to its ancestors (textbook page "更快的解码",
// section on linear chains vs candidate trees; LongSpec page, "Fast tree attention"); the node
// itself is included. Nodes are numbered topologically (parent[i] < i), -1 = attached to the
// committed prefix.
//
// Pointer jumping: start from M(i) = {i}, J(i) = parent(i). Each round sets
// M(i) |= M(J(i)) and J(i) = J(J(i)), so after k rounds M(i) holds every ancestor at distance
// below 2^k and J(i) the one at distance 2^k. The rounds stop once every J(i) has passed the
// root: about log2(depth) rounds, at most ceil(log2 T) for any tree with T <= 256. Only the
// ceil(T / 64) words a tree needs are written.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "treeattn.h"

namespace ta {

constexpr int kMaskWords = TA_MAX_TREE / 64;

// LDS scratch for one tree: two mask buffers and two jump buffers.
struct AncestorLds {
    uint64_t m[2][TA_MAX_TREE][kMaskWords];
    int32_t j[2][TA_MAX_TREE];
};

// Builds the masks of the tree ``parent`` (T entries, global memory) and returns the index of
// the buffer of ``s`` that holds them. Every thread of the block must call it. Invalid parents
// set TA_DEV_BAD_PARENT in *err (when non-null) and count as -1.
__device__ inline int build_ancestor_masks(const int32_t *parent, int T, AncestorLds &s,
                                           int32_t *err, int tid, int nthreads) {
    const int W = (T + 63) >> 6;  // mask words in use
    for (int i = tid; i < T; i += nthreads) {
        int p = parent[i];
        if (p < -1 || p >= i) {
            if (err) atomicOr(err, (int32_t)TA_DEV_BAD_PARENT);
            p = -1;
        }
        s.j[0][i] = p;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w)
            if (w < W) s.m[0][i][w] = (w == (i >> 6)) ? (1ull << (i & 63)) : 0ull;
    }
    __syncthreads();
    int cur = 0;
    for (int span = 1; span < T; span <<= 1) {
        // done once every jump pointer has passed the root (after about log2(depth) rounds)
        bool more = false;
        for (int i = tid; i < T; i += nthreads) more |= s.j[cur][i] >= 0;
        if (!__syncthreads_or(more)) break;
        for (int i = tid; i < T; i += nthreads) {
            const int j = s.j[cur][i];
#pragma unroll
            for (int w = 0; w < kMaskWords; ++w)
                if (w < W) s.m[cur ^ 1][i][w] = s.m[cur][i][w] | (j >= 0 ? s.m[cur][j][w] : 0ull);
            s.j[cur ^ 1][i] = j >= 0 ? s.j[cur][j] : -1;
        }
        __syncthreads();
        cur ^= 1;
    }
    return cur;
}

}  // namespace ta
