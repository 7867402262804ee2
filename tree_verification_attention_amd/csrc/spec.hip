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
// spec_mass_kernel (data-parallel, HBM-bound): per (row, 4096-entry chunk) of every position
//   with children, the chunk's sum of [p - q]_+ (N_2's parts: a first rejection there needs it).
// spec_walk_kernel: G workgroups per sequence, all walking the same tree with the same state.
//   The per-node values p(x), q(x) and the acceptance uniforms are gathered up front, so the walk
//   itself reads LDS only; a second trial at one position needs N_{k+1} for k >= 2, a pass over
//   that row which the G workgroups split by chunks and meet on through the workspace; the final
//   token's chunk is found from the chunk sums, then its owner scans it with a block prefix sum.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace ta {

namespace {

constexpr int kMassThreads = 256;
constexpr int kWalkThreads = 256;
constexpr int kSpinLimit = 1 << 20;      // polls before a workgroup stops waiting for its peers
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
                                                                 double *sums, double *pass_sums) {
    const int chunk = blockIdx.x;
    const int row_id = blockIdx.y;  // b * (T + 1) + row
    // the walk's pass slots (as many as chunk sums here) start empty
    if (threadIdx.x == 0) pass_sums[(int64_t)row_id * nch + chunk] = -1.0;
    const int b = row_id / (T + 1), row = row_id % (T + 1);
    // rows of positions without children are never needed here: a bonus token's weights come
    // from a pass of the walk over the one row it ends on
    if (!position_has_child(parent + (int64_t)b * T, T, row - 1)) return;
    constexpr bool use_q = true;
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

constexpr int kKidWords = TA_MAX_TREE / 64;

struct WalkShared {
    unsigned long long kids[TA_MAX_TREE + 1][kKidWords];  // children of each row, as bit sets
    int32_t first_child[TA_MAX_TREE + 1];
    int32_t next_sib[TA_MAX_TREE];
    float pv[TA_MAX_TREE];             // p(x) and q(x) of every node's draft token at its row
    float qv[TA_MAX_TREE];
    double ua[TA_MAX_TREE];            // every node's acceptance uniform
    double n2[TA_MAX_TREE + 1];        // N_2 of every row with children
    double cs[TA_MAX_VOCAB / kChunk];  // chunk sums of the current final weights
    double red[kWalkThreads / 64];
    int32_t path[TA_MAX_TREE];
    // walk state (written by thread 0; every workgroup of a sequence holds the same)
    int32_t pos, child, k, n_path, have_pass, done, bonus, n_pass, pass_q;
    double Cprev, Nk, pass_C, pass_N, theta, base;
    int32_t pass_row, chunk_hit;
};

// Sum of R = [p - C q]_+ (or p) over chunk ch of one row, by the whole workgroup; the result is
// valid in thread 0. Fixed thread mapping and order, so every workgroup gets the same bits.
__device__ inline double chunk_sum_block(const float *pr, const float *qr, double C, bool use_q,
                                         int ch, int nch, int V, double *red) {
    const int tid = threadIdx.x, nvec = V / 4;
    double s = 0.0;
    float4 pv[kChunkVec / kWalkThreads], qv[kChunkVec / kWalkThreads];
#pragma unroll
    for (int k = 0; k < kChunkVec / kWalkThreads; ++k) {
        const int v = ch * kChunkVec + k * kWalkThreads + tid;
        pv[k] = v < nvec ? reinterpret_cast<const float4 *>(pr)[v] : make_float4(0, 0, 0, 0);
        qv[k] = use_q && v < nvec ? reinterpret_cast<const float4 *>(qr)[v]
                                  : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kChunkVec / kWalkThreads; ++k) s += entry4(pv[k], qv[k], C, use_q);
    if (ch == nch - 1)
        for (int e = nvec * 4 + tid; e < V; e += kWalkThreads) s += entry(pr[e], use_q ? qr[e] : 0.f, C, use_q);
    s = wave_sum(s);
    __syncthreads();  // red is free
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    double t = 0.0;
    if (tid == 0)
        for (int w = 0; w < kWalkThreads / 64; ++w) t += red[w];
    return t;
}

// One sequence is walked by G workgroups (blockIdx.x = g). They hold identical walk state and
// take identical decisions; a row pass is split between them (chunk c by workgroup c mod G) and
// its chunk sums meet in fresh workspace slots that start at -1, each reader polling a slot
// until its owner has filled it. A workgroup that waits too long (its peers not resident)
// computes the missing chunks itself with the same arithmetic, so the decisions never depend on
// the schedule.
__global__ __launch_bounds__(kWalkThreads) void spec_walk_kernel(SpecArgs a, int nch, int G) {
    __shared__ WalkShared sh;
    const float *p = a.p, *q = a.q;
    const int64_t row_stride = a.row_stride;
    const int T = a.T, V = a.V;
    const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row0 = (int64_t)b * (T + 1);
    int32_t *err = a.err;
    int pa = -1, x = 0;
    double ua = 0.0;
    if (tid < T) {
        pa = a.parent[(int64_t)b * T + tid];
        x = a.draft[(int64_t)b * T + tid];
        ua = a.u_accept[(int64_t)b * T + tid];
    }
    // N_2 of every row with children: four threads per row, thread j summing chunks j, j + 4, ...
    // in order, then two butterfly steps. The first kPre chunk sums of every thread in the first
    // group of rows are loaded here, before the tree is even known, so that the wait for them
    // overlaps the gathers and the child lists (a leaf row holds no sums; its total is dropped)
    constexpr int kRowsPerPass = kWalkThreads / 4, kPre = 8;
    const int n2_row = tid >> 2, n2_j = tid & 3;
    double n_pre[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int c = n2_j + 4 * k;
        n_pre[k] = n2_row <= T && c < nch ? a.sums[(row0 + n2_row) * nch + c] : 0.0;
    }
    for (int i = tid; i < (T + 1) * kKidWords; i += kWalkThreads) (&sh.kids[0][0])[i] = 0;
    if (tid < T) {
        if (pa < -1 || pa >= tid) {
            if (err && g == 0) atomicOr(err, (int32_t)TA_DEV_BAD_PARENT);
            pa = -1;
        }
        sh.ua[tid] = ua;
        // p(x) and q(x) of the node's draft token, at its parent's row
        const int64_t ro = (row0 + pa + 1) * row_stride;
        if (x >= 0 && x < V) {
            sh.pv[tid] = p[ro + x];
            sh.qv[tid] = q[ro + x];
        } else {
            // a token outside the vocabulary has no target mass: it is always rejected
            if (err && g == 0) atomicOr(err, (int32_t)TA_DEV_BAD_TOKEN);
            sh.pv[tid] = 0.f;
            sh.qv[tid] = 1.f;
        }
    }
    __syncthreads();
    // child lists as bit sets: bit i of row pa + 1 for node i; a row's first child is its lowest
    // bit, a node's next sibling the lowest bit above its own
    if (tid < T) atomicOr(&sh.kids[pa + 1][tid >> 6], 1ull << (tid & 63));
    __syncthreads();
    for (int r = tid; r <= T; r += kWalkThreads) {
        int fc = -1;
        for (int w = kKidWords - 1; w >= 0; --w)
            if (sh.kids[r][w]) fc = 64 * w + __builtin_ctzll(sh.kids[r][w]);
        sh.first_child[r] = fc;
    }
    if (tid < T) {
        int nx = -1;
        for (int w = kKidWords - 1; w >= tid >> 6; --w) {
            unsigned long long m = sh.kids[pa + 1][w];
            if (w == tid >> 6) m &= (tid & 63) == 63 ? 0ull : ~0ull << ((tid & 63) + 1);
            if (m) nx = 64 * w + __builtin_ctzll(m);
        }
        sh.next_sib[tid] = nx;
    }
    __syncthreads();
    for (int r0 = 0; r0 <= T; r0 += kRowsPerPass) {
        const int r = r0 + n2_row;
        const double *sr = a.sums + (row0 + r) * nch;
        double v = 0.0;
#pragma unroll
        for (int k = 0; k < kPre; ++k) {
            const int c = n2_j + 4 * k;
            v += r0 == 0 ? n_pre[k] : (r <= T && c < nch ? sr[c] : 0.0);
        }
        if (r <= T)
            for (int c = n2_j + 4 * kPre; c < nch; c += 4) v += sr[c];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        if (n2_j == 0 && r <= T) sh.n2[r] = sh.first_child[r] >= 0 ? v : 0.0;
    }
    if (tid == 0) {
        sh.pos = -1;
        sh.child = -2;
        sh.n_path = 0;
        sh.have_pass = 0;
        sh.done = 0;
        sh.n_pass = 0;
    }
    __syncthreads();
    // -------- the walk: thread 0 advances it; the workgroups make the row passes it asks for --
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
                if (c < 0) {  // no children: bonus token from this row's p, whose chunk sums a
                              // pass over the row provides
                    if (!sh.have_pass) {
                        sh.pass_row = row;
                        sh.pass_C = 0.0;
                        sh.pass_q = 0;
                        break;
                    }
                    sh.bonus = 1;
                    sh.done = 1;
                    break;
                }
                double n_next;
                if (sh.k == 1) {
                    n_next = sh.n2[row];
                } else if (sh.have_pass) {
                    n_next = sh.pass_N;
                } else {  // N_{k+1} = sum [p - C_k q]_+ : ask for a pass over the row
                    sh.pass_row = row;
                    sh.pass_C = sh.Cprev + sh.Nk;
                    sh.pass_q = 1;
                    break;
                }
                const double R = fmax(0.0, (double)sh.pv[c] - sh.Cprev * (double)sh.qv[c]);
                const bool accept = n_next == 0.0 || sh.ua[c] * sh.Nk * (double)sh.qv[c] < R;
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
        // row pass: this workgroup's chunks of [p - pass_C q]_+, then everyone's
        const int64_t ro = (row0 + sh.pass_row) * row_stride;
        const double C = sh.pass_C;
        const bool pq = sh.pass_q;
        const int pass = sh.n_pass;
        double *buf = a.pass_sums + ((int64_t)b * (T + 1) + pass) * nch;
        for (int ch = g; ch < nch; ch += G) {
            const double s = chunk_sum_block(p + ro, q + ro, C, pq, ch, nch, V, sh.red);
            if (tid == 0) {
                __hip_atomic_store(buf + ch, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                sh.cs[ch] = s;
            }
        }
        // the peers' chunks: a thread per chunk polls its slot until the owner has written it
        // (the mass kernel set every slot to -1; sums are >= 0). The slot's value is all that is
        // handed over, so device-scope relaxed atomics suffice: they bypass the XCD's L2 without
        // the L2 write-back and invalidation that release / acquire order would add per access
        bool late = false;
        for (int ch = tid; ch < nch; ch += kWalkThreads) {
            if (ch % G == g) continue;
            double v = __hip_atomic_load(buf + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int spin = 0; v < 0.0 && spin < kSpinLimit; ++spin) {
                __builtin_amdgcn_s_sleep(2);
                v = __hip_atomic_load(buf + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (v < 0.0) late = true;
            else sh.cs[ch] = v;
        }
        if (__syncthreads_or(late)) {
            // peers not resident: every other chunk here, with the same arithmetic
            for (int ch = 0; ch < nch; ++ch)
                if (ch % G != g) {
                    const double s = chunk_sum_block(p + ro, q + ro, C, pq, ch, nch, V, sh.red);
                    if (tid == 0) sh.cs[ch] = s;
                }
        }
        __syncthreads();
        if (wave == 0) {
            // N_{k+1}: lane l sums chunks l, l + 64, ..., then a butterfly (a fixed order)
            double n = 0.0;
            for (int c = lane; c < nch; c += 64) n += sh.cs[c];
            n = wave_sum(n);
            if (lane == 0) {
                sh.pass_N = n;
                sh.have_pass = 1;
                sh.n_pass = pass + 1;
            }
        }
        __syncthreads();
    }
    // -------- the emitted token --------
    const int row = sh.pos + 1;
    const int64_t ro = (row0 + row) * row_stride;
    const bool use_q = !sh.bonus;
    const double C = sh.Cprev;
    // chunk sums of the final weights: the mass kernel's for a correction after one trial
    // ([p - q]_+), else those of the last row pass (already in cs; the bonus's pass sums p)
    const bool from_pass = sh.bonus || sh.k > 2;
    if (!from_pass)
        for (int c = tid; c < nch; c += kWalkThreads) sh.cs[c] = a.sums[(row0 + row) * nch + c];
    __syncthreads();
    if (wave == 0) {
        // running sums of the chunk sums: lane l holds chunks 4l .. 4l + 3 (nch <= 256)
        double cl[4], own = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * lane + i;
            cl[i] = c < nch ? sh.cs[c] : 0.0;
            own += cl[i];
        }
        double incl = own;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const double o = __shfl_up(incl, m);
            if (lane >= m) incl += o;
        }
        const double total = __shfl(incl, 63);
        const double theta = a.u_sample[b] * total;
        // the first chunk whose running sum passes theta, and the last chunk with mass
        double cum = incl - own;
        int hit = -1, last_pos = -1;
        double base = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (cl[i] > 0.0) last_pos = 4 * lane + i;
            if (hit < 0 && cum + cl[i] > theta) {
                hit = 4 * lane + i;
                base = cum;
            }
            cum += cl[i];
        }
        const uint64_t hits = __ballot(hit >= 0);
        int lp = last_pos;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) lp = max(lp, __shfl_xor(lp, m));
        const int first = hits ? __builtin_ctzll(hits) : -1;
        if (lane == (first < 0 ? 0 : first)) {
            sh.theta = theta;
            if (first >= 0) {
                sh.chunk_hit = hit;
                sh.base = base;
            } else {  // rounding left theta past the total: the last chunk with mass
                sh.chunk_hit = lp < 0 ? 0 : lp;
                sh.base = -INFINITY;  // no entry passes: take the chunk's last positive entry
            }
            if (g == 0) a.accept_len[b] = sh.n_path;
        }
    }
    __syncthreads();
    if (g == 0)
        for (int j = tid; j < T; j += kWalkThreads)
            a.path[(int64_t)b * T + j] = j < sh.n_path ? sh.path[j] : -1;
    if (sh.chunk_hit % G != g) return;  // the chunk's owner draws the token
    {
        // this thread's entries e0 .. e0 + kEntries - 1 of the chunk
        constexpr int kEntries = kChunk / kWalkThreads;
        const int e0 = sh.chunk_hit * kChunk + kEntries * tid;
        double w[kEntries], t = 0.0;
#pragma unroll
        for (int j = 0; j < kEntries; ++j) {
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
        for (int j = 0; j < kEntries; ++j) {
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
            a.next_token[b] = k2 != INT32_MAX ? k2 : (l2 >= 0 ? l2 : 0);
        }
    }
}

}  // namespace

int spec_sample_chunks(int V) { return (V + kChunk - 1) / kChunk; }

hipError_t launch_spec_sample(const SpecArgs &a, int cus, hipStream_t s) {
    const int nch = spec_sample_chunks(a.V);
    // workgroups per sequence: one per chunk, as far as the compute units go
    int G = cus / (a.B > 0 ? a.B : 1);
    G = G < 1 ? 1 : (G > nch ? nch : G);
    hipLaunchKernelGGL(spec_mass_kernel, dim3(nch, a.B * (a.T + 1)), dim3(kMassThreads), 0, s, a.p,
                       a.q, a.row_stride, a.T, a.V, nch, a.parent, a.sums, a.pass_sums);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(spec_walk_kernel, dim3(G, a.B), dim3(kWalkThreads), 0, s, a, nch, G);
    return hipGetLastError();
}

}  // namespace ta
