// fp32 attention parts for tree verification (the fp32-input path).
//
// Same partial outputs as the bf16 kernel -- one (O, LSE) per (part, row) for a prefix chunk,
// plus the masked tree keys in the last part -- computed with plain fp32 vector arithmetic: there
// is no fp32 MFMA shape worth using at these sizes. One 256-thread workgroup per (row, part): 64
// key slots of four lanes each (a key's D entries split over the four), every slot walking its
// own keys with an online softmax, then the 64 slot partials merged through LDS by the
// log-sum-exp identity. A single-split problem runs its prefix and tree keys in this one launch
// and writes the final output (tree_attn_forward's fp32 path).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace ta {

constexpr int kF32Threads = 256;
constexpr int kLanesPerKey = 4;                         // lanes sharing one key's D entries
constexpr int kKeySlots = kF32Threads / kLanesPerKey;   // keys in flight per workgroup

template <int D>
__global__ __launch_bounds__(kF32Threads) void attn_f32_kernel(AttnArgs a) {
    constexpr int DL = D / kLanesPerKey;  // entries of a key (and of O) per lane
    __shared__ float qs[D];
    __shared__ int32_t par[TA_MAX_TREE];
    __shared__ uint32_t anc[TA_MAX_TREE / 32];
    __shared__ float red_o[kKeySlots][D + 1];
    __shared__ float red_m[kKeySlots], red_l[kKeySlots], red_w[kKeySlots];
    constexpr int NQ = kF32Threads / D;  // threads per output entry in the final sum
    __shared__ float red_part[NQ][D];
    __shared__ float red_tot, red_mx;

    const int tid = threadIdx.x, slot = tid / kLanesPerKey, sub = tid % kLanesPerKey;
    const int64_t row = blockIdx.x;  // (b * T + node) * Hq + h
    const int part = blockIdx.y;
    const int h = (int)(row % a.Hq);
    const int node = (int)((row / a.Hq) % a.T);
    const int b = (int)(row / ((int64_t)a.Hq * a.T));
    const int g = h / a.G;
    const bool has_tree = a.with_tree && part == a.n_splits - 1;
    if (a.seq_parts && a.with_prefix && row == 0 && part == 0)
        for (int i = tid; i < a.B; i += kF32Threads) a.seq_parts[i] = a.n_splits;

    // every key slot keeps an online softmax over its keys; the four lanes of a slot hold DL
    // entries each of the dot product (summed by two butterfly steps) and of the output
    float m = -INFINITY, l = 0.f, acc[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[i] = 0.f;
    // a slot takes KB of its keys at a time: all their K and V slices are loaded before any is
    // used, so the batch waits for memory once; the keys are then taken in order
    constexpr int KB = D == 64 ? 4 : 2;
    struct KeyVals {
        float4 k4[DL / 4], v4[DL / 4];
    };
    auto load_key = [&](const float *kp, const float *vp, KeyVals &kv) {
#pragma unroll
        for (int i = 0; i < DL / 4; ++i) {
            kv.k4[i] = reinterpret_cast<const float4 *>(kp + sub * DL)[i];
            kv.v4[i] = reinterpret_cast<const float4 *>(vp + sub * DL)[i];
        }
    };
    auto take_key = [&](const KeyVals &kv) {
        const float4 *k4 = kv.k4, *v4 = kv.v4;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < DL / 4; ++i) {
            const float *qq = qs + sub * DL + 4 * i;
            s = fmaf(qq[0], k4[i].x, s);
            s = fmaf(qq[1], k4[i].y, s);
            s = fmaf(qq[2], k4[i].z, s);
            s = fmaf(qq[3], k4[i].w, s);
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s *= a.scale;
        if (s > m) {
            const float alpha = m == -INFINITY ? 0.f : expf(m - s);
            l *= alpha;
#pragma unroll
            for (int i = 0; i < DL; ++i) acc[i] *= alpha;
            m = s;
        }
        const float pw = expf(s - m);
        l += pw;
#pragma unroll
        for (int i = 0; i < DL / 4; ++i) {
            acc[4 * i] = fmaf(pw, v4[i].x, acc[4 * i]);
            acc[4 * i + 1] = fmaf(pw, v4[i].y, acc[4 * i + 1]);
            acc[4 * i + 2] = fmaf(pw, v4[i].z, acc[4 * i + 2]);
            acc[4 * i + 3] = fmaf(pw, v4[i].w, acc[4 * i + 3]);
        }
    };
    // The query row and the tree's parents go to LDS, and the length, the slot's first batch of
    // prefix keys (contiguous layout) and, at D = 64, its first tree key to registers, all issued
    // together:
    // none of these addresses depends on the length or on the tree. Prefix keys past the length
    // (cache rows below the capacity) and tree keys outside the node's ancestors are loaded and
    // then dropped.
    const float *q = reinterpret_cast<const float *>(a.q) + b * a.q_sb + node * a.q_st + h * a.q_sh;
    if (tid < D) qs[tid] = q[tid];
    if (has_tree && tid < a.T) par[tid] = a.parent[(int64_t)b * a.T + tid];
    for (int w = tid; w < TA_MAX_TREE / 32; w += kF32Threads) anc[w] = 0u;
    int L = a.with_prefix ? a.seq_lens[b] : 0;
    const int pb = a.with_prefix ? part * a.chunk : 0;
    const bool early = a.with_prefix && !a.block_table;
    KeyVals kv0[KB];
    bool got0[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
        const int k = slot + i * kKeySlots, j = pb + k;
        got0[i] = early && k < a.chunk && j < a.capacity;
        if (got0[i]) {
            const int64_t off = b * a.kv_s0 + j * a.kv_s1 + g * a.kv_s2;
            load_key(reinterpret_cast<const float *>(a.kc) + off,
                     reinterpret_cast<const float *>(a.vc) + off, kv0[i]);
        }
    }
    KeyVals tk;
    const bool tgot = D == 64 && has_tree && slot < a.T;  // D = 128: registers for one batch only
    if (tgot) {
        const int64_t off = b * a.kt_sb + slot * a.kt_st + g * a.kt_sh;
        load_key(reinterpret_cast<const float *>(a.kt) + off, reinterpret_cast<const float *>(a.vt) + off, tk);
    }

    // prefix keys [pb, pe) of this part
    int pe = pb;
    if (a.with_prefix) {
        if (L < 0 || L > a.capacity) {
            if (a.err && tid == 0) atomicOr(a.err, (int32_t)TA_DEV_BAD_LEN);
            L = L < 0 ? 0 : a.capacity;
        }
        pe = max(pb, min(pb + a.chunk, L));
    }
    __syncthreads();
    // ancestor-or-self bitmap of `node`, walked upwards in LDS by one thread while the others
    // start on the prefix keys (it is read only after the barrier below)
    if (has_tree && tid == 0) {
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

    // prefix keys (a slot's four lanes agree on every key, so the branches stay uniform per
    // slot; the butterfly stays inside the slot's lanes)
    int k_first = slot;
    if (early) {  // the batch loaded with the query
#pragma unroll
        for (int i = 0; i < KB; ++i)
            if (got0[i] && slot + i * kKeySlots < pe - pb) take_key(kv0[i]);
        k_first = slot + KB * kKeySlots;
    }
    for (int k0 = k_first; k0 < pe - pb; k0 += KB * kKeySlots) {
        KeyVals kv[KB];
        bool ok[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) {
            const int k = k0 + i * kKeySlots, j = pb + k;
            ok[i] = k < pe - pb;
            if (!ok[i]) continue;
            int64_t off;
            if (a.block_table) {
                const int pg = a.block_table[(int64_t)b * a.max_blocks + (j >> a.page_shift)];
                if ((unsigned)pg >= (unsigned)a.num_pages) {
                    if (a.err && sub == 0) atomicOr(a.err, (int32_t)TA_DEV_BAD_PAGE);
                    ok[i] = false;
                    continue;
                }
                off = pg * a.kv_s0 + (j & a.page_mask) * a.kv_s1 + g * a.kv_s2;
            } else {
                off = b * a.kv_s0 + j * a.kv_s1 + g * a.kv_s2;
            }
            load_key(reinterpret_cast<const float *>(a.kc) + off, reinterpret_cast<const float *>(a.vc) + off, kv[i]);
        }
#pragma unroll
        for (int i = 0; i < KB; ++i)
            if (ok[i]) take_key(kv[i]);
    }
    __syncthreads();  // the ancestor bitmap is complete
    if (has_tree)
        for (int j0 = slot; j0 < a.T; j0 += KB * kKeySlots) {
            KeyVals kv[KB];
            bool ok[KB];
#pragma unroll
            for (int i = 0; i < KB; ++i) {
                const int j = j0 + i * kKeySlots;
                ok[i] = j < a.T && ((anc[j >> 5] >> (j & 31)) & 1u);
                if (!ok[i]) continue;
                if (tgot && j == slot) {  // loaded with the query
                    kv[i] = tk;
                    continue;
                }
                const int64_t off = b * a.kt_sb + j * a.kt_st + g * a.kt_sh;
                load_key(reinterpret_cast<const float *>(a.kt) + off, reinterpret_cast<const float *>(a.vt) + off, kv[i]);
            }
#pragma unroll
            for (int i = 0; i < KB; ++i)
                if (ok[i]) take_key(kv[i]);
        }

    // merge the key slots' partials by the log-sum-exp identity
    if (sub == 0) {
        red_m[slot] = m;
        red_l[slot] = l;
    }
#pragma unroll
    for (int i = 0; i < DL; ++i) red_o[slot][sub * DL + i] = acc[i];
    __syncthreads();
    // the slots' weights e^{m_i - max} and the total, by one wavefront (slot i in lane i)
    static_assert(kKeySlots == 64, "one slot per lane of the first wavefront");
    if (tid < kKeySlots) {
        const float mi = red_m[tid];
        float mxw = mi;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mxw = fmaxf(mxw, __shfl_xor(mxw, o));
        const float wi = mi == -INFINITY ? 0.f : expf(mi - mxw);
        float t = red_l[tid] * wi;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
        red_w[tid] = wi;
        if (tid == 0) {
            red_tot = t;
            red_mx = mxw;
        }
    }
    __syncthreads();
    // output entry d: NQ threads each sum every NQ-th slot, then one adds their sums
    {
        const int d = tid % D, qd = tid / D;
        float sacc = 0.f;
        for (int i = qd; i < kKeySlots; i += NQ) sacc = fmaf(red_o[i][d], red_w[i], sacc);
        red_part[qd][d] = sacc;
    }
    __syncthreads();
    const float tot = red_tot, mx = red_mx;
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    float *op = a.out_o + part * a.part_so + row * D;
    if (tid < D) {
        float sacc = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < NQ; ++q4) sacc += red_part[q4][tid];
        op[tid] = sacc * inv;
    }
    if (tid == 0) a.out_lse[part * a.part_sl + row] = tot > 0.f ? mx + logf(tot) : -INFINITY;
}

hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s) {
    const int parts = a.n_splits;
    const int64_t rows = (int64_t)a.B * a.T * a.Hq;
    if (parts == 0 || rows == 0) return hipSuccess;
    const dim3 grid((unsigned)rows, parts);
    if (a.D == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kF32Threads), 0, s, a);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kF32Threads), 0, s, a);
    return hipGetLastError();
}

}  // namespace ta
