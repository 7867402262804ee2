// bf16 split-KV attention kernel for tree verification on gfx950 (CDNA4).
//
// One workgroup handles one (part, kv-head, row block, sequence). A part is either a chunk of
// the committed prefix (no mask) or the draft tree's own keys (ancestor mask). This is the
// divide step of LongSpec's Hybrid Tree Attention (LongSpec page, "Fast tree attention": the
// cache part needs no mask, only the few speculative tokens do); the prefix is further divided
// along its length so that the chip stays busy, and every part is later combined by the same
// log-sum-exp identity (merge kernel).
//
// Query packing. The G = Hq / Hkv query heads that share a KV head and the T tree nodes form
// R = T * G packed rows, row r = node * G + group member. Each wavefront owns 64 rows (two
// 32-row MFMA column tiles); a workgroup of NW wavefronts shares every K/V tile, so the KV
// stream is read once from HBM per 64 * NW rows.
//
// Per 64-key tile:
//   HBM -> registers: 16-byte loads, 16 lanes per 256-byte key row (D = 128), issued one tile
//     ahead of the compute so the next tile's loads are in flight during the current MFMAs.
//   registers -> LDS (two stages): K keeps its [key][d] layout, V is transposed into [d][key];
//     rows are padded (16 B for K, 8 B for V^T) so that neither the writes nor the MFMA-operand
//     reads of 16 consecutive lanes share a bank.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the keys are the MFMA rows, so every lane ends up
//     holding 32 scores of a single query row -- exactly the operand layout P^T needs next.
//   online softmax in fp32 with exp2 (log2(e) folded into the scale); the running maximum is
//     only moved (and the accumulators rescaled) when it grows by more than 2^8 in exp2 terms,
//     which keeps every exp2 argument below 8 and so cannot overflow.
//   O^T += V^T P^T on the same MFMA, with P rounded to bf16 by the hardware converter.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ancestors.h"
#include "launch.h"
#include "treeattn.h"

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Largest growth of the running maximum (in exp2 units) that is absorbed without rescaling.
constexpr float kRescaleThreshold = 8.0f;

enum { kModeContig = 0, kModePaged = 1, kModeTree = 2 };

// One part (prefix chunk or tree) of one (kv-head, row block, sequence).
template <int D, int NW, int MODE>
__device__ __forceinline__ void attn_part(const AttnArgs &a, uint16_t *smem,
                                          uint64_t (*node_mask)[kMaskWords]) {
    constexpr int KT = kKeyTile;
    constexpr int NT = NW * 64;
    constexpr int DC = D / 8;                 // 16-byte chunks per key row
    constexpr int NGRP_TOTAL = (KT / 4) * DC; // (4 keys x 8 dims) groups per tile
    constexpr int NGRP = (NGRP_TOTAL + NT - 1) / NT;
    constexpr int KS = D / 16;                // MFMA k-steps over the head dimension
    constexpr int DT = D / 32;                // 32-row tiles of O^T
    constexpr int KROW = D + 8;               // padded K row (bf16): 16 B shift per row
    constexpr int VROW = KT + 4;              // padded V^T row (bf16): 8 B shift per row
    constexpr int KSTAGE = KT * KROW;
    constexpr int STAGE = KSTAGE + D * VROW;  // bf16 elements per LDS stage
    constexpr bool TREE = MODE == kModeTree;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, l32 = lane & 31;
    const int part = blockIdx.x;
    const int g = blockIdx.y / a.n_rb, rb = blockIdx.y % a.n_rb;
    const int b = blockIdx.z;
    const int G = a.G, R = a.T * G;
    const int row0 = rb * NT + wave * 64;
    const bool wave_active = row0 < R;

    int k_begin, k_end;
    if (TREE) {
        k_begin = 0;
        k_end = a.T;
    } else {
        int L = a.seq_lens[b];
        if (L < 0 || L > a.capacity) {
            if (a.err && tid == 0) atomicOr(a.err, (int32_t)TA_DEV_BAD_LEN);
            L = L < 0 ? 0 : a.capacity;
        }
        k_begin = part * a.chunk;
        k_end = min(k_begin + a.chunk, L);
    }
    const int n_tiles = k_end > k_begin ? (k_end - k_begin + KT - 1) / KT : 0;
    const int32_t *btab = nullptr;
    if (MODE == kModePaged) {
        btab = a.block_table + (int64_t)b * a.max_blocks;
        // every page this chunk reads must exist; bad entries are reported here and read as page 0
        if (n_tiles > 0 && a.err) {
            const int p0 = k_begin >> a.page_shift, p1 = (k_end - 1) >> a.page_shift;
            for (int pi = p0 + tid; pi <= p1; pi += NT)
                if ((unsigned)btab[pi] >= (unsigned)a.num_pages) atomicOr(a.err, (int32_t)TA_DEV_BAD_PAGE);
        }
    }

    // ---- queries of this lane's two 32-row tiles, in the MFMA B-operand layout
    bf16x8 qreg[2][KS];
    int node_of[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int r = row0 + qt * 32 + l32;
        const bool ok = r < R;
        const int rr = ok ? r : 0;
        const int node = rr / G, h = g * G + rr % G;
        node_of[qt] = ok ? node : -1;
        const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + b * a.q_sb + node * a.q_st +
                           h * a.q_sh + hf * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = *reinterpret_cast<const u32x4 *>(qp + ks * 16);
            if (!ok) v = u32x4{0u, 0u, 0u, 0u};
            qreg[qt][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- tree part: ancestor-or-self masks of every node, kept in LDS
    if (TREE) {
        AncestorLds &anc = *reinterpret_cast<AncestorLds *>(smem);
        const int cur = build_ancestor_masks(a.parent + (int64_t)b * a.T, a.T, anc, a.err, tid, NT);
        for (int e = tid; e < a.T * kMaskWords; e += NT)
            node_mask[e / kMaskWords][e % kMaskWords] = anc.m[cur][e / kMaskWords][e % kMaskWords];
        __syncthreads();  // the tile stages reuse the scratch
    }

    // ---- KV tile staging: HBM -> registers -> LDS.
    // K: 16 lanes cover one key row chunk by chunk (contiguous 256-byte rows at D = 128).
    // V: 16 lanes cover 16 different 4-key groups at one 8-dim chunk, so that the transposed
    //    LDS writes of those lanes land in one V^T row.
    // Keys past the end of the part are read from a valid row and replaced by zeros.
    const __bf16 *kbase = reinterpret_cast<const __bf16 *>(TREE ? a.kt : a.kc);
    const __bf16 *vbase = reinterpret_cast<const __bf16 *>(TREE ? a.vt : a.vc);
    u32x4 stK[NGRP][4], stV[NGRP][4];

    // Row offsets are 32-bit relative to a per-(sequence, kv-head) base; the host guarantees
    // that every row of a sequence (or of the page pool row within a page) fits.
    const __bf16 *kseq, *vseq;
    if (TREE) {
        kseq = kbase + b * a.kt_sb + g * a.kt_sh;
        vseq = vbase + b * a.kt_sb + g * a.kt_sh;
    } else if (MODE == kModePaged) {
        kseq = kbase + g * a.kv_s2;
        vseq = vbase + g * a.kv_s2;
    } else {
        kseq = kbase + b * a.kv_s0 + g * a.kv_s2;
        vseq = vbase + b * a.kv_s0 + g * a.kv_s2;
    }
    const int row_stride = (int)(TREE ? a.kt_st : a.kv_s1);
    auto key_offset = [&](int j) -> int64_t {
        const int jc = min(j, k_end - 1);
        if (MODE == kModePaged) {
            int pg = btab[jc >> a.page_shift];
            pg = (unsigned)pg < (unsigned)a.num_pages ? pg : 0;
            return (int64_t)pg * (int32_t)a.kv_s0 + (jc & a.page_mask) * row_stride;
        }
        return jc * row_stride;
    };

    auto load_tile = [&](int t) {
        const int kb = k_begin + t * KT;
#pragma unroll
        for (int gi = 0; gi < NGRP; ++gi) {
            const int idx = min(tid + gi * NT, NGRP_TOTAL - 1);
            const int kqa = idx / DC, dca = idx % DC;   // K mapping
            const int kqb = idx % 16, dcb = idx / 16;   // V mapping
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ja = kb + kqa * 4 + e, jb = kb + kqb * 4 + e;
                u32x4 kv = *reinterpret_cast<const u32x4 *>(kseq + key_offset(ja) + dca * 8);
                u32x4 vv = *reinterpret_cast<const u32x4 *>(vseq + key_offset(jb) + dcb * 8);
                if (ja >= k_end) kv = u32x4{0u, 0u, 0u, 0u};
                if (jb >= k_end) vv = u32x4{0u, 0u, 0u, 0u};
                stK[gi][e] = kv;
                stV[gi][e] = vv;
            }
        }
    };

    auto store_tile = [&](int s) {
        uint16_t *Ks = smem + s * STAGE;
        uint16_t *Vs = Ks + KSTAGE;
#pragma unroll
        for (int gi = 0; gi < NGRP; ++gi) {
            const int idx = tid + gi * NT;
            if (NGRP_TOTAL % NT == 0 || idx < NGRP_TOTAL) {
                const int kqa = idx / DC, dca = idx % DC;
                const int kqb = idx % 16, dcb = idx / 16;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    *reinterpret_cast<u32x4 *>(Ks + (kqa * 4 + e) * KROW + dca * 8) = stK[gi][e];
                // transpose 4 keys x 8 dims into 8 rows of V^T (4 keys each)
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    const int w = e2 >> 1, sh = (e2 & 1) * 16;
                    const uint32_t k0 = (stV[gi][0][w] >> sh) & 0xffffu;
                    const uint32_t k1 = (stV[gi][1][w] >> sh) & 0xffffu;
                    const uint32_t k2 = (stV[gi][2][w] >> sh) & 0xffffu;
                    const uint32_t k3 = (stV[gi][3][w] >> sh) & 0xffffu;
                    u32x2 pk = {k0 | (k1 << 16), k2 | (k3 << 16)};
                    *reinterpret_cast<u32x2 *>(Vs + (dcb * 8 + e2) * VROW + kqb * 4) = pk;
                }
            }
        }
    };

    // ---- accumulators
    f32x16 acc[2][DT];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qt][dt][r] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    const float c2 = a.scale_log2;

    auto compute_tile = [&](int s, int t) {
        const uint16_t *Ks = smem + s * STAGE;
        const uint16_t *Vs = Ks + KSTAGE;
        // S^T tiles: [key tile kt][query tile qt], keys are MFMA rows
        f32x16 S[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int r = 0; r < 16; ++r) S[kt][qt][r] = 0.f;
        const uint16_t *kp = Ks + l32 * KROW + hf * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kp + kt * 32 * KROW + ks * 16);
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    S[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qt][ks], S[kt][qt],
                                                                        0, 0, 0);
            }
        }
        // masking: key index inside the tile of register r is kt*32 + 8*(r/4) + 4*hf + r%4
        const int kb = k_begin + t * KT;
        if (TREE) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const uint64_t word = node_of[qt] >= 0 ? node_mask[node_of[qt]][t] : 0ull;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (!((word >> key) & 1ull)) S[kt][qt][r] = -INFINITY;
                    }
            }
        } else if (kb + KT > k_end) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb + kt * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (key >= k_end) S[kt][qt][r] = -INFINITY;
                    }
        }
        // online softmax statistics, per query tile
        float mb[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kt][qt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[qt], mx);
            const bool grow = (m_new - m_run[qt]) * c2 > kRescaleThreshold;  // false for NaN
            if (__any(grow)) {
                const float alpha = m_run[qt] == -INFINITY
                                        ? 0.f
                                        : __builtin_amdgcn_exp2f((m_run[qt] - m_new) * c2);
                l_run[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[qt][dt][r] *= alpha;
                m_run[qt] = m_new;
            }
            mb[qt] = m_run[qt] == -INFINITY ? 0.f : m_run[qt] * c2;
        }
        // P = exp2(S*c2 - m) in bf16, then O^T += V^T P^T, 16 keys at a time
        const uint16_t *vp = Vs + l32 * VROW + hf * 4;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                bf16x8 P[2];
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    float lsum = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float p = __builtin_amdgcn_exp2f(S[kt][qt][8 * u + e] * c2 - mb[qt]);
                        lsum += p;
                        P[qt][e] = (__bf16)p;
                    }
                    l_run[qt] += lsum;
                }
                const int key0 = kt * 32 + u * 16;  // keys key0 + 4*hf + {0..3, 8..11}
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const uint16_t *vr = vp + dt * 32 * VROW + key0;
                    const u32x2 x1 = *reinterpret_cast<const u32x2 *>(vr);
                    const u32x2 x2 = *reinterpret_cast<const u32x2 *>(vr + 8);
                    const u32x4 xv = {x1[0], x1[1], x2[0], x2[1]};
                    const bf16x8 va = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        acc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[qt], acc[qt][dt],
                                                                              0, 0, 0);
                }
            }
    };

    // ---- main loop: one barrier per tile, next tile's loads in flight during the compute
    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
        const int s = t & 1;
        if (t + 1 < n_tiles) load_tile(t + 1);
        if (wave_active) compute_tile(s, t);
        if (t + 1 < n_tiles) store_tile(s ^ 1);
        __syncthreads();
    }

    // ---- normalise and write this part's (O, LSE)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int r = row0 + qt * 32 + l32;
        const float l_tot = l_run[qt] + __shfl_xor(l_run[qt], 32);
        if (r >= R) continue;
        const int node = r / G, h = g * G + r % G;
        const int64_t orow = ((int64_t)b * a.T + node) * a.Hq + h;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *op = a.out_o + part * a.part_so + orow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float4 v;
                v.x = acc[qt][dt][4 * q4 + 0] * inv;
                v.y = acc[qt][dt][4 * q4 + 1] * inv;
                v.z = acc[qt][dt][4 * q4 + 2] * inv;
                v.w = acc[qt][dt][4 * q4 + 3] * inv;
                *reinterpret_cast<float4 *>(op + dt * 32 + 8 * q4 + 4 * hf) = v;
            }
        if (hf == 0)
            a.out_lse[part * a.part_sl + orow] =
                l_tot > 0.f ? m_run[qt] * a.scale + logf(l_tot) : -INFINITY;
    }
}

template <int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnArgs a) {
    constexpr int STAGE = kKeyTile * (D + 8) + D * (kKeyTile + 4);
    static_assert(sizeof(AncestorLds) <= 2 * STAGE * 2, "mask scratch must fit the tile LDS");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ uint64_t node_mask[TA_MAX_TREE][kMaskWords];
    if (a.with_tree && (int)blockIdx.x == a.n_splits)
        attn_part<D, NW, kModeTree>(a, smem, node_mask);
    else
        attn_part<D, NW, PAGED ? kModePaged : kModeContig>(a, smem, node_mask);
}

hipError_t launch_attn_bf16(const AttnArgs &a, int nw, hipStream_t s) {
    const int parts = a.n_splits + (a.with_tree ? 1 : 0);
    if (parts == 0 || a.B == 0) return hipSuccess;
    const dim3 grid(parts, a.Hkv * a.n_rb, a.B);
#define TA_LAUNCH(DD, NN)                                                                   \
    do {                                                                                     \
        if (a.block_table)                                                                   \
            hipLaunchKernelGGL((attn_bf16_kernel<DD, NN, true>), grid, dim3(NN * 64), 0, s, a);  \
        else                                                                                 \
            hipLaunchKernelGGL((attn_bf16_kernel<DD, NN, false>), grid, dim3(NN * 64), 0, s, a); \
    } while (0)
    if (a.D == 128) {
        if (nw == 1) TA_LAUNCH(128, 1);
        else if (nw == 2) TA_LAUNCH(128, 2);
        else TA_LAUNCH(128, 4);
    } else {
        if (nw == 1) TA_LAUNCH(64, 1);
        else if (nw == 2) TA_LAUNCH(64, 2);
        else TA_LAUNCH(64, 4);
    }
#undef TA_LAUNCH
    return hipGetLastError();
}

}  // namespace ta
