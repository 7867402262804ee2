// bf16 masked attention for tree verification on gfx950 (CDNA4): the speculative part.
//
// The speculative part of LongSpec's Hybrid Tree Attention: every draft-tree node attends to the
// tree's own keys under the ancestor mask -- node i sees node j iff j == i or j is an ancestor
// of i (LongSpec page, "Fast tree attention"; textbook page, tree attention mask). The masks are
// built per workgroup in LDS from the parent array and applied in-register. The same kernel also
// takes the prefix keys that the prefix kernel leaves out (those past the last full 64-key tile,
// in tail mode) and, for direct calls, any prefix chunk: its part covers prefix keys [pb, pe)
// with no mask, then the tree keys.
//
// Layout and streaming are those of the prefix kernel: 32 packed rows (node x GQA group member)
// per wavefront, 64-key tiles of K and V loaded straight into a ring of LDS stages, K in 16-key
// x 4-chunk blocks, V in 4-key x 4-chunk blocks read through ds_read_b64_tr_b16, S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16. Rows past the end of the prefix part (or of the
// tree) are clamped to its last row and masked out of the scores.
//
// Softmax: the first tile and the tree tiles take an exact path that moves each row's maximum
// and rescales what is accumulated; later prefix tiles keep it fixed. Should a block's
// exponentials there sum past 2^64 the whole workgroup redoes its part on the exact path.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ancestors.h"
#include "launch.h"
#include "lds_dma.h"
#include "treeattn.h"

namespace ta {

template <int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void attn_tree_kernel(AttnArgs a) {
    constexpr int KT = kKeyTile;
    constexpr int NT = NW * 64;
    constexpr int DCH = D / 8;                  // 16-byte chunks per key row
    constexpr int CB = DCH / 4;                 // 4-chunk column blocks per key row
    constexpr int KS = D / 16;                  // MFMA k-steps over the head dimension
    constexpr int DT = D / 32;                  // 32-row tiles of O^T
    constexpr int NS = 4;                       // LDS stages in the ring
    constexpr int TILE_B = KT * D * 2;          // bytes of one K (or V) tile
    constexpr int STAGE_B = 2 * TILE_B;
    constexpr int NI = KT * DCH / 64;           // load instructions per K (or V) tile
    constexpr int NIW = 2 * NI / NW;            // load instructions per wavefront per tile
    static_assert((2 * NI) % NW == 0, "tile loads must divide over the wavefronts");
    static_assert(sizeof(AncestorLds) <= NS * STAGE_B, "mask scratch must fit the tile LDS");

    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE_B];
    __shared__ uint64_t node_mask[TA_MAX_TREE][kMaskWords];
    __shared__ int32_t page_cache[PAGED ? kPageCache : 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    const int part = blockIdx.x;
    const int g = blockIdx.y / a.n_rb, rb = blockIdx.y % a.n_rb;
    const int b = blockIdx.z;
    const int G = a.G, R = a.T * G;
    const int row0 = rb * (32 * NW) + wave * 32;
    const bool wave_active = row0 < R;

    // ---- key ranges: prefix chunk, then (last part only) the tree
    int pb = 0, pe = 0;
    if (a.with_prefix) {
        int L = a.seq_lens[b];
        if (L < 0 || L > a.capacity) {
            if (a.err && tid == 0) atomicOr(a.err, (int32_t)TA_DEV_BAD_LEN);
            L = L < 0 ? 0 : a.capacity;
        }
        pb = a.tail_only ? (L & ~(KT - 1)) : part * a.chunk;
        pe = a.tail_only ? L : min(pb + a.chunk, L);
    }
    const int n_ptiles = pe > pb ? (pe - pb + KT - 1) / KT : 0;
    const bool has_tree = a.with_tree && part == a.n_splits - 1;
    const int n_tiles = n_ptiles + (has_tree ? (a.T + KT - 1) / KT : 0);

    // ---- paged layout: this part's block-table entries, validated, cached in LDS
    int page0 = 0;
    if (PAGED && n_ptiles > 0) {
        page0 = pb >> a.page_shift;
        const int np = ((pe - 1) >> a.page_shift) - page0 + 1;  // host keeps np <= kPageCache
        const int32_t *btab = a.block_table + (int64_t)b * a.max_blocks + page0;
        for (int i = tid; i < np; i += NT) {
            int pg = btab[i];
            if ((unsigned)pg >= (unsigned)a.num_pages) {
                if (a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_PAGE);
                pg = 0;
            }
            page_cache[i] = pg;
        }
    }

    // ---- queries of this lane's row, in the MFMA B-operand layout
    bf16x8 qreg[KS];
    int node_of;
    {
        const int r = row0 + l32;
        const bool ok = r < R;
        const int rr = ok ? r : 0;
        const int node = rr / G, h = g * G + rr % G;
        node_of = ok ? node : -1;
        const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + b * a.q_sb + node * a.q_st +
                           h * a.q_sh + hf * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = *reinterpret_cast<const u32x4 *>(qp + ks * 16);
            if (!ok) v = u32x4{0u, 0u, 0u, 0u};
            qreg[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // ---- tree masks of every node, kept in LDS
    if (has_tree) {
        AncestorLds &anc = *reinterpret_cast<AncestorLds *>(smem);
        const int cur = build_ancestor_masks(a.parent + (int64_t)b * a.T, a.T, anc, a.err, tid, NT);
        const int W = (a.T + 63) >> 6;
        for (int e = tid; e < a.T * W; e += NT) node_mask[e / W][e % W] = anc.m[cur][e / W][e % W];
    }
    __syncthreads();  // page cache and masks visible; the tile stages reuse the mask scratch

    // ---- this lane's share of a tile's loads: instruction i of this wavefront is tile-load
    // number j = wave * NIW + i; j < NI fills K block j, otherwise V blocks 4 (j - NI) .. + 3.
    // ld_row / ld_off: key row inside the tile and byte offset inside the row; ld_lds: LDS byte
    // offset of the instruction's 1 KB inside a stage.
    int ld_row[NIW];
    uint32_t ld_off[NIW], ld_lds[NIW];
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
        const int j = wave * NIW + i;
        tile_load_pos<DCH>(j >= NI, j < NI ? j : j - NI, lane, ld_row[i], ld_off[i]);
        ld_lds[i] = j < NI ? 1024u * (uint32_t)j : (uint32_t)TILE_B + 1024u * (uint32_t)(j - NI);
    }
    const uint32_t smem_lds = lds_addr(smem);
    const uint32_t prow = 2u * (uint32_t)a.kv_s1, trow = 2u * (uint32_t)a.kt_st;
    const uint64_t ppage = 2ull * (uint64_t)a.kv_s0;
    const char *kc_b = reinterpret_cast<const char *>(a.kc) +
                       2 * ((PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2);
    const char *vc_b = reinterpret_cast<const char *>(a.vc) +
                       2 * ((PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2);
    const char *kt_b = reinterpret_cast<const char *>(a.kt) + 2 * (b * a.kt_sb + g * a.kt_sh);
    const char *vt_b = reinterpret_cast<const char *>(a.vt) + 2 * (b * a.kt_sb + g * a.kt_sh);

    // Issue tile t's loads into stage t % NS. Rows past the end of the part (or of the tree) are
    // clamped to its last row: they are masked out of the scores, and a clamped row holds finite
    // values, so 0 * V stays 0.
    auto issue_tile = [&](int t) TA_INLINE {
        const uint32_t st = smem_lds + (uint32_t)((t % NS) * STAGE_B);
        const bool tree_tile = t >= n_ptiles;
        if (tree_tile || !PAGED) {
            const int k0 = tree_tile ? (t - n_ptiles) * KT : pb + t * KT;
            const int last = (tree_tile ? a.T : pe) - 1 - k0;
            const uint32_t rowb = tree_tile ? trow : prow;
            const char *kb = (tree_tile ? kt_b : kc_b) + (uint64_t)k0 * rowb;
            const char *vb = (tree_tile ? vt_b : vc_b) + (uint64_t)k0 * rowb;
#pragma unroll
            for (int i = 0; i < NIW; ++i) {
                const uint32_t off = (uint32_t)min(ld_row[i], last) * rowb + ld_off[i];
                const bool is_k = wave * NIW + i < NI;  // uniform per wavefront
                load_lds_saddr(is_k ? kb : vb, off, st + ld_lds[i]);
            }
        } else {
            // Every instruction's rows form one aligned group of at most 16 keys (K: 16, V: 4
            // rows at D = 128, 8 at D = 64), and pages hold a power of two >= 16 keys, so an
            // instruction reads a single page (clamped rows stay inside the group or all land on
            // the last row): the page base is a scalar and the lanes add 32-bit row offsets.
            const int k0 = pb + t * KT;
            const int last = pe - 1 - k0;
#pragma unroll
            for (int i = 0; i < NIW; ++i) {
                const int j = wave * NIW + i;
                const int g0 = tile_load_group<DCH>(j >= NI, j < NI ? j : j - NI);
                const int pkey = k0 + min(g0, last);
                const int pg = __builtin_amdgcn_readfirstlane(page_cache[(pkey >> a.page_shift) - page0]);
                const char *base = (j < NI ? kc_b : vc_b) + (uint64_t)pg * ppage;
                const int key = k0 + min(ld_row[i], last);
                load_lds_saddr(base, (uint32_t)(key & a.page_mask) * prow + ld_off[i], st + ld_lds[i]);
            }
        }
    };

    // wait for this wavefront's loads of tile t, given the tiles issued after it
    auto wait_tile = [&](int t) TA_INLINE {
        const int after = min(NS - 2, n_tiles - 1 - t);
        if (after >= 2) wait_vmem<2 * NIW>();
        else if (after == 1) wait_vmem<NIW>();
        else wait_vmem<0>();
    };

    // ---- accumulators and softmax state
    f32x16 acc[DT];
    float m_run, l_run;
    auto reset_state = [&]() TA_INLINE {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
        m_run = -INFINITY;
        l_run = 0.f;
    };
    const float c2 = a.scale_log2;

    // Operand read bases (bytes inside a stage). K: lane (l32, hf) reads key jb*32 + l32, chunk
    // 2*ks + hf. V: lane (g16 = lane / 16, j = lane % 16) addresses key 4*hf + j/4 (+ 16u + 8v of
    // the block) at d = 16*(g16 % 2) + 4*(j % 4) (+ 32 dt).
    const uint32_t k_rd = (uint32_t)((l32 >> 4) * CB * 1024 + hf * 256 + (l32 & 15) * 16);
    const int jv = lane & 15, g16 = lane >> 4;
    const uint32_t v_rd = (uint32_t)(hf * CB * 256 + (4 * (jv >> 2) + 2 * (g16 & 1) + ((jv & 3) >> 1)) * 16 +
                                     (jv & 1) * 8);

    // S^T for one 32-key block (jb): key jb*32 + 8*(r/4) + 4*hf + r%4 in register r. All K
    // fragments are read before the MFMA chain starts, so the LDS latency is paid once.
    auto qk = [&](const char *Ks, int jb, f32x16 &S) TA_INLINE {
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[ks] = *reinterpret_cast<const bf16x8 *>(Ks + k_rd + jb * 2 * CB * 1024 +
                                                       (ks >> 1) * 1024 + (ks & 1) * 512);
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qreg[ks], S, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // the KS LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);  // then the KS MFMAs
        __builtin_amdgcn_sched_barrier(0);
    };

    // V^T fragments of one 32-key block, read ahead of its exponentials: k-slots 0..3 of a lane
    // are keys 16u + 4hf + 0..3, k-slots 4..7 the same + 8 (the P^T layout of the S^T tile).
    auto load_vt = [&](const char *Vs, int jb, bf16x8 (&vf)[2][DT]) TA_INLINE {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const char *p = Vs + v_rd + (8 * jb + 4 * u) * CB * 256 + dt * 256;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
                const bf16x4 hi =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + 2 * CB * 256));
                vf[u][dt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        __builtin_amdgcn_sched_barrier(0);
    };

    // O^T += V^T P^T for one 32-key block
    auto pv = [&](const bf16x8 (&vf)[2][DT], const bf16x8 (&P)[2]) TA_INLINE {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u][dt], P[u], acc[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // mask a block's scores: keys past the prefix end, or tree keys that are not ancestors
    auto mask_block = [&](f32x16 &S, int t, int jb) TA_INLINE {
        if (t >= n_ptiles) {
            const uint64_t word = node_of >= 0 ? node_mask[node_of][t - n_ptiles] : 0ull;
            const uint32_t bits = (uint32_t)(word >> (jb * 32 + 4 * hf));
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (!((bits >> (8 * (r >> 2) + (r & 3))) & 1u)) S[r] = -INFINITY;
        } else {
            const int kb = pb + t * KT + jb * 32;
            if (kb + 32 > pe) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kb + 8 * (r >> 2) + 4 * hf + (r & 3) >= pe) S[r] = -INFINITY;
            }
        }
    };

    // fast path: exponentials against the fixed maximum; returns whether the block's sum left
    // the safe range
    auto exps_fast = [&](const f32x16 &S, bf16x8 (&P)[2]) TA_INLINE -> bool {
        const float mb = m_run * c2;
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * u + e], c2, -mb));
                s += p;
                P[u][e] = (__bf16)p;
            }
        l_run += s;
        return !(s <= kSumGuard);
    };

    // exact path: move the maximum to cover the block (rescaling what is accumulated) first
    auto exps_exact = [&](const f32x16 &S, bf16x8 (&P)[2]) TA_INLINE {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run)) {
            const float alpha =
                m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
            m_run = m_new;
        }
        const float mb = m_run == -INFINITY ? 0.f : m_run * c2;
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * u + e], c2, -mb));
                s += p;
                P[u][e] = (__bf16)p;
            }
        l_run += s;
    };

    // compute one tile from LDS stage s, one 32-key block at a time (the other wavefront on the
    // SIMD fills the MFMA and VALU gaps)
    auto compute_tile = [&](int t, int s, bool cold) TA_INLINE -> bool {
        bool bad = false;
        if (!wave_active) return false;
        const char *Ks = smem + s * STAGE_B;
        const char *Vs = Ks + TILE_B;
        const bool exact = cold || t == 0 || t >= n_ptiles;
        if (!exact && pb + (t + 1) * KT <= pe) {
            // the hot path: a full prefix tile
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x16 S;
                bf16x8 P[2], vf[2][DT];
                qk(Ks, jb, S);
                load_vt(Vs, jb, vf);
                bad |= exps_fast(S, P);
                pv(vf, P);
            }
        } else {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                f32x16 S;
                bf16x8 P[2], vf[2][DT];
                qk(Ks, jb, S);
                load_vt(Vs, jb, vf);
                mask_block(S, t, jb);
                if (exact) exps_exact(S, P);
                else bad |= exps_fast(S, P);
                pv(vf, P);
            }
        }
        return bad;
    };

    // One pass over every tile of the part. At the top of iteration t the barrier publishes
    // tile t (every wavefront has waited for its own loads of it) and retires tile t - 1, whose
    // stage then takes the loads of tile t + NS - 1.
    auto run_pass = [&](bool cold) TA_INLINE -> bool {
        bool bad = false;
#pragma unroll
        for (int t = 0; t < NS - 1; ++t)
            if (t < n_tiles) issue_tile(t);
        for (int t = 0; t < n_tiles; ++t) {
            wait_tile(t);
            lds_barrier();
            if (t + NS - 1 < n_tiles) issue_tile(t + NS - 1);
            bad |= compute_tile(t, t % NS, cold);
        }
        return bad;
    };

    reset_state();
    const bool overflow = run_pass(false);
    if (__syncthreads_or(overflow)) {
        // some row's exponentials outgrew its fixed maximum: redo the part exactly
        reset_state();
        run_pass(true);
    }

    // ---- normalise and write this part's (O, LSE); register r of O^T tile dt holds
    // d = dt*32 + 8*(r/4) + 4*hf + r%4
    const int r = row0 + l32;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (r < R) {
        const int node = r / G, h = g * G + r % G;
        const int64_t orow = ((int64_t)b * a.T + node) * a.Hq + h;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float *op = a.out_o + part * a.part_so + orow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float4 v;
                v.x = acc[dt][4 * q4 + 0] * inv;
                v.y = acc[dt][4 * q4 + 1] * inv;
                v.z = acc[dt][4 * q4 + 2] * inv;
                v.w = acc[dt][4 * q4 + 3] * inv;
                *reinterpret_cast<float4 *>(op + dt * 32 + 8 * q4 + 4 * hf) = v;
            }
        if (hf == 0)
            a.out_lse[part * a.part_sl + orow] =
                l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
    }
}

hipError_t launch_attn_tree(const AttnArgs &a, int nw, hipStream_t s) {
    if (a.n_splits == 0 || a.B == 0) return hipSuccess;
    const dim3 grid(a.n_splits, a.Hkv * a.n_rb, a.B);
#define TA_LAUNCH(DD, NN)                                                                        \
    do {                                                                                         \
        if (a.block_table)                                                                       \
            hipLaunchKernelGGL((attn_tree_kernel<DD, NN, true>), grid, dim3(NN * 64), 0, s, a);  \
        else                                                                                     \
            hipLaunchKernelGGL((attn_tree_kernel<DD, NN, false>), grid, dim3(NN * 64), 0, s, a); \
    } while (0)
    if (a.D == 128) {
        if (nw == 2) TA_LAUNCH(128, 2);
        else if (nw == 4) TA_LAUNCH(128, 4);
        else TA_LAUNCH(128, 8);
    } else {
        if (nw == 2) TA_LAUNCH(64, 2);
        else if (nw == 4) TA_LAUNCH(64, 4);
        else TA_LAUNCH(64, 8);
    }
#undef TA_LAUNCH
    return hipGetLastError();
}

}  // namespace ta
