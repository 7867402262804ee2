// bf16 prefix attention for tree verification on gfx950 (CDNA4): the cache part.
//
// The cache part of LongSpec's Hybrid Tree Attention needs no mask: every draft-tree node sees
// the whole committed prefix of its sequence (LongSpec page, "Fast tree attention"). This kernel
// computes it over the prefix's full 64-key tiles, split along the prefix so that every compute
// unit streams its own slice. The keys past the last full tile (fewer than 64) and the tree's
// own keys form the masked part, which the last split's workgroups -- sized a few tiles short for
// it -- take after their prefix tiles, under the ancestor-or-self mask built in LDS (the tree
// alone, for tree_attn_tree, is the same part with no prefix). All parts are combined afterwards
// by the log-sum-exp identity of the same section (merge kernel). The prefix loop itself holds
// no mask, no ragged tile and no tree: nothing but the streaming and the two products.
//
// One workgroup handles one (part, kv-head, row block, sequence). Query packing: the G = Hq / Hkv
// query heads sharing a KV head and the T tree nodes form R = T * G rows, row = node * G + group
// member; each wavefront owns 32 rows (one 32-column MFMA tile), and the NW wavefronts of a
// workgroup share every K/V tile, so the KV stream is read from HBM once per 32 * NW rows.
//
// KV streaming: 64-key tiles of K and V go from HBM straight into LDS (direct-to-LDS loads, 16
// bytes per lane into 1 KB of consecutive LDS per instruction) through a ring of NS stages; while
// a tile is computed the next NS - 1 are in flight. K is laid out in 16-key x 4-chunk blocks
// (conflict-free QK operand reads), V in 4-key x 4-chunk blocks that the transposing LDS read
// ds_read_b64_tr_b16 turns into the PV operand V^T. Every operand address is a per-lane base
// plus an immediate.
//
// Per 32-key block: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys are the MFMA rows, so a lane
// holds scores of one query row -- the layout P^T needs as a B operand), exponentials in fp32
// with exp2 (log2(e) folded into the scale), O^T += V^T P^T on the same MFMA.
//
// Softmax reference: each row's maximum over the part's first 32 keys, fixed for the whole
// part, so nothing is ever rescaled. Should a block's exponentials sum past 2^64 (or be NaN), the
// workgroup redoes its part in two passes: the rows' exact maxima, then the values against them,
// where no exponential exceeds 1.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ancestors.h"
#include "launch.h"
#include "lds_dma.h"
#include "treeattn.h"

namespace ta {

__device__ TA_INLINE int64_t wave_sum64(int64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ TA_INLINE int64_t wave_max64(int64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (int64_t)__shfl_xor(v, o));
    return v;
}

// exclusive prefix sum over the 64 lanes of a wavefront
__device__ TA_INLINE int wave_exclusive_sum(int v) {
    const int lane = threadIdx.x & 63;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x - v;
}

template <int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void attn_prefix_kernel(AttnArgs a) {
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

    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE_B];
    __shared__ int32_t page_cache[PAGED ? kPageCache : 1];
    __shared__ uint64_t node_mask[TA_MAX_TREE][kMaskWords];  // masked part only
    constexpr int SCR = (int)((sizeof(AncestorLds) + STAGE_B - 1) / STAGE_B);  // mask scratch stages
    static_assert(SCR < NS, "mask scratch must leave a stage for the tiles");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, l32 = lane & 31;
    // XCD-aware order: consecutive workgroups go to the eight XCDs in turn (each with its own
    // L2). With several row blocks the logical order hands every XCD a contiguous range in which
    // the row blocks of one (part, KV head, sequence) -- which stream the same K/V tiles -- are
    // neighbours; with one row block the hardware order is kept (spreading every sequence over
    // all XCDs streams faster there)
    int wg_x, wg_z, g, rb;
    {
        const int n = gridDim.x * gridDim.y * gridDim.z;
        int w = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
        if (a.n_rb > 1 && (n & 7) == 0) w = (w & 7) * (n >> 3) + (w >> 3);
        rb = w % a.n_rb;
        w /= a.n_rb;
        wg_x = w % gridDim.x;
        w /= gridDim.x;
        g = w % a.Hkv;
        wg_z = w / a.Hkv;
    }
    const int G = a.G, R = a.T * G;
    const int row0 = (rb * NW + wave) * 32;
    const bool wave_active = row0 < R;
    const bool first_wg = wg_x == 0 && g == 0 && rb == 0 && wg_z == 0;

    // ---- which sequence, which of its parts, and the part's keys [pb, pe) (full tiles only).
    // Without a prefix, or with one split: sequence wg_z, part wg_x. With several
    // splits and at most 64 sequences the B * n_splits workgroups of this (kv head, row block)
    // are dealt to the sequences by their work -- full prefix tiles plus the masked part's
    // reserve -- so that a ragged batch is not paced by its longest sequence: every sequence
    // first gets the parts its block-table entries need (paged) or one, the rest go out in
    // proportion to the work, and leftovers one at a time to the sequence with the most work
    // per part; a sequence gets at most 2 n_splits parts. With more sequences every one gets
    // n_splits parts of a chunk sized from the longest prefix. Either way the cache capacity
    // plays no part, so a cache allocated longer than what it holds leaves no split idle.
    __shared__ int deal[5];  // sequence (-1: no part for this workgroup), part, chunk, length, parts
    __shared__ int len_max[NW];
    int b = wg_z, part = wg_x, chunk = a.chunk, L = 0, n_parts = a.n_splits;
    const bool several = a.with_prefix && a.n_splits > 1;
    if (several && a.B <= 64) {
        if (wave == 0) {
            const bool on = lane < a.B;
            int lb = on ? a.seq_lens[lane] : 0;
            if (lb < 0 || lb > a.capacity) {
                if (a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_LEN);
                lb = lb < 0 ? 0 : a.capacity;
            }
            const int64_t full = lb & ~(KT - 1);
            const int64_t work = on ? full + a.reserve : 0;
            // paged: a part's block-table entries must fit the LDS cache, so no part spans more
            // than `most` keys (the host's split count already covers any length with such parts)
            const int64_t most =
                PAGED ? (((int64_t)(kPageCache - 2) << a.page_shift) & ~(int64_t)(KT - 1)) : 0;
            const int cap = 2 * a.n_splits;
            int nb = on ? (PAGED ? (int)max((int64_t)1, (full + most - 1) / most) : 1) : 0;
            const int64_t n_wg = (int64_t)a.n_splits * a.B;
            const int64_t total = wave_sum64(work);
            const int64_t rest = n_wg - wave_sum64(nb);
            if (on && total > 0) nb = min(cap, nb + (int)(rest * work / total));
            for (int it = 0; it < 8; ++it) {
                if (wave_sum64(nb) >= n_wg) break;
                // (work per part, lane) packed so that the maximum prefers the lower lane on ties
                const int64_t key = on && nb < cap ? ((work / nb) << 8) | (63 - lane) : -1;
                if (key == wave_max64(key) && key >= 0) ++nb;
            }
            int64_t cb = on ? ((work + nb - 1) / nb + KT - 1) & ~(int64_t)(KT - 1) : 0;
            if (PAGED) cb = min(cb, most);
            const int off = wave_exclusive_sum(nb);
            const int wid = wg_z * a.n_splits + wg_x;
            if (lane == 0) deal[0] = -1;
            if (on && wid >= off && wid < off + nb) {
                deal[0] = lane;
                deal[1] = wid - off;
                deal[2] = (int)min(cb, (int64_t)INT32_MAX);
                deal[3] = lb;
                deal[4] = nb;
            }
            if (first_wg && on && a.seq_parts) a.seq_parts[lane] = nb;
        }
        __syncthreads();
        b = __builtin_amdgcn_readfirstlane(deal[0]);
        if (b < 0) return;  // more workgroups than parts: none for this one
        part = __builtin_amdgcn_readfirstlane(deal[1]);
        chunk = __builtin_amdgcn_readfirstlane(deal[2]);
        L = __builtin_amdgcn_readfirstlane(deal[3]);
        n_parts = __builtin_amdgcn_readfirstlane(deal[4]);
    } else {
        L = a.with_prefix ? a.seq_lens[b] : 0;
        if (L < 0 || L > a.capacity) {
            if (a.err && tid == 0) atomicOr(a.err, (int32_t)TA_DEV_BAD_LEN);
            L = L < 0 ? 0 : a.capacity;
        }
        if (first_wg && a.with_prefix && a.seq_parts)
            for (int i = tid; i < a.B; i += NT) a.seq_parts[i] = a.n_splits;
        if (several) {
            int mx = 0;
            for (int i = tid; i < a.B; i += NT) mx = max(mx, min(max(a.seq_lens[i], 0), a.capacity));
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
            if (lane == 0) len_max[wave] = mx;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < NW; ++w) mx = max(mx, len_max[w]);
            const int64_t c = ((int64_t)mx + a.reserve + a.n_splits - 1) / a.n_splits;
            // the same in every lane: keep it scalar, as the loop bounds below must be
            chunk = __builtin_amdgcn_readfirstlane(
                (int)min((int64_t)chunk, max((int64_t)KT, (c + KT - 1) & ~(int64_t)(KT - 1))));
        }
    }
    const int pb = part * chunk;
    const int pe = min(pb + chunk, L & ~(KT - 1));
    const int n_tiles = pe > pb ? (pe - pb) / KT : 0;

    // ---- paged layout: this part's block-table entries, validated, cached in LDS
    int page0 = 0;
    if (PAGED && n_tiles > 0) {
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
    {
        const int r = row0 + l32;
        const bool ok = r < R;
        const int rr = ok ? r : 0;
        const int node = rr / G, h = g * G + rr % G;
        const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) + b * a.q_sb + node * a.q_st +
                           h * a.q_sh + hf * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = *reinterpret_cast<const u32x4 *>(qp + ks * 16);
            if (!ok) v = u32x4{0u, 0u, 0u, 0u};
            qreg[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    __syncthreads();  // page cache visible

    // ---- this wavefront's loads: instruction i is tile-load j = wave * NIW + i (K block j for
    // j < NI, V blocks of instruction j - NI otherwise); ld_voff is the lane's byte offset from the
    // tile's first key row.
    const uint32_t prow = 2u * (uint32_t)a.kv_s1;
    const uint64_t ppage = 2ull * (uint64_t)a.kv_s0;
    uint32_t ld_voff[NIW];
    int ld_group[NIW];      // paged: first key (in the tile) of the instruction's aligned group
    int64_t ld_pofs[NIW];   // paged, pages below 64 keys: byte offset of the group's page start
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
        const int j = wave * NIW + i;
        int row;
        uint32_t off;
        tile_load_pos<DCH>(j >= NI, j < NI ? j : j - NI, lane, row, off);
        ld_voff[i] = (uint32_t)row * prow + off;
        ld_group[i] = tile_load_group<DCH>(j >= NI, j < NI ? j : j - NI);
        ld_pofs[i] = PAGED ? (int64_t)((ld_group[i] & a.page_mask) - ld_group[i]) * prow : 0;
    }
    auto ld_lds = [&](int i) TA_INLINE -> uint32_t {  // LDS offset of the instruction's 1 KB
        const int j = wave * NIW + i;
        return j < NI ? 1024u * (uint32_t)j : (uint32_t)TILE_B + 1024u * (uint32_t)(j - NI);
    };
    const uint32_t smem_lds = lds_addr(smem);
    const char *kc_b = reinterpret_cast<const char *>(a.kc) +
                       2 * ((PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2);
    const char *vc_b = reinterpret_cast<const char *>(a.vc) +
                       2 * ((PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2);

    // Issue tile t's loads into stage t % NS. Paged: an instruction's rows are one aligned group
    // of at most 16 keys, which one page holds, so its base is the page (a scalar) shifted back
    // by the group's offset in the tile.
    auto issue_tile = [&](int t) TA_INLINE {
        const uint32_t st = smem_lds + (uint32_t)((t % NS) * STAGE_B);
        const int k0 = pb + t * KT;
        if (!PAGED) {
            const char *kb = kc_b + (uint64_t)k0 * prow;
            const char *vb = vc_b + (uint64_t)k0 * prow;
#pragma unroll
            for (int i = 0; i < NIW; ++i)
                load_lds_saddr(wave * NIW + i < NI ? kb : vb, ld_voff[i], st + ld_lds(i));
        } else if (a.page_shift >= 6) {
            // pages of 64 keys or more hold whole tiles: one block-table entry per tile
            const int pg = __builtin_amdgcn_readfirstlane(page_cache[(k0 >> a.page_shift) - page0]);
            const uint64_t off =
                (uint64_t)(uint32_t)pg * ppage + (uint64_t)(uint32_t)(k0 & a.page_mask) * prow;
            const char *kb = kc_b + off;
            const char *vb = vc_b + off;
#pragma unroll
            for (int i = 0; i < NIW; ++i)
                load_lds_saddr(wave * NIW + i < NI ? kb : vb, ld_voff[i], st + ld_lds(i));
        } else {
            // 16- or 32-key pages: one entry per instruction, all read before the first load; the
            // tile starts a page, so an instruction's rows sit at a fixed offset in theirs
            int pgs[NIW];
#pragma unroll
            for (int i = 0; i < NIW; ++i)
                pgs[i] = page_cache[((k0 + ld_group[i]) >> a.page_shift) - page0];
#pragma unroll
            for (int i = 0; i < NIW; ++i) {
                const int pg = __builtin_amdgcn_readfirstlane(pgs[i]);
                const char *base = (wave * NIW + i < NI ? kc_b : vc_b) +
                                   (uint64_t)(uint32_t)pg * ppage + ld_pofs[i];
                load_lds_saddr(base, ld_voff[i], st + ld_lds(i));
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
    float m_run = -INFINITY, l_run = 0.f;
    auto reset_acc = [&]() TA_INLINE {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
        l_run = 0.f;
    };
    const float c2 = a.scale_log2;

    // Operand read bases (bytes inside a stage). K: lane (l32, hf) reads key jb*32 + l32, chunk
    // 2*ks + hf. V: lane (g16 = lane / 16, j = lane % 16) addresses key 4*hf + j/4 (+ 16u + 8v of
    // the block) at d = 16*(g16 % 2) + 4*(j % 4) (+ 32 dt).
    const uint32_t k_rd = (uint32_t)((l32 >> 4) * CB * 1024 + hf * 256 + (l32 & 15) * 16);
    const int jv = lane & 15, g16 = lane >> 4;
    const uint32_t v_rd = (uint32_t)(hf * CB * 256 +
                                     (4 * (jv >> 2) + 2 * (g16 & 1) + ((jv & 3) >> 1)) * 16 + (jv & 1) * 8);

    // S^T for one 32-key block: key jb*32 + 8*(r/4) + 4*hf + r%4 in register r. All K fragments
    // are read before the MFMA chain starts, so the LDS latency is paid once.
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

    // V^T fragments of one 32-key block: k-slots 0..3 of a lane are keys 16u + 4hf + 0..3,
    // k-slots 4..7 the same + 8 (the P^T layout of the S^T tile).
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

    // exponentials against the fixed reference; returns whether the block's sum left the safe
    // range (or is NaN)
    auto exps = [&](const f32x16 &S, bf16x8 (&P)[2]) TA_INLINE -> bool {
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

    // row maximum over blocks 0 .. nblk - 1 of a tile (both lane halves hold parts of the row)
    auto raise_max = [&](const char *Ks, int nblk) TA_INLINE {
        for (int jb = 0; jb < nblk; ++jb) {
            f32x16 S;
            qk(Ks, jb, S);
            float mx = S[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
            m_run = fmaxf(m_run, fmaxf(mx, __shfl_xor(mx, 32)));
        }
    };

    auto tile = [&](const char *Ks, const char *Vs) TA_INLINE -> bool {
        bool bad = false;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f32x16 S;
            bf16x8 P[2], vf[2][DT];
            qk(Ks, jb, S);
            load_vt(Vs, jb, vf);
            bad |= exps(S, P);
            pv(vf, P);
        }
        return bad;
    };

    // mode 0: reference from the part's first block, then values; 1: exact maxima only;
    // 2: values against the exact maxima. At the top of iteration t the barrier publishes tile t
    // (every wavefront has waited for its own loads of it) and retires tile t - 1, whose stage
    // then takes the loads of tile t + NS - 1.
    auto run_pass = [&](int mode) TA_INLINE -> bool {
        bool bad = false;
#pragma unroll
        for (int t = 0; t < NS - 1; ++t)
            if (t < n_tiles) issue_tile(t);
        for (int t = 0; t < n_tiles; ++t) {
            wait_tile(t);
            lds_barrier();
            if (t + NS - 1 < n_tiles) issue_tile(t + NS - 1);
            if (!wave_active) continue;
            const char *Ks = smem + (t % NS) * STAGE_B;
            if (mode == 1) {
                raise_max(Ks, 2);
                continue;
            }
            if (mode == 0 && t == 0) raise_max(Ks, 1);
            bad |= tile(Ks, Ks + TILE_B);
        }
        return bad;
    };

    // The passes are written out one after another (not as a loop over the mode), so that the
    // compiler keeps no state of one pass alive through another.
    reset_acc();
    if (__syncthreads_or(run_pass(0))) {
        m_run = -INFINITY;
        reset_acc();
        run_pass(1);
        __syncthreads();
        run_pass(2);
    }

    // ---- normalise and write a part's (O, LSE); register r of O^T tile dt holds
    // d = dt*32 + 8*(r/4) + 4*hf + r%4
    const int r = row0 + l32;
    auto write_part = [&](float *out_o, float *out_lse) TA_INLINE {
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        if (r < R) {
            const int node = r / G, h = g * G + r % G;
            const int64_t orow = ((int64_t)b * a.T + node) * a.Hq + h;
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            float *op = out_o + orow * D + 4 * hf;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float4 v;
                    v.x = acc[dt][4 * q4 + 0] * inv;
                    v.y = acc[dt][4 * q4 + 1] * inv;
                    v.z = acc[dt][4 * q4 + 2] * inv;
                    v.w = acc[dt][4 * q4 + 3] * inv;
                    *reinterpret_cast<float4 *>(op + dt * 32 + 8 * q4) = v;
                }
            if (hf == 0) out_lse[orow] = l_tot > 0.f ? m_run * a.scale + logf(l_tot) : -INFINITY;
        }
    };
    if (a.with_prefix) write_part(a.out_o + part * a.part_so, a.out_lse + part * a.part_sl);

    // ---- the masked part: the last split (the shortest, or empty for short sequences) goes on
    // with the prefix keys past the last full tile and, with the tree, the tree's own keys under
    // the ancestor-or-self mask (LongSpec page, "Fast tree attention"), into out_o_m / out_lse_m.
    // Every masked tile takes the exact path: the running maximum moves to cover each block and
    // what is accumulated is rescaled.
    if (part != n_parts - 1 || !(a.with_prefix || a.with_tree)) return;
    __syncthreads();  // every wavefront is done with the ring
    const int tb = L & ~(KT - 1);  // the tail: prefix keys [tb, L)
    const int n_tail = L > tb ? 1 : 0;
    const int n_mt = n_tail + (a.with_tree ? (a.T + KT - 1) / KT : 0);
    int tpage0 = 0;
    if (PAGED && n_tail) {
        tpage0 = tb >> a.page_shift;
        const int np = ((L - 1) >> a.page_shift) - tpage0 + 1;
        const int32_t *btab = a.block_table + (int64_t)b * a.max_blocks + tpage0;
        for (int i = tid; i < np; i += NT) {
            int pg = btab[i];
            if ((unsigned)pg >= (unsigned)a.num_pages) {
                if (a.err) atomicOr(a.err, (int32_t)TA_DEV_BAD_PAGE);
                pg = 0;
            }
            page_cache[i] = pg;
        }
        __syncthreads();
    }
    const uint32_t trow = 2u * (uint32_t)a.kt_st;
    const char *kt_b = reinterpret_cast<const char *>(a.kt) + 2 * (b * a.kt_sb + g * a.kt_sh);
    const char *vt_b = reinterpret_cast<const char *>(a.vt) + 2 * (b * a.kt_sb + g * a.kt_sh);

    // masked tile t (the tail first, if any, then the tree tiles) into stage st; rows past the
    // tail (or the tree) are clamped to its last row and masked out of the scores. The three
    // sources are separate branches (uniform per tile), not selects between their pointers.
    auto issue_masked = [&](int t, int st) TA_INLINE {
        const uint32_t sb = smem_lds + (uint32_t)(st * STAGE_B);
        if (t >= n_tail) {
            const int k0 = (t - n_tail) * KT;
            const int last = a.T - 1 - k0;
            const char *kb = kt_b + (uint64_t)k0 * trow;
            const char *vb = vt_b + (uint64_t)k0 * trow;
#pragma unroll
            for (int i = 0; i < NIW; ++i) {
                const int j = wave * NIW + i;
                int row;
                uint32_t off;
                tile_load_pos<DCH>(j >= NI, j < NI ? j : j - NI, lane, row, off);
                load_lds_saddr(j < NI ? kb : vb, (uint32_t)min(row, last) * trow + off, sb + ld_lds(i));
            }
        } else if (!PAGED) {
            const int last = L - 1 - tb;
            const char *kb = kc_b + (uint64_t)tb * prow;
            const char *vb = vc_b + (uint64_t)tb * prow;
#pragma unroll
            for (int i = 0; i < NIW; ++i) {
                const int j = wave * NIW + i;
                int row;
                uint32_t off;
                tile_load_pos<DCH>(j >= NI, j < NI ? j : j - NI, lane, row, off);
                load_lds_saddr(j < NI ? kb : vb, (uint32_t)min(row, last) * prow + off, sb + ld_lds(i));
            }
        } else {
            // one aligned group of at most 16 keys per instruction: a single page
            const int last = L - 1 - tb;
#pragma unroll
            for (int i = 0; i < NIW; ++i) {
                const int j = wave * NIW + i;
                int row;
                uint32_t off;
                tile_load_pos<DCH>(j >= NI, j < NI ? j : j - NI, lane, row, off);
                const int g0 = tile_load_group<DCH>(j >= NI, j < NI ? j : j - NI);
                const int pkey = tb + min(g0, last);
                const int pg = __builtin_amdgcn_readfirstlane(page_cache[(pkey >> a.page_shift) - tpage0]);
                const char *base = (j < NI ? kc_b : vc_b) + (uint64_t)pg * ppage;
                const int key = tb + min(row, last);
                load_lds_saddr(base, (uint32_t)(key & a.page_mask) * prow + off, sb + ld_lds(i));
            }
        }
    };

    // the first tiles go to stages 0 .. NS - SCR - 1 while the masks are built in the last SCR
    // stages; tile k always lives in stage k % NS
    int issued = 0;
    for (; issued < min(n_mt, NS - SCR); ++issued) issue_masked(issued, issued);
    if (a.with_tree) {
        AncestorLds &anc = *reinterpret_cast<AncestorLds *>(smem + (NS - SCR) * STAGE_B);
        const int cur = build_ancestor_masks(a.parent + (int64_t)b * a.T, a.T, anc, a.err, tid, NT);
        const int W = (a.T + 63) >> 6;
        for (int e = tid; e < a.T * W; e += NT) node_mask[e / W][e % W] = anc.m[cur][e / W][e % W];
    }
    wait_vmem<0>();   // the prefetched tiles have landed
    __syncthreads();  // masks and tiles visible; the scratch stages are free for the ring

    const int node_of = r < R ? r / G : -1;
    auto mask_masked = [&](f32x16 &S, int t, int jb) TA_INLINE {
        if (t >= n_tail) {
            const uint64_t word = node_of >= 0 ? node_mask[node_of][t - n_tail] : 0ull;
            const uint32_t bits = (uint32_t)(word >> (jb * 32 + 4 * hf));
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (!((bits >> (8 * (q >> 2) + (q & 3))) & 1u)) S[q] = -INFINITY;
        } else {
            const int kb = tb + jb * 32;
            if (kb + 32 > L) {
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (kb + 8 * (q >> 2) + 4 * hf + (q & 3) >= L) S[q] = -INFINITY;
            }
        }
    };
    auto exps_exact = [&](const f32x16 &S, bf16x8 (&P)[2]) TA_INLINE {
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < 16; ++q) mx = fmaxf(mx, S[q]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run)) {
            const float alpha =
                m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[dt][q] *= alpha;
            m_run = m_new;
        }
        const float mb = m_run == -INFINITY ? 0.f : m_run * c2;
        float sum = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe_ = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * u + e], c2, -mb));
                sum += pe_;
                P[u][e] = (__bf16)pe_;
            }
        l_run += sum;
    };

    reset_acc();
    m_run = -INFINITY;
    for (int t = 0; t < n_mt; ++t) {
        const int after = min(NS - 2, n_mt - 1 - t);
        if (after >= 2) wait_vmem<2 * NIW>();
        else if (after == 1) wait_vmem<NIW>();
        else wait_vmem<0>();
        lds_barrier();
        for (; issued < min(n_mt, t + NS); ++issued) issue_masked(issued, issued % NS);
        if (!wave_active) continue;
        const char *Ks = smem + (t % NS) * STAGE_B;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            f32x16 S;
            bf16x8 P[2], vf[2][DT];
            qk(Ks, jb, S);
            load_vt(Ks + TILE_B, jb, vf);
            mask_masked(S, t, jb);
            exps_exact(S, P);
            pv(vf, P);
        }
    }
    write_part(a.out_o_m, a.out_lse_m);
}

hipError_t launch_attn_prefix(const AttnArgs &a, int nw, hipStream_t s) {
    if (a.n_splits == 0 || a.B == 0) return hipSuccess;
    const dim3 grid(a.n_splits, a.Hkv * a.n_rb, a.B);
#define TA_LAUNCH(DD, NN)                                                                          \
    do {                                                                                           \
        if (a.block_table)                                                                         \
            hipLaunchKernelGGL((attn_prefix_kernel<DD, NN, true>), grid, dim3(NN * 64), 0, s, a);  \
        else                                                                                       \
            hipLaunchKernelGGL((attn_prefix_kernel<DD, NN, false>), grid, dim3(NN * 64), 0, s, a); \
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
