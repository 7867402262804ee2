// bf16 split-KV attention kernel for tree verification on gfx950 (CDNA4).
//
// One workgroup handles one (part, kv-head, row block, sequence). Part p covers one chunk of the
// committed prefix with no mask; the last part also covers the draft tree's own keys under the
// ancestor mask. This is the divide step of LongSpec's Hybrid Tree Attention (LongSpec page,
// "Fast tree attention": the cache part needs no mask, only the few speculative tokens do); the
// prefix is further divided along its length so that every compute unit streams its own slice,
// and the parts are combined afterwards by the same log-sum-exp identity (merge kernel).
//
// Query packing. The G = Hq / Hkv query heads that share a KV head and the T tree nodes form
// R = T * G packed rows, row r = node * G + group member. Each wavefront owns 32 rows (one
// 32-column MFMA tile, so two wavefronts share every SIMD and the hardware interleaves one's
// MFMAs with the other's softmax); a workgroup of NW wavefronts shares every K/V tile, so the KV
// stream is read from HBM once per 32 * NW rows.
//
// KV streaming. 64-key tiles of K and V go from HBM straight into LDS with direct-to-LDS loads
// (each instruction moves 16 bytes per lane into 1 KB of consecutive LDS), through a ring of NS
// stages: while a tile is computed, the next NS - 1 tiles are in flight, with no registers held
// for them. The loads are issued from inline assembly and their completion is awaited with
// explicit vector-memory counter waits, one tile at a time; the compiler would otherwise wait
// for every outstanding LDS load before any LDS read.
//
// LDS layouts (16-byte chunk = 8 bf16 of one key row):
//   K: blocks of 16 keys x 4 chunks, chunk-major inside the block. One load instruction fills
//      one block from 16 rows x 64 contiguous bytes; the QK operand read of 16 lanes (16
//      consecutive keys, one chunk) is 256 consecutive bytes.
//   V: blocks of 4 keys x 4 chunks, key-major inside the block. One load instruction fills four
//      blocks from 4 whole key rows. The PV operand V^T comes from the transposing LDS read
//      (ds_read_b64_tr_b16): 16 lanes that each address 4 d-values of one key return to every
//      lane 4 keys of one d; the 32 lanes of a half-wave touch one block's 16 chunks once each.
//   Every operand address is one per-lane base plus an immediate.
//
// Per 32-key block: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys are the MFMA rows, so every
// lane holds scores of a single query row -- the layout P^T needs as a B operand), softmax in
// fp32 with exp2 (log2(e) folded into the scale), O^T += V^T P^T on the same MFMA. The first tile
// and the tree tiles take an exact path that moves each row's maximum and rescales what is
// accumulated; the remaining prefix tiles keep the maximum fixed and never rescale. Should a
// block's exponentials there sum past 2^64 the whole workgroup redoes its part on the exact path.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ancestors.h"
#include "launch.h"
#include "treeattn.h"

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// A 32-key block whose exponentials (relative to the fixed maximum) sum past this sends the
// workgroup to the exact path; below it nothing can overflow fp32 or bf16.
constexpr float kSumGuard = 18446744073709551616.0f;  // 2^64

#define TA_INLINE __attribute__((always_inline))

// Wait until at most N vector-memory operations of this wavefront are outstanding.
template <int N>
__device__ TA_INLINE void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// LDS byte address of a shared-memory pointer (the value a load-to-LDS instruction takes in M0).
__device__ TA_INLINE uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 16 bytes per lane from saddr + voff into LDS at m0 + 16 * lane. The compiler does not insert
// wait states for what an inline-assembly load reads, so the s_nop supplies them: five after a
// VALU write of an SGPR the load reads (saddr may come from v_readfirstlane), one after an SALU
// write of M0.
__device__ TA_INLINE void load_lds_saddr(const void *saddr, uint32_t voff, uint32_t m0) {
    const uint64_t p = (uint64_t)(uintptr_t)saddr;
    const uint64_t u = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p) |
                       ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32);
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(u), "{m0}"(m0) : "memory");
}

template <int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnArgs a) {
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
        pb = part * a.chunk;
        pe = min(pb + a.chunk, L);
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
        for (int e = tid; e < a.T * kMaskWords; e += NT)
            node_mask[e / kMaskWords][e % kMaskWords] = anc.m[cur][e / kMaskWords][e % kMaskWords];
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
        if (j < NI) {
            const int ri = j / CB, ci = j % CB;
            ld_row[i] = 16 * ri + (lane & 15);
            ld_off[i] = 16u * (uint32_t)(4 * ci + (lane >> 4));
            ld_lds[i] = 1024u * (uint32_t)j;
        } else {
            const int jv = j - NI;
            const int blk = 4 * jv + (lane >> 4);
            const int ka = blk / CB, cb = blk % CB;
            ld_row[i] = 4 * ka + ((lane >> 2) & 3);
            ld_off[i] = 16u * (uint32_t)(4 * cb + (lane & 3));
            ld_lds[i] = (uint32_t)TILE_B + 1024u * (uint32_t)jv;
        }
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
                const int g0 = j < NI ? 16 * (j / CB) : 4 * ((4 * (j - NI)) / CB);  // group's first row
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

    // Barrier that orders LDS only (the loads in flight are tracked by wait_tile).
    auto lds_barrier = []() TA_INLINE {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

hipError_t launch_attn_bf16(const AttnArgs &a, int nw, hipStream_t s) {
    if (a.n_splits == 0 || a.B == 0) return hipSuccess;
    const dim3 grid(a.n_splits, a.Hkv * a.n_rb, a.B);
#define TA_LAUNCH(DD, NN)                                                                        \
    do {                                                                                         \
        if (a.block_table)                                                                       \
            hipLaunchKernelGGL((attn_bf16_kernel<DD, NN, true>), grid, dim3(NN * 64), 0, s, a);  \
        else                                                                                     \
            hipLaunchKernelGGL((attn_bf16_kernel<DD, NN, false>), grid, dim3(NN * 64), 0, s, a); \
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
