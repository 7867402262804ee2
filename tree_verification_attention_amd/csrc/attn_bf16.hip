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
// 32-column MFMA tile, ~200 registers, so two wavefronts share every SIMD and the hardware
// interleaves one's MFMAs with the other's softmax); a workgroup of NW wavefronts shares every
// K/V tile, so the KV stream is read from HBM once per 32 * NW rows.
//
// Per 64-key tile:
//   HBM -> registers: 16-byte buffer loads whose per-lane offsets never change; the tile's
//     position is a scalar offset, and rows past the end of the sequence read as zeros. The next
//     tile's loads are in flight during the current tile's MFMAs; registers -> LDS (two stages),
//     ordered by an LDS-only barrier.
//   K keeps its [key][d] layout; V is transposed on the way into LDS, to [d][key] with keys
//     permuted inside each 16-key group so that one lane's eight PV k-slots are one contiguous
//     16-byte read. Both rows are padded by 16 bytes, which spreads the 16 lanes of every read
//     and write phase over distinct banks and keeps every operand address a single per-lane base
//     plus an immediate.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16, 32 keys at a time: the keys are the MFMA rows, so
//     every lane holds scores of a single query row -- the layout P^T needs as a B operand. All
//     operand reads of a 32-key block are issued before its MFMA chain.
//   O^T += V^T P^T on the same MFMA.
//   Softmax in fp32 with exp2 (log2(e) folded into the scale). The first tile and the tree tiles
//     take an exact path that moves each row's maximum and rescales what is accumulated; the
//     remaining prefix tiles keep the maximum fixed and never rescale (no per-element maximum,
//     no accumulator traffic). Should a block's exponentials there sum past 2^64 the whole
//     workgroup redoes its part on the exact path.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "ancestors.h"
#include "launch.h"
#include "treeattn.h"

namespace ta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A 32-key block whose exponentials (relative to the fixed maximum) sum past this sends the
// workgroup to the exact path; below it nothing can overflow fp32 or bf16.
constexpr float kSumGuard = 18446744073709551616.0f;  // 2^64

#define TA_INLINE __attribute__((always_inline))

template <int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KT = kKeyTile;
    constexpr int NT = NW * 64;
    constexpr int DCH = D / 8;                      // 16-byte chunks per key row
    constexpr int KN = KT * DCH / NT;               // K chunks per thread per tile
    constexpr int VITEMS = (KT / 2) * DCH;          // (key pair, chunk) items of a V tile
    constexpr int VN = (VITEMS + NT - 1) / NT;      // V items per thread per tile
    constexpr int KS = D / 16;                      // MFMA k-steps over the head dimension
    constexpr int DT = D / 32;                      // 32-row tiles of O^T
    constexpr int KROW = D + 8;                     // padded K row (bf16 elements)
    constexpr int VROW = KT + 8;                    // padded V^T row (bf16 elements)
    constexpr int KTILE = KT * KROW;
    constexpr int STAGE = KTILE + D * VROW;         // bf16 elements of one LDS stage
    constexpr bool DEEP = false;                    // two tiles of loads in flight
    static_assert((KT * DCH) % NT == 0, "K chunks must divide over the threads");
    static_assert(sizeof(AncestorLds) <= 2 * STAGE * 2, "mask scratch must fit the tile LDS");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ uint64_t node_mask[TA_MAX_TREE][kMaskWords];
    __shared__ int32_t page_cache[PAGED ? kPageCache : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    // ---- KV tile staging: HBM -> registers -> LDS.
    // K: thread t moves chunk (t % DCH) of key rows t / DCH + i * NT / DCH.
    // V: item i = t + n * NT is key pair (i % 32) at chunk (i / 32): keys 2*(i%32) and +1.
    // Contiguous prefix and tree tiles use buffer loads: a row past the end of the sequence (or
    // tree) reads as zeros, and rows past the end of the part are masked to -inf; the paged
    // prefix clamps its rows to the part's last row instead.
    const uint32_t prow = 2u * (uint32_t)a.kv_s1, trow = 2u * (uint32_t)a.kt_st;
    const uint64_t ppage = 2ull * (uint64_t)a.kv_s0;
    const char *kc_b = reinterpret_cast<const char *>(a.kc) +
                       2 * ((PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2);
    const char *vc_b = reinterpret_cast<const char *>(a.vc) +
                       2 * ((PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2);
    const char *kt_b = reinterpret_cast<const char *>(a.kt) + 2 * (b * a.kt_sb + g * a.kt_sh);
    const char *vt_b = reinterpret_cast<const char *>(a.vt) + 2 * (b * a.kt_sb + g * a.kt_sh);
    const int seq_len = a.with_prefix ? min(max(a.seq_lens[b], 0), a.capacity) : 0;
    const __amdgpu_buffer_rsrc_t rs_kc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)kc_b, (short)0, PAGED ? 0 : seq_len * (int)prow, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_vc = __builtin_amdgcn_make_buffer_rsrc(
        (void *)vc_b, (short)0, PAGED ? 0 : seq_len * (int)prow, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_kt = __builtin_amdgcn_make_buffer_rsrc(
        (void *)kt_b, (short)0, has_tree ? a.T * (int)trow : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_vt = __builtin_amdgcn_make_buffer_rsrc(
        (void *)vt_b, (short)0, has_tree ? a.T * (int)trow : 0, 0x00020000);

    u32x4 stA_K[KN], stA_V[2 * VN];
    u32x4 stB_K[DEEP ? KN : 1], stB_V[DEEP ? 2 * VN : 1];

    auto load_tile = [&](int t, u32x4 (&sK)[KN], u32x4 (&sV)[2 * VN]) TA_INLINE {
        const bool tree_tile = t >= n_ptiles;
        if (tree_tile || !PAGED) {
            const int k0 = tree_tile ? (t - n_ptiles) * KT : pb + t * KT;
            const uint32_t rowb = tree_tile ? trow : prow;
            const __amdgpu_buffer_rsrc_t rk = tree_tile ? rs_kt : rs_kc;
            const __amdgpu_buffer_rsrc_t rv = tree_tile ? rs_vt : rs_vc;
            const int soff = k0 * (int)rowb;
#pragma unroll
            for (int i = 0; i < KN; ++i) {
                const int c = tid + i * NT;
                sK[i] = __builtin_amdgcn_raw_buffer_load_b128(
                    rk, (int)((c / DCH) * rowb + (c % DCH) * 16u), soff, 0);
            }
#pragma unroll
            for (int n = 0; n < VN; ++n) {
                const int it = min(tid + n * NT, VITEMS - 1);
                const int kp = it & 31, dc = it >> 5;
                sV[2 * n] = __builtin_amdgcn_raw_buffer_load_b128(
                    rv, (int)((2 * kp) * rowb + dc * 16u), soff, 0);
                sV[2 * n + 1] = __builtin_amdgcn_raw_buffer_load_b128(
                    rv, (int)((2 * kp + 1) * rowb + dc * 16u), soff, 0);
            }
        } else {
            const int k0 = pb + t * KT;
            const int last = pe - 1 - k0;
            auto row_addr = [&](const char *base, int row) TA_INLINE -> const char * {
                const int key = k0 + min(row, last);
                const int pg = page_cache[(key >> a.page_shift) - page0];
                return base + (uint64_t)pg * ppage + (uint32_t)(key & a.page_mask) * prow;
            };
#pragma unroll
            for (int i = 0; i < KN; ++i) {
                const int c = tid + i * NT;
                sK[i] = *reinterpret_cast<const u32x4 *>(row_addr(kc_b, c / DCH) + (c % DCH) * 16);
            }
#pragma unroll
            for (int n = 0; n < VN; ++n) {
                const int it = min(tid + n * NT, VITEMS - 1);
                const int kp = it & 31, dc = it >> 5;
                sV[2 * n] = *reinterpret_cast<const u32x4 *>(row_addr(vc_b, 2 * kp) + dc * 16);
                sV[2 * n + 1] = *reinterpret_cast<const u32x4 *>(row_addr(vc_b, 2 * kp + 1) + dc * 16);
            }
        }
    };

    // LDS positions. K: row k, chunk c at k * KROW + 8c. V^T: row d, key k at d * VROW +
    // 8 * (2*(k/16) + (k/4)%2) + 4 * ((k/8)%2) + k%4: the 16-byte block 2*(k/16) + h holds keys
    // 16*(k/16) + 4h + {0..3} and + 8 + {0..3}, the eight k-slots one PV lane consumes.
    auto vt_off = [](int d, int k) TA_INLINE {
        return d * VROW + 8 * (2 * (k >> 4) + ((k >> 2) & 1)) + 4 * ((k >> 3) & 1) + (k & 3);
    };

    auto store_tile = [&](int s, const u32x4 (&sK)[KN], const u32x4 (&sV)[2 * VN]) TA_INLINE {
        uint16_t *Ks = smem + s * STAGE;
        uint16_t *Vs = Ks + KTILE;
#pragma unroll
        for (int i = 0; i < KN; ++i) {
            const int c = tid + i * NT;
            *reinterpret_cast<u32x4 *>(Ks + (c / DCH) * KROW + (c % DCH) * 8) = sK[i];
        }
#pragma unroll
        for (int n = 0; n < VN; ++n) {
            const int it = tid + n * NT;
            if (VITEMS % NT == 0 || it < VITEMS) {
                const int kp = it & 31, dc = it >> 5;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w0 = sV[2 * n][e >> 1], w1 = sV[2 * n + 1][e >> 1];
                    const uint32_t pk = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                                : ((w0 & 0xffffu) | (w1 << 16));
                    *reinterpret_cast<uint32_t *>(Vs + vt_off(dc * 8 + e, 2 * kp)) = pk;
                }
            }
        }
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

    // S^T for one 32-key block (jb): key jb*32 + 8*(r/4) + 4*hf + r%4 in register r. All K
    // fragments are read before the MFMA chain starts, so the LDS latency is paid once.
    auto qk = [&](const uint16_t *Ks, int jb, f32x16 &S) TA_INLINE {
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[ks] = *reinterpret_cast<const bf16x8 *>(Ks + (jb * 32 + l32) * KROW + (2 * ks + hf) * 8);
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qreg[ks], S, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // the KS LDS reads first
        __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);  // then the KS MFMAs
        __builtin_amdgcn_sched_barrier(0);
    };

    // V^T fragments of one 32-key block, read ahead of its exponentials
    auto load_vt = [&](const uint16_t *Vs, int jb, bf16x8 (&vf)[2][DT]) TA_INLINE {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                vf[u][dt] = *reinterpret_cast<const bf16x8 *>(
                    Vs + (dt * 32 + l32) * VROW + 8 * (2 * (2 * jb + u) + hf));
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
        const uint16_t *Ks = smem + s * STAGE;
        const uint16_t *Vs = Ks + KTILE;
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

    // Barrier that orders LDS only: outstanding global loads (the prefetched tiles) stay in
    // flight across it, unlike a full __syncthreads().
    auto lds_barrier = []() TA_INLINE {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    // One pass over every tile of the part. Tile t is staged through LDS stage t % 2; with
    // eight wavefronts its loads are issued two tiles ahead into register set t % 2.
    auto run_pass = [&](bool cold) TA_INLINE -> bool {
        bool bad = false;
        if (n_tiles > 0) {
            load_tile(0, stA_K, stA_V);
            store_tile(0, stA_K, stA_V);
        }
        if constexpr (DEEP) {
            if (n_tiles > 1) load_tile(1, stB_K, stB_V);
            lds_barrier();
            for (int t = 0; t < n_tiles; t += 2) {
                if (t + 2 < n_tiles) load_tile(t + 2, stA_K, stA_V);
                bad |= compute_tile(t, 0, cold);
                if (t + 1 < n_tiles) store_tile(1, stB_K, stB_V);
                lds_barrier();
                if (t + 1 >= n_tiles) break;
                if (t + 3 < n_tiles) load_tile(t + 3, stB_K, stB_V);
                bad |= compute_tile(t + 1, 1, cold);
                if (t + 2 < n_tiles) store_tile(0, stA_K, stA_V);
                lds_barrier();
            }
        } else {
            lds_barrier();
            for (int t = 0; t < n_tiles; ++t) {
                const int s = t & 1;
                if (t + 1 < n_tiles) load_tile(t + 1, stA_K, stA_V);
                bad |= compute_tile(t, s, cold);
                if (t + 1 < n_tiles) store_tile(s ^ 1, stA_K, stA_V);
                lds_barrier();
            }
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
