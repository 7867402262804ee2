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
// R = T * G packed rows, row r = node * G + group member. Each wavefront owns 64 rows (two
// 32-column MFMA tiles); a workgroup of NW wavefronts shares every K/V tile, so the KV stream
// is read from HBM once per 64 * NW rows.
//
// Per 64-key tile:
//   HBM -> registers: 16-byte loads, 16 lanes per 256-byte key row, issued one tile ahead so
//     they are in flight during the current tile's MFMAs; then registers -> LDS (two stages).
//   LDS layout: K and V both keep their natural [key][d] layout. 16-byte chunks are XOR-swizzled
//     (K: chunk ^ key%8, V: chunk ^ 2*(key%4)) so that the MFMA operand reads below touch
//     distinct banks.
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16, 32 keys at a time: the keys are the MFMA rows, so
//     every lane holds scores of a single query row -- the layout P^T needs as a B operand.
//   O^T += V^T P^T on the same MFMA; the V^T operand comes straight from the natural V layout
//     through ds_read_b64_tr_b16 (the gfx950 LDS transpose load).
//   Softmax in fp32 with exp2 (log2(e) folded into the scale). Each row's reference maximum is
//     fixed by the first 32-key block in which the row sees a key and the accumulators are
//     never rescaled on this fast path, so it needs no per-element maximum. Should any block's
//     exponentials sum past 2^64 (scores far above the reference), the whole workgroup redoes
//     its part on an exact path that moves the maximum and rescales as usual. The exponentials
//     of one 32-key block overlap the MFMAs of its neighbour.
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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// A 32-key block whose exponentials (relative to the running maximum) sum past this is redone
// with an exact maximum; below it nothing can overflow fp32 or bf16.
constexpr float kSumGuard = 18446744073709551616.0f;  // 2^64

template <int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KT = kKeyTile;
    constexpr int NT = NW * 64;
    constexpr int DCH = D / 8;                // 16-byte chunks per key row
    constexpr int NLOAD = KT * DCH / NT;      // chunks of K (and of V) per thread per tile
    constexpr int KS = D / 16;                // MFMA k-steps over the head dimension
    constexpr int DT = D / 32;                // 32-row tiles of O^T
    constexpr int TILE = KT * D;              // bf16 elements of one K or V tile
    constexpr int STAGE = 2 * TILE;
    static_assert((KT * DCH) % NT == 0, "tile chunks must divide over the threads");
    static_assert(sizeof(AncestorLds) <= 2 * STAGE * 2, "mask scratch must fit the tile LDS");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
    __shared__ uint64_t node_mask[TA_MAX_TREE][kMaskWords];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, l32 = lane & 31;
    const int part = blockIdx.x;
    const int g = blockIdx.y / a.n_rb, rb = blockIdx.y % a.n_rb;
    const int b = blockIdx.z;
    const int G = a.G, R = a.T * G;
    const int row0 = rb * NT + wave * 64;
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

    const int32_t *btab = PAGED ? a.block_table + (int64_t)b * a.max_blocks : nullptr;
    if (PAGED && n_ptiles > 0 && a.err) {
        const int p0 = pb >> a.page_shift, p1 = (pe - 1) >> a.page_shift;
        for (int pi = p0 + tid; pi <= p1; pi += NT)
            if ((unsigned)btab[pi] >= (unsigned)a.num_pages) atomicOr(a.err, (int32_t)TA_DEV_BAD_PAGE);
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

    // ---- tree masks of every node, kept in LDS
    if (has_tree) {
        AncestorLds &anc = *reinterpret_cast<AncestorLds *>(smem);
        const int cur = build_ancestor_masks(a.parent + (int64_t)b * a.T, a.T, anc, a.err, tid, NT);
        for (int e = tid; e < a.T * kMaskWords; e += NT)
            node_mask[e / kMaskWords][e % kMaskWords] = anc.m[cur][e / kMaskWords][e % kMaskWords];
        __syncthreads();  // the tile stages reuse the scratch
    }

    // ---- KV tile staging: HBM -> registers -> LDS. Thread t moves 16-byte chunk (t % DCH) of
    // key rows t / DCH, t / DCH + NT / DCH, ...; a row past the end of the range loads the last
    // valid row instead (finite data), and its scores are masked to -inf so it adds nothing.
    const __bf16 *kc_bg = reinterpret_cast<const __bf16 *>(a.kc) +
                          (PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2;
    const __bf16 *vc_bg = reinterpret_cast<const __bf16 *>(a.vc) +
                          (PAGED ? 0 : b * a.kv_s0) + g * a.kv_s2;
    const __bf16 *kt_bg = reinterpret_cast<const __bf16 *>(a.kt) + b * a.kt_sb + g * a.kt_sh;
    const __bf16 *vt_bg = reinterpret_cast<const __bf16 *>(a.vt) + b * a.kt_sb + g * a.kt_sh;
    const int pstride = (int)a.kv_s1, tstride = (int)a.kt_st, page_stride = (int)a.kv_s0;
    u32x4 stA_K[NLOAD], stA_V[NLOAD];
    u32x4 stB_K[NW == 4 ? NLOAD : 1], stB_V[NW == 4 ? NLOAD : 1];

    auto load_tile = [&](int t, u32x4 (&stK)[NLOAD], u32x4 (&stV)[NLOAD]) __attribute__((always_inline)) {
        const bool tree_tile = t >= n_ptiles;
        const int k0 = tree_tile ? (t - n_ptiles) * KT : pb + t * KT;
        const int kend = tree_tile ? a.T : pe;
        const __bf16 *kb = tree_tile ? kt_bg : kc_bg;
        const __bf16 *vb = tree_tile ? vt_bg : vc_bg;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int c = tid + i * NT;
            const int row = c / DCH, ch = c % DCH;
            const int kc = min(k0 + row, kend - 1);
            int64_t off;
            if (tree_tile) {
                off = kc * tstride;
            } else if (PAGED) {
                int pg = btab[kc >> a.page_shift];
                pg = (unsigned)pg < (unsigned)a.num_pages ? pg : 0;
                off = (int64_t)pg * page_stride + (kc & a.page_mask) * pstride;
            } else {
                off = kc * pstride;
            }
            stK[i] = *reinterpret_cast<const u32x4 *>(kb + off + ch * 8);
            stV[i] = *reinterpret_cast<const u32x4 *>(vb + off + ch * 8);
        }
    };

    auto store_tile = [&](int s, const u32x4 (&stK)[NLOAD], const u32x4 (&stV)[NLOAD]) __attribute__((always_inline)) {
        uint16_t *Ks = smem + s * STAGE;
        uint16_t *Vs = Ks + TILE;
#pragma unroll
        for (int i = 0; i < NLOAD; ++i) {
            const int c = tid + i * NT;
            const int row = c / DCH, ch = c % DCH;
            *reinterpret_cast<u32x4 *>(Ks + row * D + ((ch ^ (row & 7)) << 3)) = stK[i];
            *reinterpret_cast<u32x4 *>(Vs + row * D + ((ch ^ ((row & 3) << 1)) << 3)) = stV[i];
        }
    };

    // ---- accumulators and softmax state
    f32x16 acc[2][DT];
    float m_run[2], l_run[2];
    auto reset_state = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[qt][dt][r] = 0.f;
            m_run[qt] = -INFINITY;
            l_run[qt] = 0.f;
        }
    };
    const float c2 = a.scale_log2;

    // lane-constant parts of the LDS operand addresses
    const int gi = lane >> 4, li = lane & 15;
    // K A-operand: key l32 of a 32-key block, chunk (2*ks + hf) swizzled by key % 8, which is
    // the same as chunk 2*ks XOR k_xor
    const int k_lane = l32 * D;
    const int k_xor = hf ^ (l32 & 7);
    // V transpose read: this lane sources row key0 + li/4, 4 columns starting at
    // 16*(dt + DT*(gi&1)) + 4*(li&3); lanes of the upper half read keys 4 further on
    const int v_row = li >> 2;
    const int v_hfk = 4 * (gi >> 1);
    const int v_sw = v_row << 1;

    // S^T for one 32-key block (jb) of the stage
    auto qk = [&](const uint16_t *Ks, int jb, f32x16 (&S)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int r = 0; r < 16; ++r) S[qt][r] = 0.f;
        const uint16_t *kp = Ks + jb * 32 * D + k_lane;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8 *>(kp + (((2 * ks) ^ k_xor) << 3));
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
                S[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qt][ks], S[qt], 0, 0, 0);
        }
    };

    // O^T += V^T P^T for one 32-key block
    auto pv = [&](const uint16_t *Vs, int jb, const bf16x8 (&P)[2][2]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int key0 = jb * 32 + u * 16 + v_hfk;  // second key group: key0 + 8
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int col = 16 * (dt + DT * (gi & 1)) + 4 * (li & 3);
                const int chp = (col >> 3) ^ v_sw;
                const uint16_t *p0 = Vs + (key0 + v_row) * D + (chp << 3) + (col & 7);
                const uint16_t *p1 = p0 + 8 * D;
                const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4 *)(p0));
                const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4 *)(p1));
                const i16x8 tv = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
                const bf16x8 va = __builtin_bit_cast(bf16x8, tv);
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    acc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[qt][u], acc[qt][dt],
                                                                          0, 0, 0);
            }
        }
    };

    // Mask the scores of one 32-key block in place. Key of register r: jb*32 + 8*(r/4) + 4*hf
    // + r%4 inside the tile.
    auto mask_block = [&](f32x16 (&S)[2], int t, int jb) __attribute__((always_inline)) {
        if (t >= n_ptiles) {
            const int tt = t - n_ptiles;
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const uint64_t word = node_of[qt] >= 0 ? node_mask[node_of[qt]][tt] : 0ull;
                const uint32_t half = (uint32_t)(word >> (jb * 32 + 4 * hf));
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int bit = 8 * (r >> 2) + (r & 3);
                    if (!((half >> bit) & 1u)) S[qt][r] = -INFINITY;
                }
            }
        } else {
            const int kb = pb + t * KT + jb * 32;
            if (kb + 32 > pe) {
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb + 8 * (r >> 2) + 4 * hf + (r & 3);
                        if (key >= pe) S[qt][r] = -INFINITY;
                    }
            }
        }
    };

    // row maximum of a block (both lane halves), -inf for a fully masked row
    auto block_max = [&](const f32x16 (&S)[2], int qt) __attribute__((always_inline)) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[qt][r]);
        return fmaxf(mx, __shfl_xor(mx, 32));
    };

    // exp2 of one block against the running maximum; adds to the row sums and returns whether
    // any of this lane's block sums left the safe range
    auto exps = [&](const f32x16 (&S)[2], bf16x8 (&P)[2][2]) __attribute__((always_inline)) {
        bool bad = false;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float mb = m_run[qt] == -INFINITY ? 0.f : m_run[qt] * c2;
            float s = 0.f;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[qt][8 * u + e], c2, -mb));
                    s += p;
                    P[qt][u][e] = (__bf16)p;
                }
            l_run[qt] += s;
            bad |= !(s <= kSumGuard);
        }
        return bad;
    };

    // fast path: the reference maximum of a row is set once, by the first block in which the
    // row sees a key; afterwards the accumulators are never rescaled
    auto seed_max = [&](const f32x16 (&S)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float mx = block_max(S, qt);
            if (m_run[qt] == -INFINITY) m_run[qt] = mx;
        }
    };

    // exact path: move the running maximum to cover the block and rescale what is accumulated
    auto exact_max = [&](const f32x16 (&S)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float m_new = fmaxf(m_run[qt], block_max(S, qt));
            if (__any(m_new > m_run[qt])) {
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
        }
    };

    // Barrier that orders LDS only: outstanding global loads (the prefetched tiles) stay in
    // flight across it, unlike a full __syncthreads().
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    // compute one tile from LDS stage s
    auto compute_tile = [&](int t, int s, auto exact_tag) __attribute__((always_inline)) -> bool {
        constexpr bool EXACT = decltype(exact_tag)::value;
        bool bad = false;
        if (!wave_active) return false;
        const uint16_t *Ks = smem + s * STAGE;
        const uint16_t *Vs = Ks + TILE;
        const bool seed = t == 0 || t >= n_ptiles;
        f32x16 S0[2], S1[2];
        bf16x8 P0[2][2], P1[2][2];
        qk(Ks, 0, S0);
        mask_block(S0, t, 0);
        qk(Ks, 1, S1);  // overlaps the exponentials of block 0
        if (EXACT) exact_max(S0);
        else if (seed) seed_max(S0);
        bad |= exps(S0, P0);
        mask_block(S1, t, 1);
        pv(Vs, 0, P0);  // overlaps the exponentials of block 1
        if (EXACT) exact_max(S1);
        else if (seed) seed_max(S1);
        bad |= exps(S1, P1);
        pv(Vs, 1, P1);
        return bad;
    };

    // One pass over every tile of the part; EXACT selects the rescaling path. With four
    // wavefronts, tiles are loaded two ahead into alternating register sets (A, B) and written to
    // alternating LDS stages, so two tiles' worth of loads are in flight while one is computed;
    // smaller workgroups (more chunks per thread) load one tile ahead.
    auto run_pass = [&](auto exact_tag) __attribute__((always_inline)) -> bool {
        bool bad = false;
        if constexpr (NW == 4) {
            if (n_tiles > 0) {
                load_tile(0, stA_K, stA_V);
                store_tile(0, stA_K, stA_V);
            }
            if (n_tiles > 1) load_tile(1, stB_K, stB_V);
            lds_barrier();
            for (int t = 0; t < n_tiles; t += 2) {
                // tile t in stage 0; set B holds tile t + 1
                if (t + 2 < n_tiles) load_tile(t + 2, stA_K, stA_V);
                bad |= compute_tile(t, 0, exact_tag);
                if (t + 1 < n_tiles) store_tile(1, stB_K, stB_V);
                lds_barrier();
                if (t + 1 >= n_tiles) break;
                // tile t + 1 in stage 1; set A holds tile t + 2
                if (t + 3 < n_tiles) load_tile(t + 3, stB_K, stB_V);
                bad |= compute_tile(t + 1, 1, exact_tag);
                if (t + 2 < n_tiles) store_tile(0, stA_K, stA_V);
                lds_barrier();
            }
        } else {
            if (n_tiles > 0) {
                load_tile(0, stA_K, stA_V);
                store_tile(0, stA_K, stA_V);
            }
            lds_barrier();
            for (int t = 0; t < n_tiles; ++t) {
                const int s = t & 1;
                if (t + 1 < n_tiles) load_tile(t + 1, stA_K, stA_V);
                bad |= compute_tile(t, s, exact_tag);
                if (t + 1 < n_tiles) store_tile(s ^ 1, stA_K, stA_V);
                lds_barrier();
            }
        }
        return bad;
    };

    reset_state();
    const bool overflow = run_pass(std::integral_constant<bool, false>{});
    if (__syncthreads_or(overflow)) {
        // some row's exponentials outgrew the fixed reference: redo the part exactly
        reset_state();
        run_pass(std::integral_constant<bool, true>{});
    }

    // ---- normalise and write this part's (O, LSE).
    // O^T row m of d-tile dt holds d = 16*(dt + DT*(m/16)) + m%16 (the V transpose-read order);
    // register r of a lane holds m = 8*(r/4) + 4*hf + r%4.
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
                const int d = 16 * (dt + DT * (q4 >> 1)) + 8 * (q4 & 1) + 4 * hf;
                *reinterpret_cast<float4 *>(op + d) = v;
            }
        if (hf == 0)
            a.out_lse[part * a.part_sl + orow] =
                l_tot > 0.f ? m_run[qt] * a.scale + logf(l_tot) : -INFINITY;
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
