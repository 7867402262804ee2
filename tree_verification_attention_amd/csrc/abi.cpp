// C ABI of the tree-verification attention library: argument checks, the split plan, workspace
// layout and kernel launches. Every entry point only enqueues work on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "launch.h"
#include "treeattn.h"

namespace {

using ta::AttnArgs;
using ta::MergeArgs;

constexpr int kAbiVersion = 100;
// Workgroups the prefix launch aims for per compute unit (the bf16 kernel's 4-stage LDS ring of
// K/V tiles leaves room for one workgroup per CU at D = 128).
constexpr int kWgPerCu = 1;

// Workspace slots per row: 2 n_splits for the prefix parts (a sequence gets at most that many
// when the parts are dealt by length, n_splits otherwise), then the masked part (the tree keys
// and the prefix keys past the last full 64-key tile) in the last slot.
struct Plan {
    int nw = 1;        // wavefronts per workgroup (bf16 kernels)
    int n_rb = 1;      // row blocks per (b, kv-head)
    int n_splits = 1;  // prefix splits
    int chunk = ta::kKeyTile;
    int reserve = 0;   // keys' worth of time the last split keeps for the masked part
    int capacity = 0;  // prefix rows addressable per sequence
    int64_t rows = 0;  // B * T * Hq
    int slots = 2;     // partial slots per row: 2 n_splits prefix parts, then the masked part
    size_t o_bytes = 0, lse_bytes = 0, cnt_bytes = 0;  // workspace regions
};

// The workspace of one problem: partial O [slots][rows][D], partial LSE [slots][rows], and the
// prefix part count of every sequence [B].
struct Workspace {
    float *o, *lse;
    int32_t *parts;
};

Workspace views(const Plan &pl, const void *ws) {
    char *w = static_cast<char *>(const_cast<void *>(ws));
    return Workspace{reinterpret_cast<float *>(w), reinterpret_cast<float *>(w + pl.o_bytes),
                     reinterpret_cast<int32_t *>(w + pl.o_bytes + pl.lse_bytes)};
}

bool ws_ok(const Plan &pl, const void *ws, size_t ws_bytes) {
    return ws && ((uintptr_t)ws & 255u) == 0 && ws_bytes >= pl.o_bytes + pl.lse_bytes + pl.cnt_bytes;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bool stride_ok(int64_t s, int elem) { return s >= 0 && ((s * elem) % 16) == 0; }

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

int elem_size(int dtype) { return dtype == TA_BF16 ? 2 : 4; }

// Shape-level checks shared by every attention entry point.
int check_shape(const ta_problem *p) {
    if (!p) return TA_EINVAL;
    if (p->dtype != TA_BF16 && p->dtype != TA_F32) return TA_EUNSUPPORTED;
    if (p->D != 64 && p->D != 128) return TA_EUNSUPPORTED;
    if (p->B < 0 || p->B > 65535 || p->T < 1 || p->T > TA_MAX_TREE) return TA_EINVAL;
    if (p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv || p->Hkv > 4096) return TA_EINVAL;
    if (!(p->scale > 0.f) || !isfinite(p->scale)) return TA_EINVAL;
    if (p->num_splits < 0) return TA_EINVAL;
    // the paged parameters feed the split plan of every entry point (the capacity
    // max_blocks * page_size, the page shift), tree-only calls included
    if (p->block_table) {
        const int ps = p->page_size;
        if (ps < 16 || ps > (1 << 30) || (ps & (ps - 1)) || p->max_blocks < 1 || p->num_pages < 1)
            return TA_EINVAL;
        if ((int64_t)p->max_blocks * ps > INT32_MAX) return TA_EINVAL;
    }
    if (p->B == 0) return TA_OK;
    const int es = elem_size(p->dtype);
    if (!p->q || !aligned16(p->q)) return TA_EINVAL;
    if (!stride_ok(p->q_sb, es) || !stride_ok(p->q_st, es) || !stride_ok(p->q_sh, es))
        return TA_EINVAL;
    return TA_OK;
}

int check_prefix(const ta_problem *p) {
    if (p->B == 0) return TA_OK;
    const int es = elem_size(p->dtype);
    if (!p->seq_lens) return TA_EINVAL;
    if (!stride_ok(p->kv_s0, es) || !stride_ok(p->kv_s1, es) || !stride_ok(p->kv_s2, es))
        return TA_EINVAL;
    if (!p->block_table && p->Lmax < 0) {
        return TA_EINVAL;
    }
    if (!p->k_cache || !p->v_cache || !aligned16(p->k_cache) || !aligned16(p->v_cache))
        return TA_EINVAL;
    // the kernels address rows with 32-bit byte offsets from a 64-bit base per 64-key tile
    // (contiguous) or per page (paged)
    const int64_t rows = p->block_table ? p->page_size : ta::kKeyTile;
    if ((rows * p->kv_s1 + p->D) * es > INT32_MAX) return TA_EINVAL;
    if (p->block_table && p->kv_s0 > INT32_MAX) return TA_EINVAL;
    return TA_OK;
}

int check_tree(const ta_problem *p) {
    if (p->B == 0) return TA_OK;
    const int es = elem_size(p->dtype);
    if (!p->parent || !p->k_tree || !p->v_tree) return TA_EINVAL;
    if (!aligned16(p->k_tree) || !aligned16(p->v_tree)) return TA_EINVAL;
    if (!stride_ok(p->kt_sb, es) || !stride_ok(p->kt_st, es) || !stride_ok(p->kt_sh, es))
        return TA_EINVAL;
    if (((int64_t)p->T * p->kt_st + p->D) * es > INT32_MAX) return TA_EINVAL;
    return TA_OK;
}

// log2 of a power of two in [1, 2^30] (check_shape admits no other page size)
int ilog2(int x) {
    int s = 0;
    while (s < 30 && (1 << s) < x) ++s;
    return s;
}

Plan make_plan(const ta_problem *p) {
    Plan pl;
    const int G = p->Hq / p->Hkv;
    const int R = p->T * G;
    pl.capacity = p->block_table ? (int)((int64_t)p->max_blocks * p->page_size) : p->Lmax;
    if (pl.capacity < 0) pl.capacity = 0;
    pl.rows = (int64_t)p->B * p->T * p->Hq;
    int64_t wg_per_split;
    if (p->dtype == TA_BF16) {
        // workgroups of 2, 4 or 8 wavefronts, 32 packed rows each
        const int rb_rows = 8 * ta::kRowsPerWave;
        pl.n_rb = (R + rb_rows - 1) / rb_rows;
        const int nw = (R + ta::kRowsPerWave * pl.n_rb - 1) / (ta::kRowsPerWave * pl.n_rb);
        pl.nw = nw <= 2 ? 2 : nw <= 4 ? 4 : 8;
        wg_per_split = (int64_t)p->B * p->Hkv * pl.n_rb;
    } else {
        wg_per_split = pl.rows;
    }
    int n = p->num_splits;
    if (n == 0) {
        const int64_t target = (int64_t)kWgPerCu * cu_count();
        const int64_t per = wg_per_split > 0 ? wg_per_split : 1;
        // bf16: round down, so that the launch never needs a second round of workgroups (with
        // 24 workgroups per split, 10 splits take 368 us on the long-reasoning layer, 11 take
        // 421 us: 8 workgroups wait for a free CU); fp32 workgroups are small, several share a CU
        int64_t want = p->dtype == TA_BF16 ? target / per : (target + per - 1) / per;
        const int64_t most = (pl.capacity + 255) / 256;
        if (want > most) want = most;
        n = want < 1 ? 1 : (int)want;
    }
    // bf16: the last split also runs the masked part (the tail tile, the tree tiles and the
    // mask build, about ceil(T / 64) + 2 tiles of time), so unless the caller fixed the split
    // count the chunks are sized as if the prefix were that much longer, which leaves the last
    // split correspondingly short
    const int64_t reserve = p->dtype == TA_BF16 && p->num_splits == 0
                                ? (int64_t)ta::kKeyTile * ((p->T + ta::kKeyTile - 1) / ta::kKeyTile + 2)
                                : 0;
    pl.reserve = (int)reserve;
    int64_t chunk = pl.capacity > 0 ? ((int64_t)pl.capacity + reserve + n - 1) / n : 1;
    chunk = (chunk + ta::kKeyTile - 1) / ta::kKeyTile * ta::kKeyTile;
    if (p->block_table && p->dtype == TA_BF16) {
        // a part's block-table entries are cached in LDS (kPageCache of them)
        const int64_t most = (int64_t)(ta::kPageCache - 2) * p->page_size;
        if (chunk > most) chunk = most / ta::kKeyTile * ta::kKeyTile;
    }
    pl.chunk = (int)chunk;
    pl.n_splits = pl.capacity > 0 ? (int)((pl.capacity + chunk - 1) / chunk) : 1;
    pl.slots = 2 * pl.n_splits + 1;
    pl.o_bytes = align256((size_t)pl.slots * pl.rows * p->D * sizeof(float));
    pl.lse_bytes = align256((size_t)pl.slots * pl.rows * sizeof(float));
    pl.cnt_bytes = align256((size_t)p->B * sizeof(int32_t));
    return pl;
}

AttnArgs make_args(const ta_problem *p, const Plan &pl, int32_t *err) {
    AttnArgs a{};
    a.q = p->q;
    a.q_sb = p->q_sb;
    a.q_st = p->q_st;
    a.q_sh = p->q_sh;
    a.kc = p->k_cache;
    a.vc = p->v_cache;
    a.kv_s0 = p->kv_s0;
    a.kv_s1 = p->kv_s1;
    a.kv_s2 = p->kv_s2;
    a.seq_lens = p->seq_lens;
    a.block_table = p->block_table;
    a.max_blocks = p->max_blocks;
    a.page_shift = p->block_table ? ilog2(p->page_size) : 0;
    a.page_mask = p->block_table ? p->page_size - 1 : 0;
    a.num_pages = p->num_pages;
    a.capacity = pl.capacity;
    a.kt = p->k_tree;
    a.vt = p->v_tree;
    a.kt_sb = p->kt_sb;
    a.kt_st = p->kt_st;
    a.kt_sh = p->kt_sh;
    a.parent = p->parent;
    a.B = p->B;
    a.T = p->T;
    a.Hq = p->Hq;
    a.Hkv = p->Hkv;
    a.G = p->Hq / p->Hkv;
    a.D = p->D;
    a.chunk = pl.chunk;
    a.reserve = pl.reserve;
    a.n_rb = pl.n_rb;
    a.scale = p->scale;
    a.scale_log2 = p->scale * 1.4426950408889634f;
    a.err = err;
    return a;
}

int status(hipError_t e) { return e == hipSuccess ? TA_OK : TA_EHIP; }

// The prefix parts of every sequence into the workspace slots, their counts into w.parts. bf16:
// the parts take the full 64-key tiles, and each sequence's last part goes on, in the same
// launch, with the masked part into the last slot -- the prefix keys past the last full tile
// and, with ``tree``, the tree keys. fp32: n_splits parts of every prefix key; the tree is a
// launch of its own (launch_tree_part).
int launch_prefix_parts(const ta_problem *p, const Plan &pl, int32_t *err, const Workspace &w,
                        bool tree, hipStream_t s) {
    AttnArgs a = make_args(p, pl, err);
    a.n_splits = pl.n_splits;
    a.with_prefix = 1;
    a.out_o = w.o;
    a.out_lse = w.lse;
    a.part_so = pl.rows * p->D;
    a.part_sl = pl.rows;
    a.seq_parts = w.parts;
    if (p->dtype != TA_BF16) return status(ta::launch_attn_f32(a, s));
    a.with_tree = tree;
    a.out_o_m = w.o + (int64_t)(pl.slots - 1) * a.part_so;
    a.out_lse_m = w.lse + (int64_t)(pl.slots - 1) * a.part_sl;
    return status(ta::launch_attn_prefix(a, pl.nw, s));
}

// The masked tree part alone into (o, l): the bf16 prefix kernel with no prefix (its one split's
// workgroups take only the masked part), or the fp32 kernel over the tree keys.
int launch_tree_part(const ta_problem *p, const Plan &pl, int32_t *err, float *o, float *l,
                     hipStream_t s) {
    AttnArgs a = make_args(p, pl, err);
    a.n_splits = 1;
    a.with_prefix = 0;
    a.with_tree = 1;
    if (p->dtype != TA_BF16) {
        a.out_o = o;
        a.out_lse = l;
        return status(ta::launch_attn_f32(a, s));
    }
    a.out_o_m = o;
    a.out_lse_m = l;
    // little work and no prefix: 64 rows per workgroup (two wavefronts) spread the mask builds
    // and the latency over more compute units
    a.n_rb = (p->T * (p->Hq / p->Hkv) + 63) / 64;
    return status(ta::launch_attn_prefix(a, 2, s));
}

}  // namespace

extern "C" {

int tree_attn_abi_version(void) { return kAbiVersion; }

const char *tree_attn_status_string(int status) {
    switch (status) {
        case TA_OK: return "ok";
        case TA_EINVAL: return "invalid argument (pointer, shape, stride, alignment or scale)";
        case TA_EUNSUPPORTED: return "unsupported head_dim or dtype";
        case TA_EWORKSPACE: return "workspace missing or too small";
        case TA_EHIP: return "HIP runtime or kernel launch failure";
        case TA_ESCRATCH:
            return "problem needs more split-partial space than the allocation-free entry point "
                   "holds (TA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int tree_mask_build(const int32_t *parent, int B, int T, uint64_t *mask, int32_t *err_flag,
                    hipStream_t stream) {
    if (B < 0 || T < 1 || T > TA_MAX_TREE) return TA_EINVAL;
    if (B == 0) return TA_OK;
    if (!parent || !mask) return TA_EINVAL;
    return ta::launch_mask(parent, B, T, mask, err_flag, stream) == hipSuccess ? TA_OK : TA_EHIP;
}

int tree_attn_workspace_size(const ta_problem *p, size_t *bytes) {
    if (!bytes) return TA_EINVAL;
    int rc = check_shape(p);
    if (rc) return rc;
    const Plan pl = make_plan(p);
    *bytes = pl.o_bytes + pl.lse_bytes + pl.cnt_bytes;
    return TA_OK;
}

int tree_attn_num_splits(const ta_problem *p, int *num_splits) {
    if (!num_splits) return TA_EINVAL;
    int rc = check_shape(p);
    if (rc) return rc;
    *num_splits = make_plan(p).n_splits;
    return TA_OK;
}

int tree_attn_prefix(const ta_problem *p, float *o_c, float *lse_c, void *ws, size_t ws_bytes,
                     int32_t *err_flag, hipStream_t stream) {
    int rc = check_shape(p);
    if (rc) return rc;
    if (p->B == 0) return TA_OK;
    if ((rc = check_prefix(p))) return rc;
    if (!o_c || !lse_c) return TA_EINVAL;
    const Plan pl = make_plan(p);
    if (!ws_ok(pl, ws, ws_bytes)) return TA_EWORKSPACE;
    const Workspace w = views(pl, ws);
    if ((rc = launch_prefix_parts(p, pl, err_flag, w, false, stream))) return rc;
    // bf16: the prefix keys past the last full tile are one more part, in the last slot
    const bool tail = p->dtype == TA_BF16;
    const int64_t last = (int64_t)(pl.slots - 1) * pl.rows;
    MergeArgs m{w.o, w.lse, pl.rows * p->D, pl.rows, pl.n_splits,
                tail ? w.o + last * p->D : nullptr, tail ? w.lse + last : nullptr, pl.rows, p->D,
                o_c, lse_c, w.parts, (int64_t)p->T * p->Hq};
    return status(ta::launch_merge(m, false, stream));
}

int tree_attn_tree(const ta_problem *p, float *o_s, float *lse_s, int32_t *err_flag,
                   hipStream_t stream) {
    int rc = check_shape(p);
    if (rc) return rc;
    if (p->B == 0) return TA_OK;
    if ((rc = check_tree(p))) return rc;
    if (!o_s || !lse_s) return TA_EINVAL;
    const Plan pl = make_plan(p);
    return launch_tree_part(p, pl, err_flag, o_s, lse_s, stream);
}

int tree_attn_merge(int B, int T, int Hq, int D, const float *o_a, const float *lse_a,
                    const float *o_b, const float *lse_b, void *o, int o_dtype, float *lse,
                    hipStream_t stream) {
    if (B < 0 || T < 0 || Hq < 0) return TA_EINVAL;
    if (D != 64 && D != 128) return TA_EUNSUPPORTED;
    if (o_dtype != TA_BF16 && o_dtype != TA_F32) return TA_EUNSUPPORTED;
    const int64_t rows = (int64_t)B * T * Hq;
    if (rows == 0) return TA_OK;
    if (!o_a || !lse_a || !o_b || !lse_b || !o || !lse) return TA_EINVAL;
    if (((uintptr_t)o_a & 7u) || ((uintptr_t)o_b & 7u)) return TA_EINVAL;
    MergeArgs m{o_a, lse_a, 0, 0, 1, o_b, lse_b, rows, D, o, lse};
    return ta::launch_merge(m, o_dtype == TA_BF16, stream) == hipSuccess ? TA_OK : TA_EHIP;
}

int tree_attn_workspace_lse_offset(const ta_problem *p, size_t *offset) {
    if (!offset) return TA_EINVAL;
    int rc = check_shape(p);
    if (rc) return rc;
    *offset = make_plan(p).o_bytes;
    return TA_OK;
}

int tree_attn_partials(const ta_problem *p, void *ws, size_t ws_bytes, int32_t *err_flag,
                       hipStream_t stream) {
    int rc = check_shape(p);
    if (rc) return rc;
    if (p->B == 0) return TA_OK;
    if ((rc = check_prefix(p)) || (rc = check_tree(p))) return rc;
    const Plan pl = make_plan(p);
    if (!ws_ok(pl, ws, ws_bytes)) return TA_EWORKSPACE;
    const Workspace w = views(pl, ws);
    if ((rc = launch_prefix_parts(p, pl, err_flag, w, true, stream))) return rc;
    if (p->dtype == TA_BF16) return TA_OK;  // the masked part rode with the last parts
    const int64_t last = (int64_t)(pl.slots - 1) * pl.rows;
    return launch_tree_part(p, pl, err_flag, w.o + last * p->D, w.lse + last, stream);
}

int tree_attn_combine(const ta_problem *p, const void *ws, size_t ws_bytes, void *o, float *lse,
                      hipStream_t stream) {
    int rc = check_shape(p);
    if (rc) return rc;
    if (p->B == 0) return TA_OK;
    if (!o || !lse) return TA_EINVAL;
    const Plan pl = make_plan(p);
    if (!ws_ok(pl, ws, ws_bytes)) return TA_EWORKSPACE;
    const Workspace w = views(pl, ws);
    const int64_t last = (int64_t)(pl.slots - 1) * pl.rows;
    MergeArgs m{w.o, w.lse, pl.rows * p->D, pl.rows, pl.n_splits, w.o + last * p->D, w.lse + last,
                pl.rows, p->D, o, lse, w.parts, (int64_t)p->T * p->Hq};
    return status(ta::launch_merge(m, p->dtype == TA_BF16, stream));
}

int tree_attn_forward(const ta_problem *p, void *o, float *lse, void *ws, size_t ws_bytes,
                      int32_t *err_flag, hipStream_t stream) {
    int rc = check_shape(p);
    if (rc) return rc;
    if (p->B == 0) return TA_OK;
    if (!o || !lse) return TA_EINVAL;
    if (p->dtype == TA_F32) {
        const Plan pl = make_plan(p);
        if (pl.n_splits == 1) {
            // one split: the fp32 kernel takes the prefix and the tree keys of every row in one
            // launch and writes the final output (the workspace is checked but not used)
            if ((rc = check_prefix(p)) || (rc = check_tree(p))) return rc;
            if (!ws_ok(pl, ws, ws_bytes)) return TA_EWORKSPACE;
            AttnArgs a = make_args(p, pl, err_flag);
            a.n_splits = 1;
            a.with_prefix = 1;
            a.with_tree = 1;
            a.out_o = static_cast<float *>(o);
            a.out_lse = lse;
            a.part_so = 0;
            a.part_sl = 0;
            a.seq_parts = nullptr;
            return status(ta::launch_attn_f32(a, stream));
        }
    }
    if ((rc = tree_attn_partials(p, ws, ws_bytes, err_flag, stream))) return rc;
    return tree_attn_combine(p, ws, ws_bytes, o, lse, stream);
}

static int check_accept(int dtype, int B, int T, int V) {
    if (dtype != TA_BF16 && dtype != TA_F32) return TA_EUNSUPPORTED;
    if (B < 0 || B > 65535 || T < 1 || T > TA_MAX_TREE || V < 1) return TA_EINVAL;
    // one workgroup per (row, chunk): the grid must fit its 32-bit dimension
    if ((int64_t)B * (T + 1) * ta::greedy_accept_chunks(V, dtype == TA_BF16) > INT32_MAX)
        return TA_EINVAL;
    return TA_OK;
}

int tree_greedy_accept_workspace_size(int dtype, int B, int T, int V, size_t *bytes) {
    int rc = check_accept(dtype, B, T, V);
    if (rc) return rc;
    if (!bytes) return TA_EINVAL;
    const int S = ta::greedy_accept_chunks(V, dtype == TA_BF16);
    *bytes = align256((size_t)B * (T + 1) * S * 8);
    return TA_OK;
}

int tree_greedy_accept(const void *logits, int dtype, int64_t row_stride, int B, int T, int V,
                       const int32_t *draft, const int32_t *parent, void *ws, size_t ws_bytes,
                       int32_t *greedy, int32_t *accept_len, int32_t *path, int32_t *next_token,
                       int32_t *err_flag, hipStream_t stream) {
    int rc = check_accept(dtype, B, T, V);
    if (rc) return rc;
    if (row_stride < V) return TA_EINVAL;
    if (B == 0) return TA_OK;
    if (!logits || !draft || !parent || !greedy || !accept_len || !path || !next_token)
        return TA_EINVAL;
    const int es = elem_size(dtype);
    if (!aligned16(logits) || (row_stride * es) % 16) return TA_EINVAL;
    const int S = ta::greedy_accept_chunks(V, dtype == TA_BF16);
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < (size_t)B * (T + 1) * S * 8)
        return TA_EWORKSPACE;
    return status(ta::launch_greedy_accept(logits, dtype == TA_BF16, row_stride, B, T, V, S, draft,
                                           parent, static_cast<int2 *>(ws), greedy, accept_len,
                                           path, next_token, err_flag, stream));
}

static int check_spec(int B, int T, int V) {
    if (B < 0 || B > 65535 || T < 1 || T > TA_MAX_TREE || V < 1 || V > TA_MAX_VOCAB)
        return TA_EINVAL;
    return TA_OK;
}

// Workspace of tree_spec_sample: mass chunk sums, then the walk's pass chunk sums (both
// B (T + 1) nch doubles).
static size_t spec_ws_bytes(int B, int T, int V) {
    const size_t n = (size_t)B * (T + 1) * ta::spec_sample_chunks(V);
    return align256(2 * n * sizeof(double));
}

int tree_spec_sample_workspace_size(int B, int T, int V, size_t *bytes) {
    int rc = check_spec(B, T, V);
    if (rc) return rc;
    if (!bytes) return TA_EINVAL;
    *bytes = spec_ws_bytes(B, T, V);
    return TA_OK;
}

int tree_spec_sample(const float *p, const float *q, int64_t row_stride, int B, int T, int V,
                     const int32_t *draft, const int32_t *parent, const double *u_accept,
                     const double *u_sample, void *ws, size_t ws_bytes, int32_t *accept_len,
                     int32_t *path, int32_t *next_token, int32_t *err_flag, hipStream_t stream) {
    int rc = check_spec(B, T, V);
    if (rc) return rc;
    if (row_stride < V || (row_stride * 4) % 16) return TA_EINVAL;
    if (B == 0) return TA_OK;
    if (!p || !q || !draft || !parent || !u_accept || !u_sample || !accept_len || !path ||
        !next_token)
        return TA_EINVAL;
    if (!aligned16(p) || !aligned16(q)) return TA_EINVAL;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < spec_ws_bytes(B, T, V)) return TA_EWORKSPACE;
    const size_t n = (size_t)B * (T + 1) * ta::spec_sample_chunks(V);
    double *sums = static_cast<double *>(ws);
    ta::SpecArgs a{p, q, row_stride, B, T, V, draft, parent, u_accept, u_sample, sums, sums + n,
                   accept_len, path, next_token, err_flag};
    return status(ta::launch_spec_sample(a, cu_count(), stream));
}

static int check_gdn(int B, int T, int Hk, int Hv, int dk, int dv) {
    if (dk != 64 && dk != 128) return TA_EUNSUPPORTED;
    if (dv < 32 || dv > 256 || dv % 32) return TA_EUNSUPPORTED;
    if (B < 0 || B > 65535 || T < 1 || T > TA_MAX_TREE) return TA_EINVAL;
    if (Hk < 1 || Hv < 1 || Hv % Hk || Hv > 65535) return TA_EINVAL;
    return TA_OK;
}

int tree_gdn_verify(const void *q, const void *k, const void *v, const float *g,
                    const float *beta, const int32_t *parent, const float *S0, int B, int T,
                    int Hk, int Hv, int dk, int dv, float scale, float *o, int32_t *err_flag,
                    hipStream_t stream) {
    int rc = check_gdn(B, T, Hk, Hv, dk, dv);
    if (rc) return rc;
    if (!isfinite(scale)) return TA_EINVAL;
    if (B == 0) return TA_OK;
    if (!q || !k || !v || !g || !beta || !parent || !S0 || !o) return TA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S0) || !aligned16(o))
        return TA_EINVAL;
    ta::GdnArgs a{q, k, v, g, beta, parent, S0, B, T, Hk, Hv, dk, dv, scale, o, err_flag};
    return status(ta::launch_gdn_verify(a, cu_count(), stream));
}

int tree_gdn_commit(const void *k, const void *v, const float *g, const float *beta, int B,
                    int T, int Hk, int Hv, int dk, int dv, const int32_t *path,
                    const int32_t *accept_len, float *S, int32_t *err_flag, hipStream_t stream) {
    int rc = check_gdn(B, T, Hk, Hv, dk, dv);
    if (rc) return rc;
    if (B == 0) return TA_OK;
    if (!k || !v || !g || !beta || !path || !accept_len || !S) return TA_EINVAL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(S)) return TA_EINVAL;
    ta::GdnCommitArgs a{k, v, g, beta, B, T, Hk, Hv, dk, dv, path, accept_len, S, err_flag};
    return status(ta::launch_gdn_commit(a, stream));
}

int tree_kv_commit(const ta_problem *p, void *k_cache, void *v_cache, const int32_t *path,
                   const int32_t *accept_len, int32_t *new_seq_lens, int32_t *err_flag,
                   hipStream_t stream) {
    int rc = check_shape(p);
    if (rc) return rc;
    if (p->B == 0) return TA_OK;
    if ((rc = check_prefix(p)) || (rc = check_tree(p))) return rc;
    if (!k_cache || !v_cache || !path || !accept_len || !new_seq_lens) return TA_EINVAL;
    if (!aligned16(k_cache) || !aligned16(v_cache)) return TA_EINVAL;
    const Plan pl = make_plan(p);
    ta::CommitArgs c{};
    c.kt = p->k_tree;
    c.vt = p->v_tree;
    c.kt_sb = p->kt_sb;
    c.kt_st = p->kt_st;
    c.kt_sh = p->kt_sh;
    c.kc = k_cache;
    c.vc = v_cache;
    c.kv_s0 = p->kv_s0;
    c.kv_s1 = p->kv_s1;
    c.kv_s2 = p->kv_s2;
    c.block_table = p->block_table;
    c.max_blocks = p->max_blocks;
    c.page_shift = p->block_table ? ilog2(p->page_size) : 0;
    c.page_mask = p->block_table ? p->page_size - 1 : 0;
    c.num_pages = p->num_pages;
    c.capacity = pl.capacity;
    c.seq_lens = p->seq_lens;
    c.accept_len = accept_len;
    c.path = path;
    c.T = p->T;
    c.es = elem_size(p->dtype);
    c.row_bytes = p->D * c.es;
    c.err = err_flag;
    return status(ta::launch_commit(c, p->B, p->Hkv, new_seq_lens, stream));
}

}  // extern "C"
