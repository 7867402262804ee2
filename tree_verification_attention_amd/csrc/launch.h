// Internal launch interface shared by the C ABI (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ta {

// Keys per LDS tile of the bf16 attention kernel (two 32-key MFMA sub-tiles).
constexpr int kKeyTile = 64;
// Packed query rows (tree node x GQA group member) handled by one wavefront.
constexpr int kRowsPerWave = 32;
// Block-table entries of one part that the bf16 kernel caches in LDS (paged layout).
constexpr int kPageCache = 2048;

// Device-side view of one attention launch. With with_prefix, every sequence's prefix is
// split into parts; part p of sequence b writes out_o[p][row][D] and out_lse[p][row], row =
// (b * T + node) * Hq + head, and seq_parts[b] (when non-null) receives sequence b's part count.
//   bf16 (prefix kernel): the B * n_splits workgroups of a (kv head, row block) are dealt to the
//   sequences in proportion to their lengths (at most 2 n_splits parts each; see the kernel),
//   and the parts take the prefix's full kKeyTile tiles only. Each sequence's last part then
//   computes the masked part -- the prefix keys past the last full tile (with with_prefix) and
//   the tree keys under the ancestor mask (with_tree) -- into out_o_m / out_lse_m. Without
//   with_prefix nothing is written to out_o / out_lse.
//   fp32: n_splits parts of chunk keys per sequence; with_tree folds the tree keys into the
//   last part.
struct AttnArgs {
    const void *q;
    int64_t q_sb, q_st, q_sh;
    const void *kc, *vc;
    int64_t kv_s0, kv_s1, kv_s2;
    const int32_t *seq_lens;
    const int32_t *block_table;
    int32_t max_blocks, page_shift, page_mask, num_pages, capacity;
    const void *kt, *vt;
    int64_t kt_sb, kt_st, kt_sh;
    const int32_t *parent;
    int32_t B, T, Hq, Hkv, G, D;
    int32_t n_splits;
    int32_t with_prefix;
    int32_t with_tree;
    int32_t chunk;      // prefix keys per split (multiple of kKeyTile); the bf16 kernel uses
                        // at most this, sized on the device from the longest prefix
    int32_t reserve;    // keys' worth of time the last split keeps for the masked part
    int32_t n_rb;       // row blocks per (b, kv-head)
    float scale;        // logit scale
    float scale_log2;   // scale * log2(e)
    float *out_o;
    float *out_lse;
    int64_t part_so, part_sl;  // part strides (elements) of out_o / out_lse
    float *out_o_m;            // bf16: the masked part's [row][D] and [row]
    float *out_lse_m;
    int32_t *seq_parts;        // [B] part count of every sequence, or null
    int32_t *err;
};

// Merge of n0 parts from (o0, lse0) (part strides so0 / sl0) plus, when o1 is non-null, one
// more part (o1, lse1), into o (bf16 or fp32) and lse. With seq_parts non-null, the rows of
// sequence b = row / seq_rows take seq_parts[b] parts from (o0, lse0) instead of n0.
struct MergeArgs {
    const float *o0, *lse0;
    int64_t so0, sl0;
    int32_t n0;
    const float *o1, *lse1;
    int64_t rows;
    int32_t D;
    void *o;
    float *lse;
    const int32_t *seq_parts;
    int64_t seq_rows;
};

// Accepted-path KV commit: tree K/V rows path[b][j] (j < accept_len[b]) go to cache position
// seq_lens[b] + j of sequence b (contiguous cache or page pool), row_bytes = D * es per head.
struct CommitArgs {
    const void *kt, *vt;
    int64_t kt_sb, kt_st, kt_sh;
    void *kc, *vc;
    int64_t kv_s0, kv_s1, kv_s2;
    const int32_t *block_table;
    int32_t max_blocks, page_shift, page_mask, num_pages, capacity;
    const int32_t *seq_lens, *accept_len, *path;
    int32_t T, es, row_bytes;
    int32_t *err;
};

hipError_t launch_mask(const int32_t *parent, int B, int T, uint64_t *mask, int32_t *err,
                       hipStream_t s);
hipError_t launch_attn_prefix(const AttnArgs &a, int nw, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs &a, hipStream_t s);
hipError_t launch_merge(const MergeArgs &m, bool out_bf16, hipStream_t s);
struct GdnArgs {
    const void *q, *k, *v;   // bf16 [B, T, Hk, dk], [B, T, Hk, dk], [B, T, Hv, dv]
    const float *g, *beta;   // [B, T, Hv]
    const int32_t *parent;   // [B, T]
    const float *S0;         // [B, Hv, dk, dv]
    int B, T, Hk, Hv, dk, dv;
    float scale;
    float *o;                // [B, T, Hv, dv]
    int32_t *err;
};

struct GdnCommitArgs {
    const void *k, *v;       // bf16 [B, T, Hk, dk], [B, T, Hv, dv]
    const float *g, *beta;   // [B, T, Hv]
    int B, T, Hk, Hv, dk, dv;
    const int32_t *path, *accept_len;
    float *S;                // [B, Hv, dk, dv], updated in place
    int32_t *err;
};

hipError_t launch_gdn_verify(const GdnArgs &a, int cus, hipStream_t s);
hipError_t launch_gdn_commit(const GdnCommitArgs &a, hipStream_t s);

struct SpecArgs {
    const float *p, *q;      // [B, T + 1, V] target / candidate distributions, row_stride apart
    int64_t row_stride;      // elements
    int B, T, V;
    const int32_t *draft, *parent;
    const double *u_accept;  // [B, T]
    const double *u_sample;  // [B]
    double *sums;            // workspace: [B * (T + 1)][nch] chunk sums of the mass kernel
    double *pass_sums;       // workspace: [B][T + 1][nch] chunk sums of the walk's row passes
    int32_t *accept_len, *path, *next_token, *err;
};

// 4096-entry chunks per row of tree speculative sampling.
int spec_sample_chunks(int V);
hipError_t launch_spec_sample(const SpecArgs &a, int cus, hipStream_t s);

// Chunks per logits row for the argmax (the workspace holds B * (T + 1) * chunks int2 winners).
int greedy_accept_chunks(int V, bool bf16);
hipError_t launch_greedy_accept(const void *logits, bool bf16, int64_t row_stride, int B, int T,
                                int V, int S, const int32_t *draft, const int32_t *parent,
                                int2 *part, int32_t *greedy, int32_t *accept_len, int32_t *path,
                                int32_t *next_token, int32_t *err, hipStream_t s);
hipError_t launch_commit(const CommitArgs &c, int B, int Hkv, int32_t *new_lens, hipStream_t s);

}  // namespace ta
