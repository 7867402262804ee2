/*
 * treeattn.h -- C ABI of the MI355X (gfx950) tree-verification attention library.
 *
 * The operation is LongSpec's Hybrid Tree Attention (LongSpec page, "Fast tree attention"
 * section): every node of a draft tree attends to the committed KV prefix with no mask and to
 * the tree's own keys under an ancestor mask, and the two partial results are merged through
 * their log-sum-exps (same section, aggregation equations; appendix "Correctness of attention
 * aggregation", Proposition). The library computes, for tree node i of sequence b and query
 * head h,
 *
 *     O[b,i,h]   = sum_j softmax_j(s_j) * v_j,      LSE[b,i,h] = ln sum_j exp(s_j),
 *     s_j        = scale * q[b,i,h] . k_j,
 *
 * with j running over the prefix keys 0..seq_lens[b]-1 and over the tree nodes that are i or
 * an ancestor of i. Query head h reads KV head h / (Hq / Hkv).
 *
 * Conventions shared by every call:
 *   - Pointers are device pointers unless stated otherwise. The caller allocates and owns all
 *     memory, including the workspace; the library allocates nothing, keeps no pointer after a
 *     call returns and holds no mutable global state -- except tree_attn_forward_noalloc, whose
 *     partials live in one fixed device array per GPU (see there).
 *   - All work is enqueued on ``stream`` (0 = the null stream); no call synchronises the host.
 *   - Return values are ta_status codes. Argument errors are reported before anything is
 *     enqueued. Errors that only the device can see (a parent index out of range, a prefix
 *     length above the KV capacity, a block-table entry outside the page pool) are reported by
 *     writing a nonzero TA_DEV_* bit into ``*err_flag`` (atomic OR; pass NULL to skip). The
 *     caller clears the flag and reads it after synchronising. Out-of-range parents are treated
 *     as -1 and lengths are clamped, so no invalid address is ever read.
 *   - Strides are in elements. The innermost (head_dim) stride is 1 for every tensor, and every
 *     row base must be 16-byte aligned.
 */
#ifndef TREEATTN_H
#define TREEATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ta_status {
    TA_OK = 0,
    TA_EINVAL = 1,        /* null pointer, bad shape, stride or alignment, Hq % Hkv != 0, T > 256 */
    TA_EUNSUPPORTED = 2,  /* head_dim not in {64, 128}, unknown dtype */
    TA_EWORKSPACE = 3,    /* workspace missing or smaller than tree_attn_workspace_size() */
    TA_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
    TA_ESCRATCH = 5       /* tree_attn_forward_noalloc: the problem's split partials need more
                             than TA_NOALLOC_SCRATCH_BYTES */
} ta_status;

typedef enum ta_dtype {
    TA_BF16 = 0,          /* bfloat16 inputs; fp32 accumulation */
    TA_F32 = 1            /* float32 inputs and arithmetic */
} ta_dtype;

/* Bits written into *err_flag by the device. */
#define TA_DEV_BAD_PARENT 1u   /* parent[b][i] outside [-1, i-1] */
#define TA_DEV_BAD_LEN 2u      /* seq_lens[b] outside [0, capacity] */
#define TA_DEV_BAD_PAGE 4u     /* a block-table entry used by a prefix outside [0, num_pages) */
#define TA_DEV_BAD_COMMIT 8u   /* a commit past the cache capacity, or a path entry outside [0, T) */
#define TA_DEV_BAD_TOKEN 16u   /* a draft token outside [0, V) (speculative sampling rejects it) */

/* Largest tree the kernels accept. */
#define TA_MAX_TREE 256
#define TA_MAX_VOCAB (1 << 20) /* largest vocabulary tree_spec_sample accepts */

/*
 * One attention layer of a verify step. Plain C struct, read during the call only.
 *
 * Operands (the pages' statement of the problem: Q for the tree nodes, the cache part
 * {K_cache, V_cache} and the speculative part {K_specs, V_specs}, plus the tree):
 *   q          [B, T, Hq, D] with strides (q_sb, q_st, q_sh); dtype ``dtype``.
 *   k_cache,   committed prefix. Contiguous layout (block_table == NULL): [B, Lmax, Hkv, D]
 *   v_cache    with strides (kv_s0 = batch, kv_s1 = row, kv_s2 = head). Paged layout: a page
 *              pool [num_pages, page_size, Hkv, D] with strides (kv_s0 = page, kv_s1 = row,
 *              kv_s2 = head); key j of sequence b lives in page block_table[b][j / page_size]
 *              at row j % page_size. K and V share one stride set. Strides are elements, each
 *              a multiple of 16 bytes; 64 rows (contiguous) or one page (paged) must span less
 *              than 2^31 bytes, the whole cache may be larger.
 *   seq_lens   int32 [B]: prefix length of each sequence, 0 <= seq_lens[b] <= capacity, where
 *              capacity = Lmax (contiguous) or max_blocks * page_size (paged).
 *   block_table int32 [B, max_blocks] or NULL. page_size is a power of two >= 16.
 *   k_tree,    the T tree nodes' keys and values, [B, T, Hkv, D] with strides
 *   v_tree     (kt_sb, kt_st, kt_sh), shared by K and V.
 *   parent     int32 [B, T], topological: parent[b][i] in [-1, i-1]; -1 hangs node i directly
 *              off the committed prefix (DFlash-TfM summary page, "Rollback-free tree
 *              verification": the tree is sorted topologically).
 *   scale      the logit scale, normally 1/sqrt(D).
 *   num_splits number of KV splits of the prefix, or 0 to let the library choose.
 */
typedef struct ta_problem {
    int32_t B, T, Hq, Hkv, D;
    int32_t dtype;
    float scale;
    int32_t num_splits;
    const void *q;
    int64_t q_sb, q_st, q_sh;
    const void *k_cache;
    const void *v_cache;
    int64_t kv_s0, kv_s1, kv_s2;
    const int32_t *seq_lens;
    const int32_t *block_table;
    int32_t Lmax, page_size, max_blocks, num_pages;
    const void *k_tree;
    const void *v_tree;
    int64_t kt_sb, kt_st, kt_sh;
    const int32_t *parent;
} ta_problem;

/*
 * Ancestor-or-self mask of a batch of draft trees (LongSpec page, "Fast tree attention": the
 * tree mask disables attention between speculative tokens of different branches; textbook page,
 * "Linear chains and candidate trees consume work differently": each node only attends to its
 * ancestors). parent: int32 [B, T], 1 <= T <= 256. mask: uint64 [B, T, W], W = ceil(T / 64);
 * bit (j % 64) of word j / 64 of row i is set exactly when j == i or j is an ancestor of i.
 * Invalid parents set TA_DEV_BAD_PARENT and are treated as -1.
 */
int tree_mask_build(const int32_t *parent, int B, int T, uint64_t *mask, int32_t *err_flag,
                    hipStream_t stream);

/*
 * Host-only. Bytes of workspace that tree_attn_prefix, tree_attn_partials and tree_attn_forward
 * need for ``p`` (2 S + 1 fp32 partial slots of O and LSE per row, S = tree_attn_num_splits(),
 * and one int32 part count per sequence; layout at tree_attn_partials). Writes *bytes; returns
 * TA_EINVAL / TA_EUNSUPPORTED for a problem the other calls would reject.
 */
int tree_attn_workspace_size(const ta_problem *p, size_t *bytes);

/* Host-only. The split count S the library plans for ``p`` (after automatic choice): every KV
 * head's prefixes are cut into S * B parts, S per sequence on average. */
int tree_attn_num_splits(const ta_problem *p, int *num_splits);

/*
 * Unmasked attention of every tree query over its sequence's committed prefix -- the cache part
 * of the divide-and-aggregate step (LongSpec page, "Fast tree attention", splitting the
 * key-value pairs). o_c: fp32 [B, T, Hq, D]; lse_c: fp32 [B, T, Hq] (natural log). A sequence
 * with an empty prefix gets O = 0 and LSE = -inf. ``ws`` is device memory of at least
 * tree_attn_workspace_size() bytes, 256-byte aligned.
 */
int tree_attn_prefix(const ta_problem *p, float *o_c, float *lse_c, void *ws, size_t ws_bytes,
                     int32_t *err_flag, hipStream_t stream);

/*
 * Masked attention of every tree query over the tree's own keys -- the speculative part
 * (same section). Node i sees node j iff j == i or j is an ancestor of i; the mask is derived
 * on the device from ``parent``. o_s: fp32 [B, T, Hq, D]; lse_s: fp32 [B, T, Hq]. Needs no
 * workspace. Prefix fields of ``p`` are ignored.
 */
int tree_attn_tree(const ta_problem *p, float *o_s, float *lse_s, int32_t *err_flag,
                   hipStream_t stream);

/*
 * Log-sum-exp aggregation of two partial results over disjoint key sets (LongSpec page, "Fast
 * tree attention", aggregation equations; appendix Proposition):
 *     LSE = ln(exp(LSE_a) + exp(LSE_b)),  O = O_a exp(LSE_a - LSE) + O_b exp(LSE_b - LSE).
 * Rows = B * T * Hq, each D wide, contiguous. o_a, o_b: fp32 [rows, D]; lse_a, lse_b: fp32
 * [rows]; o: [rows, D] of o_dtype (TA_BF16 rounds to nearest even, or TA_F32); lse: fp32
 * [rows]. Two empty parts (both -inf) give O = 0, LSE = -inf. Outputs may alias inputs of the
 * same type only if they are identical pointers.
 */
int tree_attn_merge(int B, int T, int Hq, int D, const float *o_a, const float *lse_a,
                    const float *o_b, const float *lse_b, void *o, int o_dtype, float *lse,
                    hipStream_t stream);

/*
 * The whole hybrid tree attention of one layer: prefix (split over the KV length), masked tree
 * part with the mask derived in-kernel, and the log-sum-exp aggregation of all partials, as
 * tree_attn_partials then tree_attn_combine (bf16: two kernel launches, the masked part riding
 * on the last prefix split; fp32 with one split: one launch that writes the output directly, the
 * workspace checked but unused). o: [B, T, Hq, D] contiguous, of p->dtype; lse: fp32 [B, T, Hq]
 * (natural log).
 */
int tree_attn_forward(const ta_problem *p, void *o, float *lse, void *ws, size_t ws_bytes,
                      int32_t *err_flag, hipStream_t stream);

/* Bytes of the device array that tree_attn_forward_noalloc keeps its split partials in. */
#define TA_NOALLOC_SCRATCH_BYTES (96u << 20)

/*
 * tree_attn_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation, the
 * same kernels and the same results, with the workspace replaced by one file-scope device array
 * of TA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds from the library's load
 * until the process ends. The call allocates nothing and calls no allocating routine; its first
 * call on a device looks the array's address up (hipGetSymbolAddress). Returns TA_ESCRATCH, with
 * nothing enqueued, when the problem needs more than that (tree_attn_workspace_size() above
 * TA_NOALLOC_SCRATCH_BYTES; at D = 128, 96 MiB holds up to 32 768 output rows with two splits
 * or 8192 rows with eight). Every call on one GPU shares the array and leaves its contents
 * there: calls that overlap on one GPU (other streams or host threads) race, and the caller
 * serialises them. Arguments and the other errors as for tree_attn_forward.
 */
int tree_attn_forward_noalloc(const ta_problem *p, void *o, float *lse, int32_t *err_flag,
                              hipStream_t stream);

/*
 * The divide step of tree_attn_forward on its own: every prefix part and the masked tree part
 * write their partial (O, LSE) into ``ws`` (LongSpec page, "Fast tree attention", splitting the
 * key-value pairs; the prefix is further split along its length). With S =
 * tree_attn_num_splits() and rows = B * T * Hq the workspace holds P = 2 S + 1 slots: fp32 O
 * [P][rows][D] at byte 0, fp32 LSE [P][rows] at byte tree_attn_workspace_lse_offset(), then
 * int32 counts [B] right after the LSE slots (at the lse offset plus P * rows * 4, rounded up to
 * 256). Sequence b's prefix is split into counts[b] <= 2 S parts, in slots 0 .. counts[b] - 1 of
 * its rows (the S * B parts of a KV head are dealt to the sequences by length, so a longer
 * sequence gets more of them); bf16 parts hold whole 64-key tiles. Slot 2 S holds the masked
 * tree keys and, for bf16, the prefix keys past the last multiple of 64. An empty part has
 * O = 0 and LSE = -inf. A caller that shards the prefix over several devices exchanges these
 * partials.
 */
int tree_attn_partials(const ta_problem *p, void *ws, size_t ws_bytes, int32_t *err_flag,
                       hipStream_t stream);

/*
 * The aggregation step on its own: merges the P parts that tree_attn_partials left in ``ws``
 * (same ``p``) by the log-sum-exp identity into o ([B, T, Hq, D], p->dtype) and lse (fp32).
 * tree_attn_forward == tree_attn_partials followed by tree_attn_combine.
 */
int tree_attn_combine(const ta_problem *p, const void *ws, size_t ws_bytes, void *o, float *lse,
                      hipStream_t stream);

/* Host-only. Byte offset of the LSE parts inside the workspace of ``p``. */
int tree_attn_workspace_lse_offset(const ta_problem *p, size_t *offset);

/*
 * Greedy tree acceptance (textbook page, "Faster decoding", greedy verification contract: accept
 * the longest draft prefix that agrees with the target's greedy tokens, then emit the target's
 * greedy token at the first disagreement), on a draft tree.
 *   logits      [B, T + 1, V] of ``dtype`` (TA_BF16 or TA_F32): row (b, 0) holds the target's
 *               logits at sequence b's last committed token, row (b, i + 1) at tree node i.
 *               ``row_stride`` (elements, >= V) separates consecutive rows; the base and every
 *               row must be 16-byte aligned.
 *   draft       int32 [B, T]: the draft token of every node.
 *   parent      int32 [B, T]: topological parent array (-1 = attached to the committed prefix).
 * Outputs (device memory, caller-owned):
 *   greedy      int32 [B, T + 1]: argmax of every row -- the first index holding the maximum of
 *               the row's non-NaN entries (a row of NaN only gives 0).
 *   accept_len  int32 [B]: nodes on the committed path.
 *   path        int32 [B, T]: the committed path, root first; -1 past accept_len. Node i is
 *               accepted iff draft[i] equals the greedy token of its parent's row (row 0 for a
 *               root-attached node) and its parent is accepted; the path ends at the deepest
 *               accepted node (the smallest index among equally deep ones).
 *   next_token  int32 [B]: the greedy token of the last path node's row (row 0 if none).
 * ``ws``: device memory of at least tree_greedy_accept_workspace_size() bytes, 256-byte aligned
 * (each row is scanned in several chunks whose winners meet there); otherwise TA_EWORKSPACE.
 * Parents outside [-1, i-1] set TA_DEV_BAD_PARENT and count as -1. 1 <= T <= TA_MAX_TREE,
 * 0 <= B <= 65535.
 */
int tree_greedy_accept(const void *logits, int dtype, int64_t row_stride, int B, int T, int V,
                       const int32_t *draft, const int32_t *parent, void *ws, size_t ws_bytes,
                       int32_t *greedy, int32_t *accept_len, int32_t *path, int32_t *next_token,
                       int32_t *err_flag, hipStream_t stream);

/* Host-only. Workspace bytes tree_greedy_accept needs for these sizes on the current device. */
int tree_greedy_accept_workspace_size(int dtype, int B, int T, int V, size_t *bytes);

/*
 * Tree speculative sampling (textbook page, "Faster decoding", section on modified rejection
 * sampling keeping the target distribution). At a position, a candidate x drawn from q is accepted
 * with probability min(1, p(x) / q(x)); a rejection draws from the residual [p - q]_+ / Z, and
 * Z = 0 means no rejection happens. The pages state this along a chain; on a tree the children of
 * a position are candidates drawn independently from its q, tried in index order, and after each
 * rejection the residual stands in for p when the next child is tried (a chain is the pages'
 * rule). With every child of a position rejected, the correction token is drawn from the last
 * residual; an accepted node without children ends the path with a bonus token drawn from its
 * row's p. "Drawn from weights w with uniform u" means: the smallest index whose running sum of w
 * exceeds u * sum(w) (if rounding leaves none, the last index with positive weight).
 *   p, q        float32 [B, T + 1, V]: target and candidate distributions of the next token at
 *               the last committed token (row 0) and after tree node i (row i + 1); consecutive
 *               rows ``row_stride`` elements (>= V) apart, base and rows 16-byte aligned.
 *   draft       int32 [B, T]: the candidate token of every node (drawn from q at its parent's row).
 *   parent      int32 [B, T]: topological parent array (-1 = attached to the committed prefix).
 *   u_accept    float64 [B, T]: uniform in [0, 1) per node (accept iff u < the acceptance
 *               probability); u_sample float64 [B]: uniform for the emitted token.
 * Outputs (device memory, caller-owned): accept_len int32 [B]; path int32 [B, T] (accepted
 * nodes, root first, -1 past accept_len); next_token int32 [B] (correction or bonus token).
 * All sums are fp64 over the fp32 inputs. ``ws``: device memory of at least
 * tree_spec_sample_workspace_size() bytes, 256-byte aligned. Parents outside [-1, i-1] set
 * TA_DEV_BAD_PARENT and count as -1; draft tokens outside [0, V) set TA_DEV_BAD_TOKEN and are
 * treated as tokens of zero target mass. 0 <= B <= 65535, 1 <= T <= TA_MAX_TREE,
 * 1 <= V <= TA_MAX_VOCAB.
 */
int tree_spec_sample(const float *p, const float *q, int64_t row_stride, int B, int T, int V,
                     const int32_t *draft, const int32_t *parent, const double *u_accept,
                     const double *u_sample, void *ws, size_t ws_bytes, int32_t *accept_len,
                     int32_t *path, int32_t *next_token, int32_t *err_flag, hipStream_t stream);

/*
 * Host-only. Workspace bytes tree_spec_sample needs: two arrays of B * (T + 1) * ceil(V / 4096)
 * doubles (chunk sums of the residual masses; the second is where the workgroups that share a
 * sequence's row passes exchange theirs).
 */
int tree_spec_sample_workspace_size(int B, int T, int V, size_t *bytes);

/*
 * Tree verification of a gated-delta-net (GDN) layer (DFlash-TfM summary page, "Rollback-free
 * tree verification for GDN"). The layer keeps a d_k x d_v state per value head and updates it
 * per token as S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T, alpha_t = e^{g_t};
 * on the tree every node continues its parent's state (root-attached nodes continue S0) and the
 * output is o_t = scale * S_t^T q_t. Computed without forming any node state: the pseudo-values U
 * solve the lower-triangular system (I + X) U = beta (V - e^{G} K S0) over the ancestor structure
 * (X_tj = beta_t e^{G_t - G_j} k_t.k_j for strict ancestors j, G = log-decay summed over the path),
 * then o_t = scale (e^{G_t} S0^T q_t + sum over ancestors-or-self j of e^{G_t - G_j} (q_t.k_j) u_j).
 *   q, k        bf16 [B, T, Hk, dk] (contiguous); v bf16 [B, T, Hv, dv]; value head h reads key
 *               head h / (Hv / Hk).
 *   g, beta     float32 [B, T, Hv]: log-decay (<= 0) and write strength of every node and head.
 *   parent      int32 [B, T] topological parent array (-1 = attached to the committed state).
 *   S0          float32 [B, Hv, dk, dv]: the committed states (read only).
 *   o           float32 [B, T, Hv, dv] (caller-owned device memory).
 * dk in {64, 128}; dv a multiple of 32, at most 256; Hv a multiple of Hk; 1 <= T <= TA_MAX_TREE;
 * every pointer 16-byte aligned. Parents outside [-1, i-1] set TA_DEV_BAD_PARENT and count as -1.
 */
int tree_gdn_verify(const void *q, const void *k, const void *v, const float *g,
                    const float *beta, const int32_t *parent, const float *S0, int B, int T,
                    int Hk, int Hv, int dk, int dv, float scale, float *o, int32_t *err_flag,
                    hipStream_t stream);

/*
 * The deferred state commit of a GDN layer (same page: the state is committed in the next
 * iteration, once the accepted branch is known, so nothing is rolled back): for every sequence b
 * and value head, S[b] becomes the state after the updates of path[b][0 .. accept_len[b] - 1]
 * (root first, as greedy acceptance or speculative sampling return it), i.e. the state of the
 * last accepted node. S: float32 [B, Hv, dk, dv], updated in place; k, v, g, beta as in
 * tree_gdn_verify. accept_len outside [0, T] leaves S[b] unchanged, a path entry outside [0, T)
 * stops the sequence's updates there; both set TA_DEV_BAD_COMMIT.
 */
int tree_gdn_commit(const void *k, const void *v, const float *g, const float *beta, int B,
                    int T, int Hk, int Hv, int dk, int dv, const int32_t *path,
                    const int32_t *accept_len, float *S, int32_t *err_flag, hipStream_t stream);

/*
 * Accepted-path KV commit (textbook page, "Faster decoding", reserve / execute / commit: only
 * the accepted draft prefix's target KV is committed, rejected branches are released). For every
 * sequence b, the tree K/V rows path[b][j], j < accept_len[b], are copied to cache positions
 * seq_lens[b] + j of k_cache / v_cache, and new_seq_lens[b] = seq_lens[b] + accept_len[b].
 * Shapes, dtype, strides, seq_lens, the cache layout (contiguous, or page pool + block_table whose
 * entries for the new positions the caller has reserved) and the tree K/V come from ``p``;
 * k_cache / v_cache are the writable buffers that p->k_cache / p->v_cache describe. A sequence
 * whose commit would pass the capacity (or with accept_len outside [0, T]) writes nothing, keeps
 * its length and sets TA_DEV_BAD_COMMIT; a path entry outside [0, T) sets it and is skipped.
 * new_seq_lens may alias p->seq_lens (one workgroup per sequence reads its old length, then
 * writes the new one). One kernel launch.
 */
int tree_kv_commit(const ta_problem *p, void *k_cache, void *v_cache, const int32_t *path,
                   const int32_t *accept_len, int32_t *new_seq_lens, int32_t *err_flag,
                   hipStream_t stream);

/* Static description of a status code. Never NULL. */
const char *tree_attn_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int tree_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREEATTN_H */
