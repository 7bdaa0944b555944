/*
 * dsa.h - dynamic sparse attention for the long-context prefill phase on
 * gfx950 (MI355X). Plain C ABI: every pointer is a plain host or device
 * pointer, every size a plain integer, streams are passed as void*
 * (a hipStream_t; NULL is the default stream).
 *
 * Method sources, cited by page title and section:
 *   [MInf]   "MInference 1.0" summary article (developer.volcengine.com):
 *            §1 Problem Formulation (attention under a dynamic mask),
 *            §2.2 Sparsity Indices Approximation and Dynamic Sparse Attention
 *            Calculation (Vertical-Slash Head, Block-Sparse Head), and the
 *            kernel-only usage listing (vertical_slash_sparse_attention,
 *            block_sparse_attention, streaming_forward).
 *   [Novita] "How KV sparsity achieves 1.5x acceleration for vLLM" (Novita AI
 *            blog), §2 Modificación de Atención (rowmax / l reuse, key
 *            scores as sums of softmax probabilities over a window of the last
 *            queries, q start/end restriction).
 *
 * Conventions shared by every call
 * --------------------------------
 * Layout. q and o are [batch][q_heads][seq_len][head_dim], k and v are
 *   [batch][kv_heads][seq_len][head_dim], contiguous row-major, all of the
 *   element type `dtype` (bf16 or fp32), in device memory. Query head h reads
 *   kv head h / (q_heads / kv_heads) (grouped-query attention).
 * Blocks. Query and key blocks are 64 rows: block a covers rows
 *   [64a, min(64a + 64, seq_len)); nb = ceil(seq_len / 64).
 * Masks. Attention is causal (key j <= query i) and further restricted by the
 *   sparse index; masked entries are excluded exactly [MInf §1]. The softmax
 *   scale is `scale`, or 1/sqrt(head_dim) when scale <= 0. A query row whose
 *   allowed key set is empty outputs zeros (reachable only through the
 *   explicit-index calls; the three public calls always keep the diagonal).
 * Head subsets. `heads` is a HOST array of n_heads distinct query-head ids the
 *   call processes (at most DSA_MAX_HEADS); NULL means all q_heads in order.
 *   Outputs of stage calls are "rows" ordered (batch, position in `heads`):
 *   row = b * n_heads + t. Attention calls write only the listed heads of o.
 * Top-k order. A top-k keeps the entries ranking first under: forced entries,
 *   then larger score, then smaller index; -0.0 counts as +0.0 and NaN as
 *   -inf; k is clamped to the candidate count; indices are returned
 *   ascending.
 * Ownership. The caller owns every buffer, including `workspace`; the library
 *   allocates and frees nothing and keeps no state between calls.
 * Execution. Calls enqueue work on `stream` and return without synchronising.
 * Errors. Argument checks happen on the host before anything is enqueued:
 *   DSA_ERR_INVALID_ARG for a NULL pointer, a negative or inconsistent size,
 *   q_heads % kv_heads != 0, a duplicated or out-of-range head id or a bad
 *   top-k/window argument; DSA_ERR_UNSUPPORTED for a head_dim other than 64 or
 *   128, an unknown dtype, last_q outside [1, 64], more than DSA_MAX_HEADS
 *   heads or a head slab (seq_len * head_dim * element size) of 2 GiB or more; DSA_ERR_WORKSPACE when workspace_bytes is below what the matching
 *   *_workspace_bytes call returns; DSA_ERR_HIP when a launch fails.
 * Empty work. A prefill call (the three pattern calls, the mixed calls, the
 *   stage calls, KV retention) with batch 0, seq_len 0 or no listed head
 *   enqueues nothing, returns DSA_OK and needs no workspace (the matching
 *   *_workspace_bytes call returns 0); its data pointers are not read and may
 *   be NULL (zero-size arrays have no address), while scalar arguments are
 *   still checked. The sparse decode step with no decode row (batch 0 or no
 *   listed head) likewise returns DSA_OK; with an empty cache or empty key
 *   lists it still runs and writes zero rows.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_BLOCK 64
#define DSA_MAX_HEADS 256

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE = 3,
  DSA_ERR_HIP = 4
} dsa_status;

typedef enum { DSA_BF16 = 0, DSA_F32 = 1 } dsa_dtype;

typedef struct {
  int32_t batch;
  int32_t q_heads;
  int32_t kv_heads;
  int32_t seq_len;
  int32_t head_dim; /* 64 or 128 */
  int32_t dtype;    /* dsa_dtype */
} dsa_shape;

/* Human-readable name of a status code (static string). */
const char* dsa_status_string(dsa_status s);

/* ======================================================================
 * The three calls of the kernel-only API [MInf, usage listing]
 * ====================================================================== */

/* Vertical-slash heads [MInf §2.2 Vertical-Slash Head; Novita §2].
 * For each listed head: estimate the vertical and slash scores from the last
 * last_q query rows (dsa_vs_estimate), keep the top vertical_topk columns and
 * the top slash_topk diagonal offsets with offset 0 forced (dsa_topk), build
 * the block sparse format (dsa_vs_build_index) and run exact attention over it
 * (dsa_sparse_attention_vs). Writes o for the listed heads.
 * vertical_topk >= 0, slash_topk >= 1, last_q in [1, 64]. workspace: device
 * memory of at least dsa_vertical_slash_workspace_bytes(...) bytes. */
dsa_status dsa_vertical_slash_sparse_attention(
    const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
    int32_t vertical_topk, int32_t slash_topk, int32_t last_q, float scale,
    const int32_t* heads, int32_t n_heads, void* workspace, size_t workspace_bytes,
    void* stream);
size_t dsa_vertical_slash_workspace_bytes(const dsa_shape* shape, int32_t vertical_topk,
                                          int32_t slash_topk, int32_t n_heads);

/* Block-sparse heads [MInf §2.2 Block-Sparse Head]. Mean-pool Q and K over
 * 64-row blocks (dsa_bs_pool), score block pairs scale * Qp[a] . Kp[c] for
 * c <= a and keep the top `topk` key blocks per query block with the diagonal
 * block forced (dsa_bs_select), then attend over the kept blocks
 * (dsa_sparse_attention_blocks). topk >= 1. */
dsa_status dsa_block_sparse_attention(
    const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
    int32_t topk, float scale, const int32_t* heads, int32_t n_heads, void* workspace,
    size_t workspace_bytes, void* stream);
size_t dsa_block_sparse_workspace_bytes(const dsa_shape* shape, int32_t topk,
                                        int32_t n_heads);

/* Streaming (A-shape) heads [MInf usage listing, streaming_forward(init_num,
 * local_window_num)]: query block a attends to key blocks c <= a with
 * c < init_blocks or a - c < local_blocks (the window counts the diagonal
 * block). init_blocks >= 0, local_blocks >= 1. Needs no workspace. */
dsa_status dsa_streaming_attention(
    const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
    int32_t init_blocks, int32_t local_blocks, float scale, const int32_t* heads,
    int32_t n_heads, void* stream);

/* Pattern of one query head in a mixed layer. */
typedef enum {
  DSA_PATTERN_NONE = -1, /* head not processed: its o rows are left untouched */
  DSA_PATTERN_VS = 0,
  DSA_PATTERN_BS = 1,
  DSA_PATTERN_STREAM = 2
} dsa_pattern;

/* A layer whose heads follow different patterns [MInf §2.2: every head has
 * one of the patterns, fixed offline; its sparse index is built online from
 * the input]. patterns: HOST int32 [q_heads], a dsa_pattern per query head.
 * Computes what dsa_vertical_slash_sparse_attention does for the VS heads,
 * dsa_block_sparse_attention for the BS heads and dsa_streaming_attention for
 * the streaming heads, each over its heads in ascending order, but the
 * attention of all heads runs as one launch (work items pattern by pattern,
 * each pattern's heads grouped by kv head). Output is bit-identical to those calls for
 * the VS and BS heads; streaming heads run the one-block-per-work-group code
 * (the streaming call runs two query blocks per work-group) and agree with it
 * to rounding. Every argument is checked whatever the patterns:
 * vertical_topk >= 0, slash_topk >= 1, last_q in [1, 64], topk >= 1,
 * init_blocks >= 0, local_blocks >= 1; a pattern value outside the enum is
 * DSA_ERR_INVALID_ARG. workspace: at least
 * dsa_mixed_sparse_attention_workspace_bytes(...) bytes. */
dsa_status dsa_mixed_sparse_attention(
    const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
    const int32_t* patterns, int32_t vertical_topk, int32_t slash_topk, int32_t last_q,
    int32_t topk, int32_t init_blocks, int32_t local_blocks, float scale, void* workspace,
    size_t workspace_bytes, void* stream);
size_t dsa_mixed_sparse_attention_workspace_bytes(const dsa_shape* shape,
                                                  const int32_t* patterns,
                                                  int32_t vertical_topk, int32_t slash_topk,
                                                  int32_t topk);

/* ======================================================================
 * Stage calls: the same kernels the calls above run, exposed one by one.
 * ====================================================================== */

/* Vertical and slash scores [MInf §2.2 VS head; Novita §2]. For each listed
 * head, with rows i_r = seq_len - lq + r (lq = min(last_q, seq_len)) and
 * p[r][j] the causal softmax of row i_r over keys j <= i_r:
 *   v_scores[row][j] = sum_r p[r][j],  s_scores[row][d] = sum_r p[r][i_r - d].
 * Outputs: fp32 device arrays [batch * n_heads][seq_len]. workspace: at least
 * dsa_vs_estimate_workspace_bytes(...) bytes. */
dsa_status dsa_vs_estimate(const void* q, const void* k, const dsa_shape* shape,
                           int32_t last_q, float scale, const int32_t* heads,
                           int32_t n_heads, float* v_scores, float* s_scores,
                           void* workspace, size_t workspace_bytes, void* stream);
size_t dsa_vs_estimate_workspace_bytes(const dsa_shape* shape, int32_t n_heads);

/* Row-wise top-k of fp32 scores [MInf §2.2: top-k verticals, slashes and
 * blocks]. scores: device [rows][n]; out: device int32 [rows][min(k, n)],
 * ascending. forced_index in [-1, n): the entry ranked first in every row
 * (-1: none). k >= 0. workspace: device memory of at least
 * dsa_topk_workspace_bytes(rows, n, k) bytes (0 for rows shorter than 65536
 * entries, which one work-group each selects; NULL is then accepted). */
dsa_status dsa_topk(const float* scores, int32_t rows, int32_t n, int32_t k,
                    int32_t forced_index, int32_t* out, void* workspace,
                    size_t workspace_bytes, void* stream);
size_t dsa_topk_workspace_bytes(int32_t rows, int32_t n, int32_t k);

/* Vertical-slash sparse format [MInf §2.2 "convert to sparse format"].
 * Inputs per row: V [rows][nv] ascending column indices and S [rows][ns]
 * ascending slash offsets, all in [0, seq_len). Offsets closer than 65 are
 * merged: intervals [rows][ns][2] receives (d_lo, d_hi) pairs in ascending
 * order and n_intervals [rows] their count. Query block a then covers the key
 * ranges [max(0, 64a - d_hi), min(seq_len, 64a + 64 - d_lo)) of every interval
 * with d_lo < 64a + 64, and the columns cols [rows][nb][nv] (count in
 * n_cols [rows][nb]): the entries of V below min(seq_len, 64a + 64) that lie
 * in none of those ranges, ascending. All device int32 arrays; entries past
 * n_intervals[row] and n_cols[row][a] are left unwritten. */
dsa_status dsa_vs_build_index(const int32_t* V, int32_t nv, const int32_t* S, int32_t ns,
                              int32_t rows, int32_t seq_len, int32_t* intervals,
                              int32_t* n_intervals, int32_t* cols, int32_t* n_cols,
                              void* stream);

/* Block mean-pool [MInf §2.2 BS head]: out[row][a][:] = mean of rows
 * [64a, min(64a+64, seq_len)) of x's head heads[t] (fp32 accumulation).
 * x: device [batch][x_heads][seq_len][head_dim] of `dtype`; out: device fp32
 * [batch * n_heads][nb][head_dim]. heads: host ids in [0, x_heads) or NULL. */
dsa_status dsa_bs_pool(const void* x, int32_t dtype, int32_t batch, int32_t x_heads,
                       int32_t seq_len, int32_t head_dim, const int32_t* heads,
                       int32_t n_heads, float* out, void* stream);

/* Block selection [MInf §2.2 BS head]. qp, kp: device fp32 [rows][nb][head_dim]
 * (row r of qp is scored against row r of kp). L[a][c] = scale * qp[a].kp[c]
 * for c <= a in fp32 (each product as hi.hi + hi.lo + lo.hi of bf16 splits,
 * within about 2^-16 relative of the exact dot); sel [rows][nb][min(topk, nb)]
 * receives the ascending
 * top-min(topk, a+1) blocks of L[a][0..a] with c = a forced and n_sel
 * [rows][nb] their count (entries of sel past the count are left unwritten).
 * logits: NULL, or device fp32 [rows][nb][nb] that
 * receives L (entries c > a are left untouched). workspace: device memory of
 * at least dsa_bs_select_workspace_bytes(rows, nb) bytes, also when logits is
 * given (it then holds only the bf16 splits of qp and kp). */
dsa_status dsa_bs_select(const float* qp, const float* kp, int32_t rows, int32_t nb,
                         int32_t head_dim, float scale, int32_t topk, int32_t* sel,
                         int32_t* n_sel, float* logits, void* workspace,
                         size_t workspace_bytes, void* stream);
size_t dsa_bs_select_workspace_bytes(int32_t rows, int32_t nb);

/* Attention under a given vertical-slash sparse format [MInf §1 Problem
 * Formulation: exact attention with the entries outside the dynamic mask
 * excluded; §2.2 Vertical-Slash Head: the slash and vertical indices drive a
 * block-sparse computation]. Query block a attends, causally, to the key
 * ranges its intervals cover and to its column list, exactly as in the
 * dsa_vs_build_index description; every other key is excluded. For the listed
 * heads, row = b * n_heads + t indexes intervals [rows][max_iv][2],
 * n_intervals [rows], cols [rows][nb][max_cols] and n_cols [rows][nb] (device
 * int32, as dsa_vs_build_index writes them; index values are clamped into
 * [0, seq_len) before any key is read). The index arrays must hold rows
 * entries of these extents: the kernel reads n_intervals[row] intervals and
 * n_cols[row][a] columns of block a. Writes o for the listed heads. */
dsa_status dsa_sparse_attention_vs(
    const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
    float scale, const int32_t* heads, int32_t n_heads, const int32_t* intervals,
    const int32_t* n_intervals, int32_t max_iv, const int32_t* cols, const int32_t* n_cols,
    int32_t max_cols, void* stream);

/* Attention over explicit key-block lists [MInf §1 Problem Formulation, with
 * the mask given by whole 64-key blocks; §2.2 Block-Sparse Head: the selected
 * blocks of each query block are computed, all others skipped]. Query block a
 * attends, causally, to the keys of the blocks sel[row][a][0 .. n_sel[row][a])
 * (device int32 [rows][nb][max_sel] and [rows][nb], ascending distinct ids;
 * ids outside [0, nb) are skipped). Writes o for the listed heads. */
dsa_status dsa_sparse_attention_blocks(
    const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
    float scale, const int32_t* heads, int32_t n_heads, const int32_t* sel,
    const int32_t* n_sel, int32_t max_sel, void* stream);

/* The attention launch of dsa_mixed_sparse_attention over given indices
 * [MInf §1 Problem Formulation; §2.2: each head keeps its own pattern, whose
 * index drives that head's block-sparse computation].
 * patterns: HOST int32 [q_heads] as there. The VS heads, in ascending order,
 * number t = 0 .. n_vs-1 and take rows b * n_vs + t of intervals, n_intervals,
 * cols and n_cols (laid out as for dsa_sparse_attention_vs); the BS heads
 * likewise take rows b * n_bs + t of sel and n_sel (as for
 * dsa_sparse_attention_blocks). The index pointers of a pattern no head
 * follows may be NULL. */
dsa_status dsa_sparse_attention_mixed(
    const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
    float scale, const int32_t* patterns, const int32_t* intervals,
    const int32_t* n_intervals, int32_t max_iv, const int32_t* cols, const int32_t* n_cols,
    int32_t max_cols, const int32_t* sel, const int32_t* n_sel, int32_t max_sel,
    int32_t init_blocks, int32_t local_blocks, void* stream);

/* ======================================================================
 * After prefill: which keys to keep in the KV cache
 * ====================================================================== */

/* KV-retention scores and kept keys [Novita §2: per head, a key's score is the
 * sum of its softmax probabilities over the window of the last queries (the
 * PyramidKV score); the highest-scoring keys keep their KV cache entries]. For
 * each listed head, with w = min(window, seq_len) and p[i][j] the causal
 * softmax of query row i over keys j <= i:
 *   scores[row][j] = sum over i in [seq_len - w, seq_len) of p[i][j]
 * (the vertical score of dsa_vs_estimate over a window of w rows, computed in
 * slices of 64 rows whose sums are added in ascending row order), and
 * kept[row][0 .. min(keep, seq_len)) the top keys of scores[row] (no forced
 * entry), ascending. window >= 1, keep >= 0. scores: device fp32
 * [batch * n_heads][seq_len]; kept: device int32 [batch * n_heads]
 * [min(keep, seq_len)] (may be NULL when keep == 0). workspace: at least
 * dsa_kv_retention_workspace_bytes(...) bytes. */
dsa_status dsa_kv_retention(const void* q, const void* k, const dsa_shape* shape,
                            int32_t window, int32_t keep, float scale,
                            const int32_t* heads, int32_t n_heads, float* scores,
                            int32_t* kept, void* workspace, size_t workspace_bytes,
                            void* stream);
size_t dsa_kv_retention_workspace_bytes(const dsa_shape* shape, int32_t keep,
                                        int32_t n_heads);

/* Sparse decode attention [Novita §2: decoding attends only to the KV entries
 * a head kept; MInf §1: attention over a key set, other keys excluded]. One
 * new query row per listed head attends over cached keys:
 *   o[row] = sum over j in K(row) of softmax_j(scale * q[row] . k[j]) v[j]
 * with K(row) = keys[row][0 .. n_keys[row]) (cache positions; entries are
 * clamped into [0, seq_len) and should be distinct), or every cached key when
 * keys is NULL. The decode row comes after the whole cache, so no causal cut
 * applies; an empty key set gives zeros, and so does an empty cache
 * (seq_len 0: every list counts as empty, and k and v, which are not read,
 * may be NULL). Layout: q and o are device
 * [batch][q_heads][head_dim] (one row per head), k and v the cache as
 * [batch][kv_heads][seq_len][head_dim] with seq_len = cached keys; keys
 * device int32 [batch * n_heads][max_keys], n_keys device int32
 * [batch * n_heads]. Only listed heads of o are written. The list is cut into
 * splits over work-groups whose partial (max, sum, output) are merged in split
 * order, so results are bit-reproducible. workspace: at least
 * dsa_sparse_decode_workspace_bytes(shape, max_keys, n_heads) bytes, with
 * max_keys = -1 when keys is NULL. */
dsa_status dsa_sparse_decode(const void* q, const void* k, const void* v, void* o,
                             const dsa_shape* shape, float scale, const int32_t* heads,
                             int32_t n_heads, const int32_t* keys, int32_t max_keys,
                             const int32_t* n_keys, void* workspace, size_t workspace_bytes,
                             void* stream);
size_t dsa_sparse_decode_workspace_bytes(const dsa_shape* shape, int32_t max_keys,
                                         int32_t n_heads);

/* Size of the static device scratch of dsa_sparse_decode_noalloc. */
#define DSA_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)

/* dsa_sparse_decode for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and results, with the split partials in a fixed device
 * array of the library instead of a workspace argument. Nothing is allocated
 * and no allocating routine is called. The array is DSA_DECODE_NOALLOC_MAX_BYTES
 * bytes, one copy per GPU, held until the process ends; its address is looked
 * up on a device's first call (with that device current, which must be the
 * device of `stream`). A call whose partials need more than that
 * (dsa_sparse_decode_workspace_bytes(shape, max_keys, n_heads) >
 * DSA_DECODE_NOALLOC_MAX_BYTES) returns DSA_ERR_WORKSPACE before any HIP call.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (other streams, other threads) race and must be serialised by the
 * caller. Each call writes every partial it reads, so nothing carries over
 * from the previous call's contents. */
dsa_status dsa_sparse_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                     const dsa_shape* shape, float scale, const int32_t* heads,
                                     int32_t n_heads, const int32_t* keys, int32_t max_keys,
                                     const int32_t* n_keys, void* stream);

/* ======================================================================
 * Hierarchical chunk pruning [InfiniteHiP summary, section "modular
 * hierarchical token pruning" (模块化分层令牌剪枝算法): the keys are cut into
 * fixed-length chunks, the highest-scoring token of each chunk is found, only
 * the best chunks go on to the next stage, and stacked stages refine the
 * block-sparse mask of a query].
 *
 * A query vector sees the keys j < limit. A token's score is
 * scale * q . k_j (scale <= 0: 1/sqrt(head_dim)); a chunk's score is the
 * largest score of its visible tokens, found exactly. Stage s keeps the
 * keep[s] best candidates of length chunk[s]: stage 1's candidates are the
 * chunks of [0, limit), a later stage's the sub-chunks of the chunks the stage
 * before kept that hold a visible key. Ranking: the chunk holding key
 * limit - 1 first (forced), then higher score, then lower chunk id (-0 counts
 * as +0, NaN as -inf). The result is the last stage's kept chunk ids,
 * ascending, min(keep, candidates) of them.
 * ====================================================================== */
#define DSA_PRUNE_MAX_STAGES 4
#define DSA_PRUNE_MAX_CANDIDATES 4096
typedef struct {
  int32_t n_stages;                     /* 1 .. DSA_PRUNE_MAX_STAGES */
  int32_t chunk[DSA_PRUNE_MAX_STAGES];  /* keys per chunk: multiples of 64, strictly
                                           decreasing, each dividing the one before */
  int32_t keep[DSA_PRUNE_MAX_STAGES];   /* chunks kept by the stage, >= 1 */
} dsa_prune_stages;
/* Stage lists are checked on the host: a malformed list is
 * DSA_ERR_INVALID_ARG; more than DSA_PRUNE_MAX_CANDIDATES candidates in a stage
 * (stage 1: ceil(seq_len / chunk[0]); stage s: keep[s-1] * chunk[s-1] /
 * chunk[s]) is DSA_ERR_UNSUPPORTED. */

/* The pruning stages for explicit query vectors. qu: device
 * [batch * n_heads][units][head_dim] (rows: batch-major, then listed heads),
 * dtype qu_dtype (DSA_BF16 or DSA_F32); k: the device cache
 * [batch][kv_heads][seq_len][head_dim] of shape->dtype; listed head h reads kv
 * head h / (q_heads / kv_heads). Unit u of a row sees the keys
 * j < min(seq_len, (u + 1) * unit_rows), or all seq_len keys when unit_rows is
 * 0 (decode rows). Outputs: sel device int32 [rows][units][keep of the last
 * stage] (entries past the count unwritten), n_sel [rows][units]; block_max
 * (optional, device fp32 [rows][units][ceil(seq_len / 64)]) receives the
 * largest token score of every visible 64-key block, which is what the stages
 * rank (a chunk's score is the largest of its blocks'); blocks a unit does not
 * see are unwritten. When block_max is NULL it lives in the workspace:
 * dsa_hier_prune_workspace_bytes(shape, units, n_heads) bytes. */
dsa_status dsa_hier_prune(const void* qu, int32_t qu_dtype, int32_t units, int32_t unit_rows,
                          const void* k, const dsa_shape* shape, const dsa_prune_stages* stages,
                          float scale, const int32_t* heads, int32_t n_heads, float* block_max,
                          int32_t* sel, int32_t* n_sel, void* workspace, size_t workspace_bytes,
                          void* stream);
size_t dsa_hier_prune_workspace_bytes(const dsa_shape* shape, int32_t units, int32_t n_heads);

/* Key lists of kept chunks, for dsa_sparse_decode: keys[r][i * chunk + t] =
 * sel[r][i] * chunk + t for the n_sel[r] chunks of row r (ids ascending, as
 * the pruning returns them), n_keys[r] = those keys below seq_len (only the
 * last chunk can be cut). sel: device int32 [rows][max_sel]; keys: device
 * int32 [rows][max_sel * chunk]. */
dsa_status dsa_chunks_to_keys(const int32_t* sel, const int32_t* n_sel, int32_t rows,
                              int32_t max_sel, int32_t chunk, int32_t seq_len, int32_t* keys,
                              int32_t* n_keys, void* stream);

/* Decode over pruned keys [InfiniteHiP summary: pruning for attention
 * decoding; Novita §2: decoding attends only to the kept entries]: each listed
 * head's new row (q, o as in dsa_sparse_decode) is the query vector, limit =
 * seq_len; the stages select chunks, and the row attends over their keys with
 * the softmax of dsa_sparse_decode (an empty cache gives zero rows, as there).
 * workspace: at least
 * dsa_hier_sparse_decode_workspace_bytes(shape, stages, n_heads) bytes. */
dsa_status dsa_hier_sparse_decode(const void* q, const void* k, const void* v, void* o,
                                  const dsa_shape* shape, const dsa_prune_stages* stages, float scale,
                                  const int32_t* heads, int32_t n_heads, void* workspace,
                                  size_t workspace_bytes, void* stream);
size_t dsa_hier_sparse_decode_workspace_bytes(const dsa_shape* shape,
                                              const dsa_prune_stages* stages, int32_t n_heads);

/* Prefill heads with the pruning as their block estimator [InfiniteHiP
 * summary: stages refine the block-sparse mask per query block; MInf §2.2
 * Block-Sparse Head for the pooled query and the block attention]: query block
 * a's query vector is its mean-pooled row, limit = min(seq_len, 64 (a + 1));
 * the last stage's chunk length must be 64, so the kept chunks are key blocks;
 * block a then attends over them, causally. Layout and head list as in
 * dsa_block_sparse_attention. The block maxima take
 * rows * nb * nb * 4 bytes of the workspace (nb = ceil(seq_len / 64)): this
 * form is for contexts up to about 128K. workspace: at least
 * dsa_hier_block_sparse_workspace_bytes(shape, stages, n_heads) bytes. */
dsa_status dsa_hier_block_sparse_attention(const void* q, const void* k, const void* v, void* o,
                                           const dsa_shape* shape, const dsa_prune_stages* stages,
                                           float scale, const int32_t* heads, int32_t n_heads,
                                           void* workspace, size_t workspace_bytes, void* stream);
size_t dsa_hier_block_sparse_workspace_bytes(const dsa_shape* shape,
                                             const dsa_prune_stages* stages, int32_t n_heads);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
