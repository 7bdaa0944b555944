// Host-side launchers of the gfx950 kernels (each defined in its own .hip file).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace dsa {

// ---- sparse attention (sparse_attention.hip) ----
struct VsIndex {       // vertical-slash sparse format
  const int32_t* iv;   // [rows][max_iv][2] (d_lo, d_hi) ascending
  const int32_t* n_iv; // [rows]
  int32_t max_iv;
  const int32_t* cols;   // [rows][nb][max_cols]
  const int32_t* n_cols; // [rows][nb]
  int32_t max_cols;
};
struct BlockIndex {    // explicit key-block lists
  const int32_t* sel;  // [rows][nb][max_sel]
  const int32_t* n_sel;
  int32_t max_sel;
};
struct StreamIndex {   // closed-form A-shape
  int32_t init_blocks, local_blocks;
};
enum : int8_t { PAT_VS = 0, PAT_BS = 1, PAT_STREAM = 2 };  // pattern of a head

// Order of the attention work items (row, query block): batch, then the
// groups of listed heads that share a kv head (kv-head order), then query
// blocks (latest first), then the heads of the group. The heads of a group
// read the same K/V rows, and neighbouring query blocks of a head read largely
// the same key ranges, so items close in this order share data.
struct WorkOrder {
  int16_t order[MAX_HEADS];       // listed-head positions sorted by kv head
  int16_t gstart[MAX_HEADS + 1];  // group g is order[gstart[g] .. gstart[g+1])
  int32_t n_groups;
};
WorkOrder make_work_order(const HeadMap& hm);
// pattern by pattern (kind[t] of listed head t: vertical-slash, block-sparse,
// streaming), each pattern's heads grouped by kv head as above
WorkOrder make_work_order(const HeadMap& hm, const int8_t* kind);

// Work-group -> (row, unit) for a grid of rows x units items, units visited
// latest first. The hardware deals consecutive work-group ids round-robin over
// the 8 XCDs, each with its own L2. Work items, ordered by WorkOrder (batch,
// kv group, unit, head of the group), are cut into chunks of XCD_CHUNK and the
// chunks are dealt round-robin to the XCDs: the work-groups an XCD runs at one
// time then share K/V rows in its L2, and every XCD still gets a mix of all kv
// groups and unit positions (whose costs differ). A tail shorter than NUM_XCD
// chunks keeps the identity mapping.
constexpr int32_t NUM_XCD = 8;
#ifndef DSA_XCD_CHUNK
#define DSA_XCD_CHUNK 32
#endif
constexpr int32_t XCD_CHUNK = DSA_XCD_CHUNK;
__device__ __forceinline__ void work_item(const HeadMap& hm, const WorkOrder& wo, int32_t units,
                                          int32_t& row, int32_t& unit) {
  const int32_t N = gridDim.x, i = blockIdx.x;
  const int32_t T = (N / (NUM_XCD * XCD_CHUNK)) * (NUM_XCD * XCD_CHUNK);
  int32_t w = i;
  if (i < T) {
    const int32_t xcd = i % NUM_XCD, k = i / NUM_XCD;
    w = ((k / XCD_CHUNK) * NUM_XCD + xcd) * XCD_CHUNK + k % XCD_CHUNK;
  }
  const int32_t n = hm.n, per_b = units * n;
  const int32_t b = w / per_b, w2 = w - b * per_b;
  int32_t gi = 0;
  while (gi + 1 < wo.n_groups && wo.gstart[gi + 1] * units <= w2) ++gi;
  const int32_t g0 = wo.gstart[gi], size = wo.gstart[gi + 1] - g0;
  const int32_t off = w2 - g0 * units;
  const int32_t u_idx = off / size, j = off - u_idx * size;
  row = b * n + wo.order[g0 + j];
  unit = units - 1 - u_idx;
}

struct AttnArgs {
  const void* q; const void* k; const void* v; void* o;
  int32_t seq_len, head_dim, dtype;
  int32_t rows;        // batch * listed heads
  float scale_log2;    // softmax scale * log2(e)
  HeadMap hm;
  WorkOrder wo;
};

hipError_t launch_attention_vs(const AttnArgs& a, const VsIndex& ix, hipStream_t s);
hipError_t launch_attention_blocks(const AttnArgs& a, const BlockIndex& ix, hipStream_t s);
hipError_t launch_attention_stream(const AttnArgs& a, const StreamIndex& ix, hipStream_t s);

// One launch over the heads of a mixed layer: listed head t (of a.hm) follows
// pattern kind[t]; its rows in that pattern's index arrays are
// b * (heads of that pattern) + slot[t]. bf16 work items follow a.wo.
struct MixedIndex {
  VsIndex vs;
  BlockIndex bs;
  StreamIndex st;
  int32_t n_vs, n_bs;
  int8_t kind[MAX_HEADS];
  int16_t slot[MAX_HEADS];
};
hipError_t launch_attention_mixed(const AttnArgs& a, const MixedIndex& ix, hipStream_t s);

// ---- vertical-slash estimate (vs_estimate.hip) ----
// keys per estimator work-group, at most: 1024 measured fastest at 128K-1M
// (each wave loads its 64-row Q window once per chunk; 256: 12% slower at
// 1M); shorter rows take 512 down to 64 (est_chunk_keys)
constexpr int EST_CHUNK = 1024;
struct EstArgs {
  const void* q; const void* k;
  int32_t seq_len, head_dim, dtype, last_q;  // last_q: window rows of this launch (<= 64)
  int32_t win_start;   // sequence row of window row 0 (seq_len - lq_eff() for the last rows)
  int32_t add_v;       // 0: write v, 1: add into v (window slices after the first)
  int32_t want_s;      // 0: no slash scores (s_scores and s_part unused)
  int32_t rows;
  float scale_log2;
  HeadMap hm;
  WorkOrder wo;
  float* v_scores; float* s_scores;       // [rows][seq_len]
  float* part_stats;  // [rows][nchunks][64][2]
  float* row_stats;   // [rows][64]
  float* s_part;      // [rows][nchunks][chunk + 63]
  int32_t chunk;      // keys per work-group (est_chunk_keys; set by est_carve)
  __host__ __device__ int32_t lq_eff() const { return last_q < seq_len ? last_q : seq_len; }
};
int32_t est_chunk_keys(int32_t seq_len);
size_t est_workspace_bytes(int32_t rows, int32_t seq_len);
void est_carve(EstArgs& a, void* ws);
hipError_t launch_vs_estimate(const EstArgs& a, hipStream_t s);
// v over a window of `window` rows ending at the last row, in slices of 64
// rows, no slash scores; workspace from est_window_workspace_bytes, laid out
// by est_window_carve
size_t est_window_workspace_bytes(int32_t rows, int32_t seq_len);
void est_window_carve(EstArgs& a, void* ws);
hipError_t launch_window_column_scores(EstArgs a, int32_t window, hipStream_t s);

// ---- sparse decode (decode.hip) ----
struct DecodeArgs {
  const void* q; const void* k; const void* v; void* o;  // q, o: [batch][q_heads][1][D]
  int32_t n, head_dim, dtype, rows;   // n: cached keys
  int32_t splits, split_keys;         // set by launch_decode
  int32_t bundles_per_batch;          // whole cache: head bundles per batch (set by launch_decode)
  float scale_log2;
  HeadMap hm;
  WorkOrder wo;
  const int32_t* keys;    // [rows][max_keys] cache positions, or NULL for all n
  int32_t max_keys;
  const int32_t* n_keys;  // [rows]
  float* part;            // [rows][splits][2 + D]: (max, sum, output) per split
};
int32_t decode_splits(int32_t rows, int32_t max_keys, int32_t& split_keys);
size_t decode_workspace_bytes(int32_t rows, int32_t max_keys, int32_t head_dim);
hipError_t launch_decode(DecodeArgs a, hipStream_t s);
// Device address (on the current device) and size of the static scratch that
// the allocation-free decode entry point uses for its split partials.
hipError_t decode_static_scratch(float** ptr, size_t* bytes);

// ---- top-k (topk.hip) ----
// scratch of launch_topk_rows (0 when one work-group per row selects: rows
// shorter than 64K entries)
size_t topk_workspace_bytes(int32_t rows, int32_t n, int32_t k);
hipError_t launch_topk_rows(const float* scores, int32_t rows, int32_t n, int32_t k,
                            int32_t forced, int32_t* out, void* ws, hipStream_t s);
// per (row, query block a): top-min(topk, a+1) of logits[row][a][0..a], a forced
hipError_t launch_block_topk(const float* logits, int32_t rows, int32_t nb, int32_t topk,
                             int32_t* sel, int32_t* n_sel, hipStream_t s);

// ---- hierarchical chunk pruning (hier_prune.hip) ----
constexpr int32_t PR_MAX_STAGES = 4;
constexpr int32_t PR_MAX_CAND = 4096;  // candidates of one stage
struct PruneArgs {
  // query vectors: qu_full ? [batch][q_heads][units][D] (rows map through hm)
  //                        : [rows][units][D]
  const void* qu; int32_t qu_dtype, qu_full;
  const void* k; int32_t k_dtype;         // [batch][kv_heads][n][D]
  int32_t n, head_dim, units, rows;
  int32_t unit_rows;   // unit u sees keys < min(n, (u+1) unit_rows); 0: all n
  float scale;
  HeadMap hm;
  WorkOrder wo;
  float* fine;         // [rows][units][nbf]: largest score of each 64-key block
  int32_t nbf, ntiles; // set by launch_prune
  int32_t n_stages;
  int32_t chunk_blocks[PR_MAX_STAGES];  // chunk lengths in 64-key blocks
  int32_t keep[PR_MAX_STAGES];
  int32_t* sel;        // [rows][units][max_sel] kept chunk ids of the last stage
  int32_t* n_sel;      // [rows][units]
  int32_t max_sel;
};
hipError_t launch_prune(PruneArgs a, hipStream_t s);
// key lists of kept chunks: keys [rows][max_sel * chunk], n_keys [rows]
hipError_t launch_chunks_to_keys(const int32_t* sel, const int32_t* n_sel, int32_t rows, int32_t max_sel,
                                 int32_t chunk, int32_t n, int32_t* keys, int32_t* n_keys, hipStream_t s);

// ---- vertical-slash index builder (vs_index.hip) ----
hipError_t launch_vs_build_index(const int32_t* V, int32_t nv, const int32_t* S, int32_t ns,
                                 int32_t rows, int32_t seq_len, int32_t* iv, int32_t* n_iv,
                                 int32_t* cols, int32_t* n_cols, hipStream_t s);

// ---- block-sparse estimate (bs_estimate.hip) ----
// rows = (batch, listed head of hm) over a tensor with hm.q_heads heads
hipError_t launch_pool(const void* x, int32_t dtype, int32_t seq_len, int32_t head_dim,
                       int32_t rows, const HeadMap& hm, float* out, hipStream_t s);
// Logits of rows [row0, row0 + rows) of a call: qp and logits point at row0's
// data. kp: with kv_map false it points at row0's data too (row r scores
// against kp row r); with kv_map true it is the whole pooled-K array
// [batch * kv_heads][nb][dim] and row r reads kp row b * kv_heads + kv head.
// split: scratch of block_split_elems(rows, nb, head_dim) bf16 values (the
// hi / lo splits of the rows' pooled Q and K).
hipError_t launch_block_logits(const float* qp, const float* kp, int32_t row0, int32_t rows,
                               int32_t nb, int32_t head_dim, float scale, bool kv_map,
                               const HeadMap& hm, uint16_t* split, float* logits, hipStream_t s);
inline size_t block_split_elems(int32_t rows, int32_t nb, int32_t head_dim) {
  return (size_t)4 * rows * nb * head_dim;
}

}  // namespace dsa
