// C ABI of the library (include/dsa.h): host-side argument checks, workspace
// layout and kernel dispatch. Every argument error is reported before any
// work is enqueued; nothing here synchronises the stream or allocates.
#include <math.h>
#include <string.h>
#include <algorithm>

#include "../../include/dsa.h"
#include "kernels.hpp"

using namespace dsa;

namespace {

constexpr size_t ALIGN = 256;
constexpr size_t LOGITS_BUDGET = (size_t)1 << 30;  // block-logit scratch per launch group

size_t al(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }

// Lays out workspace regions from a base address. The base is NULL when only
// the size is wanted, so addresses are formed as integers (pointer arithmetic
// on NULL is undefined).
struct Carver {
  uintptr_t p;
  size_t used = 0;
  template <typename T>
  T* take(size_t count) {
    T* r = reinterpret_cast<T*>(p + used);
    used += al(count * sizeof(T));
    return r;
  }
};

dsa_status check_shape(const dsa_shape* s) {
  if (!s) return DSA_ERR_INVALID_ARG;
  if (s->batch < 0 || s->q_heads <= 0 || s->kv_heads <= 0 || s->seq_len < 0)
    return DSA_ERR_INVALID_ARG;
  if (s->q_heads % s->kv_heads != 0) return DSA_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (s->dtype != DSA_BF16 && s->dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  // one head's slab is addressed with 32-bit byte offsets
  const int64_t slab = (int64_t)s->seq_len * s->head_dim * (s->dtype == DSA_BF16 ? 2 : 4);
  if (slab >= ((int64_t)1 << 31)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// Head list -> HeadMap over a tensor with `heads_total` heads.
dsa_status make_map(int32_t heads_total, int32_t kv_heads, const int32_t* heads, int32_t n_heads,
                    HeadMap& hm) {
  memset(&hm, 0, sizeof(hm));
  hm.q_heads = heads_total;
  hm.kv_heads = kv_heads;
  if (!heads) {
    if (heads_total > MAX_HEADS) return DSA_ERR_UNSUPPORTED;
    hm.n = heads_total;
    for (int32_t i = 0; i < heads_total; ++i) hm.h[i] = i;
    return DSA_OK;
  }
  if (n_heads < 0) return DSA_ERR_INVALID_ARG;
  if (n_heads > MAX_HEADS) return DSA_ERR_UNSUPPORTED;
  hm.n = n_heads;
  for (int32_t i = 0; i < n_heads; ++i) {
    if (heads[i] < 0 || heads[i] >= heads_total) return DSA_ERR_INVALID_ARG;
    for (int32_t j = 0; j < i; ++j)
      if (heads[j] == heads[i]) return DSA_ERR_INVALID_ARG;
    hm.h[i] = heads[i];
  }
  return DSA_OK;
}

float eff_scale(float scale, int32_t head_dim) {
  return scale > 0.f ? scale : 1.0f / sqrtf((float)head_dim);
}

int32_t nblocks(int32_t n) { return (n + BLOCK - 1) / BLOCK; }

// A prefill call over no row or no token has nothing to read or write: its
// data pointers may then be NULL (zero-size tensors have no address).
bool no_work(const dsa_shape* s, int32_t listed_heads) {
  return s->batch == 0 || s->seq_len == 0 || listed_heads == 0;
}

dsa_status hip_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

AttnArgs attn_args(const void* q, const void* k, const void* v, void* o, const dsa_shape* s,
                   float scale, const HeadMap& hm) {
  AttnArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.seq_len = s->seq_len;
  a.head_dim = s->head_dim;
  a.dtype = s->dtype;
  a.rows = s->batch * hm.n;
  a.scale_log2 = eff_scale(scale, s->head_dim) * LOG2E;
  a.hm = hm;
  a.wo = make_work_order(hm);
  return a;
}

// ---- vertical-slash workspace layout ----
struct VsWork {
  void* est; float* v; float* s; int32_t* V; int32_t* S; int32_t* iv; int32_t* n_iv;
  int32_t* cols; int32_t* n_cols; void* tk;
};
size_t vs_layout(int32_t rows, int32_t n, int32_t vk, int32_t sk, void* base, VsWork* w) {
  // no rows or no tokens: nothing is launched, so no workspace is needed
  if (rows == 0 || n == 0) {
    if (w) *w = VsWork{};
    return 0;
  }
  Carver c{reinterpret_cast<uintptr_t>(base)};
  const int32_t nb = nblocks(n);
  void* est = c.take<char>(est_workspace_bytes(rows, n));
  float* v = c.take<float>((size_t)rows * n);
  float* s = c.take<float>((size_t)rows * n);
  int32_t* V = c.take<int32_t>((size_t)rows * vk);
  int32_t* S = c.take<int32_t>((size_t)rows * sk);
  int32_t* iv = c.take<int32_t>((size_t)rows * sk * 2);
  int32_t* n_iv = c.take<int32_t>((size_t)rows);
  int32_t* cols = c.take<int32_t>((size_t)rows * nb * vk);
  int32_t* n_cols = c.take<int32_t>((size_t)rows * nb);
  // one top-k scratch serves both selections (they run in turn on one stream)
  const size_t tkb = std::max(topk_workspace_bytes(rows, n, vk), topk_workspace_bytes(rows, n, sk));
  void* tk = c.take<char>(tkb);
  if (w) *w = VsWork{est, v, s, V, S, iv, n_iv, cols, n_cols, tk};
  return c.used;
}

// ---- block-sparse workspace layout ----
int32_t logit_rows_per_group(int32_t rows, int32_t nb) {
  const size_t per_row = (size_t)nb * nb * sizeof(float);
  size_t g = per_row ? LOGITS_BUDGET / per_row : (size_t)rows;
  if (g < 1) g = 1;
  if (g > (size_t)rows) g = (size_t)rows;
  return (int32_t)g;
}
struct BsWork { float* qp; float* kp; float* logits; uint16_t* split; int32_t* sel; int32_t* n_sel; };
size_t bs_layout(const dsa_shape* s, int32_t rows, int32_t topk, void* base, BsWork* w) {
  Carver c{reinterpret_cast<uintptr_t>(base)};
  const int32_t nb = nblocks(s->seq_len), D = s->head_dim;
  const int32_t ke = topk < nb ? topk : nb;
  const int32_t grp = rows ? logit_rows_per_group(rows, nb) : 0;
  float* qp = c.take<float>((size_t)rows * nb * D);
  // pooled K of every kv head the listed heads may read (none without rows)
  float* kp = c.take<float>(rows ? (size_t)s->batch * s->kv_heads * nb * D : 0);
  float* lg = c.take<float>((size_t)grp * nb * nb);
  uint16_t* split = c.take<uint16_t>(block_split_elems(grp, nb, D));
  int32_t* sel = c.take<int32_t>((size_t)rows * nb * ke);
  int32_t* n_sel = c.take<int32_t>((size_t)rows * nb);
  if (w) *w = BsWork{qp, kp, lg, split, sel, n_sel};
  return c.used;
}

// scratch of dsa_bs_select: the logits of one group of rows (unless the
// caller takes them all) and that group's bf16 splits (sized for the largest
// head dimension)
struct BsSelectScratch { float* logits; uint16_t* split; };
size_t bs_select_scratch(int32_t rows, int32_t nb, bool with_logits, void* base, BsSelectScratch* w) {
  Carver c{reinterpret_cast<uintptr_t>(base)};
  const int32_t grp = logit_rows_per_group(rows, nb);
  float* lg = c.take<float>(with_logits ? (size_t)grp * nb * nb : 0);
  uint16_t* split = c.take<uint16_t>(block_split_elems(grp, nb, 128));
  if (w) *w = BsSelectScratch{lg, split};
  return c.used;
}

// block logits + per-block top-k, in groups of rows bounded by the scratch size
hipError_t bs_select_rows(const float* qp, const float* kp, int32_t rows, int32_t nb, int32_t D,
                          float scale, int32_t topk, bool kv_map, const HeadMap& hm,
                          float* logits, bool logits_full, uint16_t* split, int32_t* sel, int32_t* n_sel,
                          hipStream_t st) {
  const int32_t ke = topk < nb ? topk : nb;
  const int32_t grp = logit_rows_per_group(rows, nb);
  for (int32_t r0 = 0; r0 < rows; r0 += grp) {
    const int32_t nr = rows - r0 < grp ? rows - r0 : grp;
    float* lg = logits_full ? logits + (size_t)r0 * nb * nb : logits;
    const float* kpr = kv_map ? kp : kp + (size_t)r0 * nb * D;
    hipError_t e = launch_block_logits(qp + (size_t)r0 * nb * D, kpr, r0, nr, nb, D, scale,
                                       kv_map, hm, split, lg, st);
    if (e != hipSuccess) return e;
    e = launch_block_topk(lg, nr, nb, topk, sel + (size_t)r0 * nb * ke, n_sel + (size_t)r0 * nb, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}


// vertical-slash index of the heads of hm: scores, the two top-k, the sparse
// format, into w (laid out by vs_layout for batch * hm.n rows)
hipError_t vs_index_stages(const void* q, const void* k, const dsa_shape* shape, int32_t vk, int32_t sk,
                           int32_t last_q, float scale, const HeadMap& hm, const VsWork& w, hipStream_t s) {
  const int32_t rows = shape->batch * hm.n, n = shape->seq_len;
  EstArgs ea;
  ea.q = q; ea.k = k;
  ea.seq_len = n; ea.head_dim = shape->head_dim; ea.dtype = shape->dtype;
  ea.last_q = last_q; ea.rows = rows;
  ea.win_start = ea.seq_len - ea.lq_eff(); ea.add_v = 0; ea.want_s = 1;
  ea.scale_log2 = eff_scale(scale, shape->head_dim) * LOG2E;
  ea.hm = hm;
  ea.wo = make_work_order(hm);
  ea.v_scores = w.v; ea.s_scores = w.s;
  est_carve(ea, w.est);
  hipError_t e = launch_vs_estimate(ea, s);
  if (e == hipSuccess) e = launch_topk_rows(w.v, rows, n, vk, -1, w.V, w.tk, s);
  if (e == hipSuccess) e = launch_topk_rows(w.s, rows, n, sk, 0, w.S, w.tk, s);
  if (e == hipSuccess) e = launch_vs_build_index(w.V, vk, w.S, sk, rows, n, w.iv, w.n_iv, w.cols, w.n_cols, s);
  return e;
}

// block-sparse index of the heads of hm: pooled Q and K, block logits and the
// per-block top-k, into w (laid out by bs_layout for batch * hm.n rows)
hipError_t bs_index_stages(const void* q, const void* k, const dsa_shape* shape, int32_t topk, float scale,
                           const HeadMap& hm, const BsWork& w, hipStream_t s) {
  const int32_t rows = shape->batch * hm.n, n = shape->seq_len, nb = nblocks(n), D = shape->head_dim;
  // pooled K for every kv head the listed heads read
  HeadMap kvm;
  memset(&kvm, 0, sizeof(kvm));
  kvm.q_heads = kvm.kv_heads = shape->kv_heads;
  kvm.n = shape->kv_heads;
  for (int32_t i = 0; i < kvm.n; ++i) kvm.h[i] = i;
  hipError_t e = launch_pool(q, shape->dtype, n, D, rows, hm, w.qp, s);
  if (e == hipSuccess) e = launch_pool(k, shape->dtype, n, D, shape->batch * kvm.n, kvm, w.kp, s);
  if (e == hipSuccess)
    e = bs_select_rows(w.qp, w.kp, rows, nb, D, eff_scale(scale, D), topk, true, hm, w.logits, false,
                       w.split, w.sel, w.n_sel, s);
  return e;
}

// patterns[q_heads] -> the map of every processed head (ascending), the maps
// of the VS and BS heads and each head's pattern and position in its list
dsa_status parse_patterns(const dsa_shape* shape, const int32_t* patterns, HeadMap& all, HeadMap& vs,
                          HeadMap& bs, MixedIndex& ix) {
  if (!patterns) return DSA_ERR_INVALID_ARG;
  if (shape->q_heads > MAX_HEADS) return DSA_ERR_UNSUPPORTED;
  int32_t lists[3][MAX_HEADS], counts[3] = {0, 0, 0}, listed[MAX_HEADS], n_listed = 0;
  memset(&ix, 0, sizeof(ix));
  for (int32_t h = 0; h < shape->q_heads; ++h) {
    const int32_t p = patterns[h];
    if (p == DSA_PATTERN_NONE) continue;
    if (p != DSA_PATTERN_VS && p != DSA_PATTERN_BS && p != DSA_PATTERN_STREAM) return DSA_ERR_INVALID_ARG;
    const int8_t kind = p == DSA_PATTERN_VS ? PAT_VS : p == DSA_PATTERN_BS ? PAT_BS : PAT_STREAM;
    ix.kind[n_listed] = kind;
    ix.slot[n_listed] = (int16_t)counts[kind];
    lists[kind][counts[kind]++] = h;
    listed[n_listed++] = h;
  }
  dsa_status st = make_map(shape->q_heads, shape->kv_heads, listed, n_listed, all);
  if (st == DSA_OK) st = make_map(shape->q_heads, shape->kv_heads, lists[PAT_VS], counts[PAT_VS], vs);
  if (st == DSA_OK) st = make_map(shape->q_heads, shape->kv_heads, lists[PAT_BS], counts[PAT_BS], bs);
  ix.n_vs = counts[PAT_VS];
  ix.n_bs = counts[PAT_BS];
  return st;
}

size_t mixed_layout(const dsa_shape* shape, int32_t n_vs, int32_t n_bs, int32_t vk, int32_t sk, int32_t topk,
                    void* base, VsWork* vw, BsWork* bw) {
  const int32_t n = shape->seq_len;
  const size_t vbytes = n_vs ? vs_layout(shape->batch * n_vs, n, vk, sk, nullptr, nullptr) : 0;
  if (vw && n_vs) vs_layout(shape->batch * n_vs, n, vk, sk, base, vw);
  char* bbase = base ? static_cast<char*>(base) + vbytes : nullptr;
  const size_t bbytes = n_bs ? bs_layout(shape, shape->batch * n_bs, topk, nullptr, nullptr) : 0;
  if (bw && n_bs) bs_layout(shape, shape->batch * n_bs, topk, bbase, bw);
  return vbytes + bbytes;
}
}  // namespace

namespace dsa {
WorkOrder make_work_order(const HeadMap& hm) {
  WorkOrder wo;
  memset(&wo, 0, sizeof(wo));
  const int32_t G = hm.q_heads / hm.kv_heads;
  int32_t pos = 0;
  for (int32_t kv = 0; kv < hm.kv_heads; ++kv) {
    const int32_t start = pos;
    for (int32_t t = 0; t < hm.n; ++t)
      if (hm.h[t] / G == kv) wo.order[pos++] = (int16_t)t;
    if (pos > start) wo.gstart[wo.n_groups++] = (int16_t)start;
  }
  wo.gstart[wo.n_groups] = (int16_t)pos;
  return wo;
}
WorkOrder make_work_order(const HeadMap& hm, const int8_t* kind) {
  WorkOrder wo;
  memset(&wo, 0, sizeof(wo));
  const int32_t G = hm.q_heads / hm.kv_heads;
  int32_t pos = 0;
  for (int8_t pat : {PAT_VS, PAT_BS, PAT_STREAM})
    for (int32_t kv = 0; kv < hm.kv_heads; ++kv) {
      const int32_t start = pos;
      for (int32_t t = 0; t < hm.n; ++t)
        if (kind[t] == pat && hm.h[t] / G == kv) wo.order[pos++] = (int16_t)t;
      if (pos > start) wo.gstart[wo.n_groups++] = (int16_t)start;
    }
  wo.gstart[wo.n_groups] = (int16_t)pos;
  return wo;
}
}  // namespace dsa

extern "C" {

const char* dsa_status_string(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape, dtype or parameter";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

// ------------------------------------------------------------------ VS
size_t dsa_vs_estimate_workspace_bytes(const dsa_shape* shape, int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || n_heads < 0) return 0;
  return est_workspace_bytes(shape->batch * n_heads, shape->seq_len);
}

dsa_status dsa_vs_estimate(const void* q, const void* k, const dsa_shape* shape, int32_t last_q,
                           float scale, const int32_t* heads, int32_t n_heads, float* v_scores,
                           float* s_scores, void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (last_q < 1 || last_q > 64) return DSA_ERR_UNSUPPORTED;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !v_scores || !s_scores) return DSA_ERR_INVALID_ARG;
  const int32_t rows = shape->batch * hm.n;
  const size_t need = est_workspace_bytes(rows, shape->seq_len);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  EstArgs a;
  a.q = q; a.k = k;
  a.seq_len = shape->seq_len; a.head_dim = shape->head_dim; a.dtype = shape->dtype;
  a.last_q = last_q; a.rows = rows;
  a.win_start = a.seq_len - a.lq_eff(); a.add_v = 0; a.want_s = 1;
  a.scale_log2 = eff_scale(scale, shape->head_dim) * LOG2E;
  a.hm = hm;
  a.wo = make_work_order(hm);
  a.v_scores = v_scores; a.s_scores = s_scores;
  est_carve(a, workspace);
  return hip_status(launch_vs_estimate(a, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ KV retention
size_t dsa_kv_retention_workspace_bytes(const dsa_shape* shape, int32_t keep, int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || n_heads < 0 || keep < 0) return 0;
  const int32_t rows = shape->batch * n_heads, n = shape->seq_len;
  const size_t est = est_window_workspace_bytes(rows, n);
  const size_t tk = topk_workspace_bytes(rows, n, keep < n ? keep : n);
  return est > tk ? est : tk;  // the estimator's partials are dead when the top-k runs
}

dsa_status dsa_kv_retention(const void* q, const void* k, const dsa_shape* shape, int32_t window,
                            int32_t keep, float scale, const int32_t* heads, int32_t n_heads,
                            float* scores, int32_t* kept, void* workspace, size_t workspace_bytes,
                            void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (window < 1 || keep < 0) return DSA_ERR_INVALID_ARG;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !scores || (keep > 0 && !kept)) return DSA_ERR_INVALID_ARG;
  const int32_t rows = shape->batch * hm.n, n = shape->seq_len;
  const size_t need = dsa_kv_retention_workspace_bytes(shape, keep, hm.n);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  EstArgs a;
  a.q = q; a.k = k;
  a.seq_len = n; a.head_dim = shape->head_dim; a.dtype = shape->dtype;
  a.last_q = 64; a.rows = rows;
  a.win_start = 0; a.add_v = 0; a.want_s = 0;
  a.scale_log2 = eff_scale(scale, shape->head_dim) * LOG2E;
  a.hm = hm;
  a.wo = make_work_order(hm);
  a.v_scores = scores; a.s_scores = nullptr;
  est_window_carve(a, workspace);
  hipError_t e = launch_window_column_scores(a, window, s);
  const int32_t kk = keep < n ? keep : n;
  if (e == hipSuccess && kk > 0) e = launch_topk_rows(scores, rows, n, kk, -1, kept, workspace, s);
  return hip_status(e);
}

// ------------------------------------------------------------------ decode
size_t dsa_sparse_decode_workspace_bytes(const dsa_shape* shape, int32_t max_keys, int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || n_heads < 0 || max_keys < -1) return 0;
  const int32_t mk = max_keys < 0 ? shape->seq_len : max_keys;
  return decode_workspace_bytes(shape->batch * n_heads, mk, shape->head_dim);
}

}  // extern "C"

namespace {
// Decode step with its split partials in `workspace` (caller-owned, or the
// static scratch; `scratch_bytes` is what it holds). Returns DSA_OK without
// work when there is no decode row.
dsa_status decode_call(const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
                       float scale, const int32_t* heads, int32_t n_heads, const int32_t* keys,
                       int32_t max_keys, const int32_t* n_keys, void* workspace, size_t workspace_bytes,
                       bool static_scratch, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (keys && max_keys < 0) return DSA_ERR_INVALID_ARG;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  const int32_t rows = shape->batch * hm.n;
  if (rows == 0) return DSA_OK;  // no decode row: nothing read or written
  // an empty cache reads no key or value (the pointers of empty tensors may be NULL)
  const bool has_kv = shape->seq_len > 0;
  if (!q || !o || (has_kv && (!k || !v)) || (keys && !n_keys)) return DSA_ERR_INVALID_ARG;
  const size_t need = dsa_sparse_decode_workspace_bytes(shape, keys ? max_keys : -1, hm.n);
  if (static_scratch) {
    // checked before the scratch is looked up: a refused call makes no HIP call
    if (need > DSA_DECODE_NOALLOC_MAX_BYTES) return DSA_ERR_WORKSPACE;
    float* p = nullptr;
    size_t bytes = 0;
    if (decode_static_scratch(&p, &bytes) != hipSuccess) return DSA_ERR_HIP;
    if (bytes < need) return DSA_ERR_WORKSPACE;
    workspace = p;
  } else if (workspace_bytes < need || (need && !workspace)) {
    return DSA_ERR_WORKSPACE;
  }
  // an empty cache or empty lists still run: the rows come out as zeros
  DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.n = shape->seq_len; a.head_dim = shape->head_dim; a.dtype = shape->dtype; a.rows = rows;
  a.scale_log2 = eff_scale(scale, shape->head_dim) * LOG2E;
  a.hm = hm;
  a.wo = make_work_order(hm);
  a.keys = keys; a.max_keys = keys ? max_keys : 0; a.n_keys = n_keys;
  a.part = static_cast<float*>(workspace);
  return hip_status(launch_decode(a, static_cast<hipStream_t>(stream)));
}
}  // namespace

extern "C" {

dsa_status dsa_sparse_decode(const void* q, const void* k, const void* v, void* o,
                             const dsa_shape* shape, float scale, const int32_t* heads, int32_t n_heads,
                             const int32_t* keys, int32_t max_keys, const int32_t* n_keys,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(q, k, v, o, shape, scale, heads, n_heads, keys, max_keys, n_keys, workspace,
                     workspace_bytes, false, stream);
}

dsa_status dsa_sparse_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                     const dsa_shape* shape, float scale, const int32_t* heads,
                                     int32_t n_heads, const int32_t* keys, int32_t max_keys,
                                     const int32_t* n_keys, void* stream) {
  return decode_call(q, k, v, o, shape, scale, heads, n_heads, keys, max_keys, n_keys, nullptr, 0, true,
                     stream);
}

size_t dsa_topk_workspace_bytes(int32_t rows, int32_t n, int32_t k) {
  if (rows < 0 || n < 0 || k < 0) return 0;
  return topk_workspace_bytes(rows, n, k);
}

dsa_status dsa_topk(const float* scores, int32_t rows, int32_t n, int32_t k, int32_t forced_index,
                    int32_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || n < 0 || k < 0) return DSA_ERR_INVALID_ARG;
  if (forced_index < -1 || (forced_index >= n && forced_index != -1)) return DSA_ERR_INVALID_ARG;
  if (rows == 0 || n == 0 || k == 0) return DSA_OK;
  if (!scores || !out) return DSA_ERR_INVALID_ARG;
  const size_t need = topk_workspace_bytes(rows, n, k);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  return hip_status(launch_topk_rows(scores, rows, n, k, forced_index, out, workspace,
                                     static_cast<hipStream_t>(stream)));
}

dsa_status dsa_vs_build_index(const int32_t* V, int32_t nv, const int32_t* S, int32_t ns,
                              int32_t rows, int32_t seq_len, int32_t* intervals,
                              int32_t* n_intervals, int32_t* cols, int32_t* n_cols, void* stream) {
  if (nv < 0 || ns < 0 || rows < 0 || seq_len < 0) return DSA_ERR_INVALID_ARG;
  if (rows == 0 || seq_len == 0) return DSA_OK;
  if (!n_intervals || !n_cols || (ns && (!S || !intervals)) || (nv && (!V || !cols)))
    return DSA_ERR_INVALID_ARG;
  return hip_status(launch_vs_build_index(V, nv, S, ns, rows, seq_len, intervals, n_intervals, cols,
                                          n_cols, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_sparse_attention_vs(const void* q, const void* k, const void* v, void* o,
                                   const dsa_shape* shape, float scale, const int32_t* heads,
                                   int32_t n_heads, const int32_t* intervals,
                                   const int32_t* n_intervals, int32_t max_iv, const int32_t* cols,
                                   const int32_t* n_cols, int32_t max_cols, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (max_iv < 0 || max_cols < 0) return DSA_ERR_INVALID_ARG;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !v || !o || !n_intervals || !n_cols) return DSA_ERR_INVALID_ARG;
  if ((max_iv && !intervals) || (max_cols && !cols)) return DSA_ERR_INVALID_ARG;
  AttnArgs a = attn_args(q, k, v, o, shape, scale, hm);
  VsIndex ix{intervals, n_intervals, max_iv, cols, n_cols, max_cols};
  return hip_status(launch_attention_vs(a, ix, static_cast<hipStream_t>(stream)));
}

size_t dsa_vertical_slash_workspace_bytes(const dsa_shape* shape, int32_t vertical_topk,
                                          int32_t slash_topk, int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || n_heads < 0 || vertical_topk < 0 || slash_topk < 1) return 0;
  const int32_t n = shape->seq_len;
  const int32_t vk = vertical_topk < n ? vertical_topk : n;
  const int32_t sk = slash_topk < n ? slash_topk : n;
  return vs_layout(shape->batch * n_heads, n, vk, sk, nullptr, nullptr);
}

dsa_status dsa_vertical_slash_sparse_attention(const void* q, const void* k, const void* v, void* o,
                                               const dsa_shape* shape, int32_t vertical_topk,
                                               int32_t slash_topk, int32_t last_q, float scale,
                                               const int32_t* heads, int32_t n_heads,
                                               void* workspace, size_t workspace_bytes,
                                               void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (vertical_topk < 0 || slash_topk < 1) return DSA_ERR_INVALID_ARG;
  if (last_q < 1 || last_q > 64) return DSA_ERR_UNSUPPORTED;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !v || !o) return DSA_ERR_INVALID_ARG;
  const int32_t rows = shape->batch * hm.n, n = shape->seq_len;
  const int32_t vk = vertical_topk < n ? vertical_topk : n;
  const int32_t sk = slash_topk < n ? slash_topk : n;
  const size_t need = vs_layout(rows, n, vk, sk, nullptr, nullptr);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  VsWork w;
  vs_layout(rows, n, vk, sk, workspace, &w);

  hipError_t e = vs_index_stages(q, k, shape, vk, sk, last_q, scale, hm, w, s);
  if (e == hipSuccess) {
    AttnArgs a = attn_args(q, k, v, o, shape, scale, hm);
    e = launch_attention_vs(a, VsIndex{w.iv, w.n_iv, sk, w.cols, w.n_cols, vk}, s);
  }
  return hip_status(e);
}

// ------------------------------------------------------------------ BS
dsa_status dsa_bs_pool(const void* x, int32_t dtype, int32_t batch, int32_t x_heads, int32_t seq_len,
                       int32_t head_dim, const int32_t* heads, int32_t n_heads, float* out,
                       void* stream) {
  if (batch < 0 || x_heads <= 0 || seq_len < 0) return DSA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (dtype != DSA_BF16 && dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  HeadMap hm;
  dsa_status st = make_map(x_heads, x_heads, heads, n_heads, hm);
  if (st != DSA_OK) return st;
  if (batch == 0 || seq_len == 0 || hm.n == 0) return DSA_OK;
  if (!x || !out) return DSA_ERR_INVALID_ARG;
  return hip_status(launch_pool(x, dtype, seq_len, head_dim, batch * hm.n, hm, out,
                                static_cast<hipStream_t>(stream)));
}

size_t dsa_bs_select_workspace_bytes(int32_t rows, int32_t nb) {
  if (rows <= 0 || nb <= 0) return 0;
  return bs_select_scratch(rows, nb, true, nullptr, nullptr);
}

dsa_status dsa_bs_select(const float* qp, const float* kp, int32_t rows, int32_t nb, int32_t head_dim,
                         float scale, int32_t topk, int32_t* sel, int32_t* n_sel, float* logits,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || nb < 0 || topk < 1) return DSA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (rows == 0 || nb == 0) return DSA_OK;
  if (!qp || !kp || !sel || !n_sel) return DSA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < bs_select_scratch(rows, nb, !logits, nullptr, nullptr))
    return DSA_ERR_WORKSPACE;
  HeadMap hm;
  memset(&hm, 0, sizeof(hm));
  BsSelectScratch w;
  bs_select_scratch(rows, nb, !logits, workspace, &w);
  hipError_t e = bs_select_rows(qp, kp, rows, nb, head_dim, eff_scale(scale, head_dim), topk, false, hm,
                                logits ? logits : w.logits, logits != nullptr, w.split,
                                sel, n_sel, static_cast<hipStream_t>(stream));
  return hip_status(e);
}

dsa_status dsa_sparse_attention_blocks(const void* q, const void* k, const void* v, void* o,
                                       const dsa_shape* shape, float scale, const int32_t* heads,
                                       int32_t n_heads, const int32_t* sel, const int32_t* n_sel,
                                       int32_t max_sel, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (max_sel < 0) return DSA_ERR_INVALID_ARG;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !v || !o || !n_sel || (max_sel && !sel)) return DSA_ERR_INVALID_ARG;
  AttnArgs a = attn_args(q, k, v, o, shape, scale, hm);
  return hip_status(launch_attention_blocks(a, BlockIndex{sel, n_sel, max_sel},
                                            static_cast<hipStream_t>(stream)));
}

size_t dsa_block_sparse_workspace_bytes(const dsa_shape* shape, int32_t topk, int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || n_heads < 0 || topk < 1) return 0;
  return bs_layout(shape, shape->batch * n_heads, topk, nullptr, nullptr);
}

dsa_status dsa_block_sparse_attention(const void* q, const void* k, const void* v, void* o,
                                      const dsa_shape* shape, int32_t topk, float scale,
                                      const int32_t* heads, int32_t n_heads, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (topk < 1) return DSA_ERR_INVALID_ARG;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !v || !o) return DSA_ERR_INVALID_ARG;
  const int32_t rows = shape->batch * hm.n, n = shape->seq_len, nb = nblocks(n);
  const size_t need = bs_layout(shape, rows, topk, nullptr, nullptr);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  BsWork w;
  bs_layout(shape, rows, topk, workspace, &w);
  hipError_t e = bs_index_stages(q, k, shape, topk, scale, hm, w, s);
  if (e == hipSuccess) {
    const int32_t ke = topk < nb ? topk : nb;
    e = launch_attention_blocks(attn_args(q, k, v, o, shape, scale, hm), BlockIndex{w.sel, w.n_sel, ke}, s);
  }
  return hip_status(e);
}

// ------------------------------------------------------------------ streaming
dsa_status dsa_streaming_attention(const void* q, const void* k, const void* v, void* o,
                                   const dsa_shape* shape, int32_t init_blocks, int32_t local_blocks,
                                   float scale, const int32_t* heads, int32_t n_heads, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (init_blocks < 0 || local_blocks < 1) return DSA_ERR_INVALID_ARG;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !v || !o) return DSA_ERR_INVALID_ARG;
  AttnArgs a = attn_args(q, k, v, o, shape, scale, hm);
  return hip_status(launch_attention_stream(a, StreamIndex{init_blocks, local_blocks},
                                            static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ mixed layer
size_t dsa_mixed_sparse_attention_workspace_bytes(const dsa_shape* shape, const int32_t* patterns,
                                                  int32_t vertical_topk, int32_t slash_topk, int32_t topk) {
  if (check_shape(shape) != DSA_OK || vertical_topk < 0 || slash_topk < 1 || topk < 1) return 0;
  HeadMap all, vs, bs;
  MixedIndex ix;
  if (parse_patterns(shape, patterns, all, vs, bs, ix) != DSA_OK) return 0;
  const int32_t n = shape->seq_len;
  return mixed_layout(shape, ix.n_vs, ix.n_bs, vertical_topk < n ? vertical_topk : n,
                      slash_topk < n ? slash_topk : n, topk, nullptr, nullptr, nullptr);
}

dsa_status dsa_mixed_sparse_attention(const void* q, const void* k, const void* v, void* o,
                                      const dsa_shape* shape, const int32_t* patterns, int32_t vertical_topk,
                                      int32_t slash_topk, int32_t last_q, int32_t topk, int32_t init_blocks,
                                      int32_t local_blocks, float scale, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (vertical_topk < 0 || slash_topk < 1 || topk < 1 || init_blocks < 0 || local_blocks < 1)
    return DSA_ERR_INVALID_ARG;
  if (last_q < 1 || last_q > 64) return DSA_ERR_UNSUPPORTED;
  HeadMap all, vs, bs;
  MixedIndex ix;
  if ((st = parse_patterns(shape, patterns, all, vs, bs, ix)) != DSA_OK) return st;
  if (no_work(shape, all.n)) return DSA_OK;
  if (!q || !k || !v || !o) return DSA_ERR_INVALID_ARG;
  const int32_t n = shape->seq_len, nb = nblocks(n);
  const int32_t vk = vertical_topk < n ? vertical_topk : n;
  const int32_t sk = slash_topk < n ? slash_topk : n;
  const size_t need = mixed_layout(shape, ix.n_vs, ix.n_bs, vk, sk, topk, nullptr, nullptr, nullptr);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  VsWork vw;
  BsWork bw;
  memset(&vw, 0, sizeof(vw));
  memset(&bw, 0, sizeof(bw));
  mixed_layout(shape, ix.n_vs, ix.n_bs, vk, sk, topk, workspace, &vw, &bw);
  hipError_t e = hipSuccess;
  if (ix.n_vs) e = vs_index_stages(q, k, shape, vk, sk, last_q, scale, vs, vw, s);
  if (e == hipSuccess && ix.n_bs) e = bs_index_stages(q, k, shape, topk, scale, bs, bw, s);
  if (e == hipSuccess) {
    ix.vs = VsIndex{vw.iv, vw.n_iv, sk, vw.cols, vw.n_cols, vk};
    ix.bs = BlockIndex{bw.sel, bw.n_sel, topk < nb ? topk : nb};
    ix.st = StreamIndex{init_blocks, local_blocks};
    AttnArgs a = attn_args(q, k, v, o, shape, scale, all);
    a.wo = make_work_order(all, ix.kind);
    e = launch_attention_mixed(a, ix, s);
  }
  return hip_status(e);
}

dsa_status dsa_sparse_attention_mixed(const void* q, const void* k, const void* v, void* o,
                                      const dsa_shape* shape, float scale, const int32_t* patterns,
                                      const int32_t* intervals, const int32_t* n_intervals, int32_t max_iv,
                                      const int32_t* cols, const int32_t* n_cols, int32_t max_cols,
                                      const int32_t* sel, const int32_t* n_sel, int32_t max_sel,
                                      int32_t init_blocks, int32_t local_blocks, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (max_iv < 0 || max_cols < 0 || max_sel < 0 || init_blocks < 0 || local_blocks < 1)
    return DSA_ERR_INVALID_ARG;
  HeadMap all, vs, bs;
  MixedIndex ix;
  if ((st = parse_patterns(shape, patterns, all, vs, bs, ix)) != DSA_OK) return st;
  if (no_work(shape, all.n)) return DSA_OK;
  if (!q || !k || !v || !o) return DSA_ERR_INVALID_ARG;
  if (ix.n_vs && (!n_intervals || !n_cols || (max_iv && !intervals) || (max_cols && !cols)))
    return DSA_ERR_INVALID_ARG;
  if (ix.n_bs && (!n_sel || (max_sel && !sel))) return DSA_ERR_INVALID_ARG;
  ix.vs = VsIndex{intervals, n_intervals, max_iv, cols, n_cols, max_cols};
  ix.bs = BlockIndex{sel, n_sel, max_sel};
  ix.st = StreamIndex{init_blocks, local_blocks};
  AttnArgs a = attn_args(q, k, v, o, shape, scale, all);
  a.wo = make_work_order(all, ix.kind);
  return hip_status(launch_attention_mixed(a, ix, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ------------------------------------------------------------------ hierarchical chunk pruning
namespace {
// Stage list checks: 1..4 stages, lengths multiples of 64, strictly
// decreasing, each dividing the one before, keep >= 1; each stage's candidate
// count (stage 1: the chunks of n keys; later: keep x sub-chunks per chunk)
// at most DSA_PRUNE_MAX_CANDIDATES.
dsa_status check_stages(const dsa_prune_stages* st, int32_t n) {
  if (!st || st->n_stages < 1 || st->n_stages > DSA_PRUNE_MAX_STAGES) return DSA_ERR_INVALID_ARG;
  for (int32_t s = 0; s < st->n_stages; ++s) {
    const int32_t c = st->chunk[s];
    if (c < 64 || c % 64 != 0 || st->keep[s] < 1) return DSA_ERR_INVALID_ARG;
    if (s > 0 && (c >= st->chunk[s - 1] || st->chunk[s - 1] % c != 0)) return DSA_ERR_INVALID_ARG;
  }
  if (((int64_t)n + st->chunk[0] - 1) / st->chunk[0] > DSA_PRUNE_MAX_CANDIDATES) return DSA_ERR_UNSUPPORTED;
  for (int32_t s = 1; s < st->n_stages; ++s)
    if ((int64_t)st->keep[s - 1] * (st->chunk[s - 1] / st->chunk[s]) > DSA_PRUNE_MAX_CANDIDATES)
      return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

PruneArgs prune_args(const void* qu, int32_t qu_dtype, int32_t qu_full, int32_t units, int32_t unit_rows,
                     const void* k, const dsa_shape* shape, const dsa_prune_stages* st, float scale,
                     const HeadMap& hm, float* fine, int32_t* sel, int32_t* n_sel) {
  PruneArgs a;
  a.qu = qu; a.qu_dtype = qu_dtype; a.qu_full = qu_full;
  a.k = k; a.k_dtype = shape->dtype;
  a.n = shape->seq_len; a.head_dim = shape->head_dim; a.units = units; a.rows = shape->batch * hm.n;
  a.unit_rows = unit_rows;
  a.scale = eff_scale(scale, shape->head_dim);
  a.hm = hm;
  a.wo = make_work_order(hm);
  a.fine = fine;
  a.nbf = nblocks(shape->seq_len);
  a.ntiles = 0;
  a.n_stages = st->n_stages;
  for (int32_t s = 0; s < PR_MAX_STAGES; ++s) {
    a.chunk_blocks[s] = s < st->n_stages ? st->chunk[s] / 64 : 1;
    a.keep[s] = s < st->n_stages ? st->keep[s] : 1;
  }
  a.sel = sel; a.n_sel = n_sel;
  a.max_sel = st->keep[st->n_stages - 1];
  return a;
}

// workspace of the composite pruning calls: block maxima, chunk lists and
// (decode) key lists and split partials, or (prefill) pooled queries
struct HierWork { float* fine; int32_t* sel; int32_t* n_sel; int32_t* keys; int32_t* n_keys; float* part; float* qp; };
size_t hier_layout(const dsa_shape* s, int32_t rows, const dsa_prune_stages* st, bool decode, void* base,
                   HierWork* w) {
  const int32_t n = s->seq_len, nb = nblocks(n), units = decode ? 1 : nb;
  const int32_t ks = st->keep[st->n_stages - 1], c = st->chunk[st->n_stages - 1];
  Carver cv{reinterpret_cast<uintptr_t>(base)};
  HierWork h;
  h.fine = cv.take<float>((size_t)rows * units * nb);
  h.sel = cv.take<int32_t>((size_t)rows * units * ks);
  h.n_sel = cv.take<int32_t>((size_t)rows * units);
  h.keys = h.n_keys = nullptr;
  h.part = h.qp = nullptr;
  if (decode) {
    const int32_t mk = (int32_t)std::min<int64_t>((int64_t)ks * c, (int64_t)INT32_MAX);
    h.keys = cv.take<int32_t>((size_t)rows * ks * c);
    h.n_keys = cv.take<int32_t>((size_t)rows);
    h.part = cv.take<float>(decode_workspace_bytes(rows, mk, s->head_dim) / sizeof(float));
  } else {
    h.qp = cv.take<float>((size_t)rows * nb * s->head_dim);
  }
  if (w) *w = h;
  return cv.used;
}
}  // namespace

extern "C" {

size_t dsa_hier_prune_workspace_bytes(const dsa_shape* shape, int32_t units, int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || units < 0 || n_heads < 0) return 0;
  return al((size_t)shape->batch * n_heads * units * nblocks(shape->seq_len) * sizeof(float));
}

dsa_status dsa_hier_prune(const void* qu, int32_t qu_dtype, int32_t units, int32_t unit_rows, const void* k,
                          const dsa_shape* shape, const dsa_prune_stages* stages, float scale,
                          const int32_t* heads, int32_t n_heads, float* block_max, int32_t* sel, int32_t* n_sel,
                          void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if (units < 0 || unit_rows < 0) return DSA_ERR_INVALID_ARG;
  if (qu_dtype != DSA_BF16 && qu_dtype != DSA_F32) return DSA_ERR_UNSUPPORTED;
  if ((st = check_stages(stages, shape->seq_len)) != DSA_OK) return st;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n) || units == 0) return DSA_OK;
  if (!qu || !k || !sel || !n_sel) return DSA_ERR_INVALID_ARG;
  float* fine = block_max;
  if (!fine) {
    const size_t need = dsa_hier_prune_workspace_bytes(shape, units, hm.n);
    if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
    fine = static_cast<float*>(workspace);
  }
  const PruneArgs a = prune_args(qu, qu_dtype, 0, units, unit_rows, k, shape, stages, scale, hm, fine, sel, n_sel);
  return hip_status(launch_prune(a, static_cast<hipStream_t>(stream)));
}

dsa_status dsa_chunks_to_keys(const int32_t* sel, const int32_t* n_sel, int32_t rows, int32_t max_sel,
                              int32_t chunk, int32_t seq_len, int32_t* keys, int32_t* n_keys, void* stream) {
  if (rows < 0 || max_sel < 0 || chunk < 1 || seq_len < 1) return DSA_ERR_INVALID_ARG;
  if ((int64_t)max_sel * chunk > INT32_MAX) return DSA_ERR_UNSUPPORTED;
  if (rows == 0 || max_sel == 0) return DSA_OK;
  if (!sel || !n_sel || !keys || !n_keys) return DSA_ERR_INVALID_ARG;
  return hip_status(launch_chunks_to_keys(sel, n_sel, rows, max_sel, chunk, seq_len, keys, n_keys,
                                          static_cast<hipStream_t>(stream)));
}

size_t dsa_hier_sparse_decode_workspace_bytes(const dsa_shape* shape, const dsa_prune_stages* stages,
                                              int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || n_heads < 0 || check_stages(stages, shape->seq_len) != DSA_OK) return 0;
  return hier_layout(shape, shape->batch * n_heads, stages, true, nullptr, nullptr);
}

dsa_status dsa_hier_sparse_decode(const void* q, const void* k, const void* v, void* o, const dsa_shape* shape,
                                  const dsa_prune_stages* stages, float scale, const int32_t* heads,
                                  int32_t n_heads, void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if ((st = check_stages(stages, shape->seq_len)) != DSA_OK) return st;
  if ((int64_t)stages->keep[stages->n_stages - 1] * stages->chunk[stages->n_stages - 1] > INT32_MAX)
    return DSA_ERR_UNSUPPORTED;
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  const int32_t rows = shape->batch * hm.n;
  if (rows == 0) return DSA_OK;  // no decode row: nothing read or written
  if (!q || !o || (shape->seq_len > 0 && (!k || !v))) return DSA_ERR_INVALID_ARG;
  const size_t need = hier_layout(shape, rows, stages, true, nullptr, nullptr);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  HierWork w;
  hier_layout(shape, rows, stages, true, workspace, &w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PruneArgs pa = prune_args(q, shape->dtype, 1, 1, 0, k, shape, stages, scale, hm, w.fine, w.sel, w.n_sel);
  const int32_t c = stages->chunk[stages->n_stages - 1];
  hipError_t e = hipSuccess;
  DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.n = shape->seq_len; a.head_dim = shape->head_dim; a.dtype = shape->dtype; a.rows = rows;
  a.scale_log2 = eff_scale(scale, shape->head_dim) * LOG2E;
  a.hm = hm;
  a.wo = make_work_order(hm);
  a.part = w.part;
  if (shape->seq_len == 0) {
    // an empty cache: nothing to prune, the rows come out as zeros (as in dsa_sparse_decode)
    a.keys = nullptr; a.max_keys = 0; a.n_keys = nullptr;
  } else {
    e = launch_prune(pa, s);
    if (e == hipSuccess)
      e = launch_chunks_to_keys(w.sel, w.n_sel, rows, pa.max_sel, c, shape->seq_len, w.keys, w.n_keys, s);
    a.keys = w.keys; a.max_keys = pa.max_sel * c; a.n_keys = w.n_keys;
  }
  if (e == hipSuccess) e = launch_decode(a, s);
  return hip_status(e);
}

size_t dsa_hier_block_sparse_workspace_bytes(const dsa_shape* shape, const dsa_prune_stages* stages,
                                             int32_t n_heads) {
  if (check_shape(shape) != DSA_OK || n_heads < 0 || check_stages(stages, shape->seq_len) != DSA_OK) return 0;
  return hier_layout(shape, shape->batch * n_heads, stages, false, nullptr, nullptr);
}

dsa_status dsa_hier_block_sparse_attention(const void* q, const void* k, const void* v, void* o,
                                           const dsa_shape* shape, const dsa_prune_stages* stages, float scale,
                                           const int32_t* heads, int32_t n_heads, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  dsa_status st = check_shape(shape);
  if (st != DSA_OK) return st;
  if ((st = check_stages(stages, shape->seq_len)) != DSA_OK) return st;
  if (stages->chunk[stages->n_stages - 1] != 64) return DSA_ERR_INVALID_ARG;  // key blocks
  HeadMap hm;
  if ((st = make_map(shape->q_heads, shape->kv_heads, heads, n_heads, hm)) != DSA_OK) return st;
  if (no_work(shape, hm.n)) return DSA_OK;
  if (!q || !k || !v || !o) return DSA_ERR_INVALID_ARG;
  const int32_t rows = shape->batch * hm.n, n = shape->seq_len, nb = nblocks(n);
  const size_t need = hier_layout(shape, rows, stages, false, nullptr, nullptr);
  if (workspace_bytes < need || (need && !workspace)) return DSA_ERR_WORKSPACE;
  HierWork w;
  hier_layout(shape, rows, stages, false, workspace, &w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_pool(q, shape->dtype, n, shape->head_dim, rows, hm, w.qp, s);
  PruneArgs pa = prune_args(w.qp, DSA_F32, 0, nb, BLOCK, k, shape, stages, scale, hm, w.fine, w.sel, w.n_sel);
  if (e == hipSuccess) e = launch_prune(pa, s);
  if (e == hipSuccess)
    e = launch_attention_blocks(attn_args(q, k, v, o, shape, scale, hm), BlockIndex{w.sel, w.n_sel, pa.max_sel}, s);
  return hip_status(e);
}

}  // extern "C"
