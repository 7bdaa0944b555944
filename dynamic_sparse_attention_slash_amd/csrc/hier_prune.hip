// Multi-stage hierarchical chunk pruning, gfx950.
//
// [InfiniteHiP summary, section "modular hierarchical token pruning": the keys
// are cut into fixed-length chunks, the highest-scoring token of each chunk is
// found in parallel, only the best chunks go on to the next stage, and stacked
// stages refine the block-sparse mask of a query block.]
//
// A query vector (a decode row, or a query block's mean-pooled row) sees the
// keys j < limit. A token's score is scale * q . k_j; a chunk's score is the
// largest score among its visible tokens. Stage s keeps the keep[s] best chunks
// of length chunk[s] among the sub-chunks of the chunks stage s-1 kept (stage
// 1: all chunks), ranked as the rest of the library ranks (forced first, then
// higher score, then lower id), with the chunk holding key limit - 1 forced.
//
// Two kernels:
//   blockmax: the largest score of every 64-key block, per query vector. One
//     lane per key holds the key's row as floats; a wave covers one 64-key
//     block and takes its maximum with cross-lane steps. For one query vector
//     per head (decode) it streams K once, memory-bound; for many (a query
//     block each) it is VALU-bound, one FMA per key, dimension and vector.
//   select: one work-group per query vector runs the stages. A chunk's score
//     is the largest of its 64-key blocks' maxima (the same quantity), taken
//     over all (candidate, block) pairs in parallel with an LDS maximum on
//     order-preserving keys. Each candidate gets a distinct 64-bit rank key
//     (forced bit | score key | inverted id); the keep[s] best are those with
//     fewer than keep[s] keys above them (one candidate per thread, up to 256
//     candidates) or at least the keep[s]-th largest key, found bit by bit
//     from block-wide counts; the kept chunks are compacted in ascending id
//     order, and their sub-chunks become the next stage's candidates in
//     ascending order.
// The chunk lists of a decode row expand to key lists for the sparse decode.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int32_t PR_TILE = 256;  // keys per blockmax work-group (4 waves x 64)

__device__ __forceinline__ int32_t unit_limit(const PruneArgs& a, int32_t u) {
  return a.unit_rows > 0 ? min(a.n, (u + 1) * a.unit_rows) : a.n;
}

// unit vector element d as float
template <typename TQ>
__device__ __forceinline__ float qval(const TQ* p, int32_t d) {
  if constexpr (sizeof(TQ) == 2) return bf16_bits_to_f32(p[d]);
  else return p[d];
}

template <typename TK, typename TQ, int D>
__global__ __launch_bounds__(PR_TILE) void prune_blockmax_kernel(PruneArgs a) {
  int32_t row, tile;
  work_item(a.hm, a.wo, a.ntiles, row, tile);
  const int32_t tid = threadIdx.x, lane = tid & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t blk = tile * (PR_TILE / 64) + wave;  // this wave's 64-key block
  if (blk * 64 >= a.n) return;                       // past the cache: no block
  const int32_t j = blk * 64 + lane;
  const TK* ks = static_cast<const TK*>(a.k) + a.hm.kv_slab(row, a.n, D);
  // key j as floats (a lane past the end reads the last key; its score is masked)
  float kf[D];
  {
    const TK* kr = ks + (size_t)min(j, a.n - 1) * D;
    if constexpr (sizeof(TK) == 2) {
      const u32x4* src = reinterpret_cast<const u32x4*>(kr);
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const u32x4 x = src[c];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          kf[8 * c + 2 * t] = __uint_as_float(x[t] << 16);
          kf[8 * c + 2 * t + 1] = __uint_as_float(x[t] & 0xffff0000u);
        }
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(kr);
#pragma unroll
      for (int c = 0; c < D / 4; ++c) {
        const f32x4 x = src[c];
#pragma unroll
        for (int t = 0; t < 4; ++t) kf[4 * c + t] = x[t];
      }
    }
  }
  // units that see no key of this block are skipped (prefill: unit u sees
  // keys below (u + 1) * unit_rows)
  const int32_t u_lo = a.unit_rows > 0 ? (blk * 64) / a.unit_rows : 0;
  const TQ* qbase = static_cast<const TQ*>(a.qu) +
                    (a.qu_full ? a.hm.q_slab(row, a.units, D) : (size_t)row * a.units * D);
  float* out = a.fine + (size_t)row * a.units * a.nbf + blk;
  for (int32_t u = u_lo; u < a.units; ++u) {
    const int32_t limit = unit_limit(a, u);
    const TQ* qv = qbase + (size_t)u * D;
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) dot = __builtin_fmaf(kf[d], qval(qv, d), dot);
    float x = j < limit ? dot * a.scale : -INFINITY;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x = xor_max(x, m);
    if (lane == 0) out[(size_t)u * a.nbf] = x;
  }
}

// Decode rows (one query vector per head that sees the whole cache, bf16 q
// and k): the heads of a kv group
// share one pass over K. A work-group (four waves, 64 keys each) takes one
// (batch, kv group, 256-key tile); for up to 16 heads at a time the scores
// are one MFMA block per 16 keys, S^T = Q K^T (A = 16 query heads x 32 dims,
// B = 32 dims x 16 keys, both read straight from memory: lane l holds 8 dims
// of head / key l % 16), four MFMAs over the head dimension. In the output a
// lane holds four heads' scores of one key; the block maximum is a per-lane
// maximum over the four 16-key tiles and then over the 16 key lanes. bf16
// products are exact in fp32, so this is the fp32 dot product up to the order
// of its additions.
template <int D>
__global__ __launch_bounds__(PR_TILE) void prune_decode_blockmax_kernel(PruneArgs a) {
  constexpr int DS = D / 32;
  const int32_t ng = a.wo.n_groups;
  const int32_t item = blockIdx.x;
  const int32_t tile = item % a.ntiles, bg = item / a.ntiles;
  const int32_t b = bg / ng, g = bg - b * ng;
  const int32_t lane = threadIdx.x & 63, l16 = lane & 15, grp = lane >> 4;
  const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
  const int32_t blk = tile * (PR_TILE / 64) + wave;
  if (blk * 64 >= a.n) return;
  const int32_t g0 = a.wo.gstart[g], gsize = a.wo.gstart[g + 1] - g0;
  const int32_t kvh = a.hm.h[a.wo.order[g0]] / (a.hm.q_heads / a.hm.kv_heads);
  const uint16_t* ks = static_cast<const uint16_t*>(a.k) + ((size_t)b * a.hm.kv_heads + kvh) * (size_t)a.n * D;
  // B operands of the block's four 16-key tiles (keys past the end read the
  // last key; their scores are masked)
  u32x4 kop[4][DS];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int32_t key = min(blk * 64 + 16 * t + l16, a.n - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(ks + (size_t)key * D + 8 * grp);
#pragma unroll
    for (int s = 0; s < DS; ++s) kop[t][s] = src[4 * s];
  }
  const uint16_t* qbase = static_cast<const uint16_t*>(a.qu);
  for (int32_t h0 = 0; h0 < gsize; h0 += 16) {
    // A operand: head h0 + l16 of the group (a lane past the group reads its
    // first head; its rows are not written)
    const int32_t t_head = a.wo.order[g0 + min(h0 + l16, gsize - 1)];
    const size_t qrow = a.qu_full ? (size_t)b * a.hm.q_heads + a.hm.h[t_head] : (size_t)b * a.hm.n + t_head;
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(qbase + qrow * D + 8 * grp);
    u32x4 qop[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[s] = qsrc[4 * s];
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) acc = mfma_bf16(qop[s], kop[t][s], acc);
      const bool ok = blk * 64 + 16 * t + l16 < a.n;
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], ok ? acc[i] * a.scale : -INFINITY);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) mx[i] = xor_max(mx[i], m);
    }
    if (l16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t hh = h0 + 4 * grp + i;
        if (hh < gsize) a.fine[((size_t)b * a.hm.n + a.wo.order[g0 + hh]) * a.nbf + blk] = mx[i];
      }
    }
  }
}

// Pooled query blocks (units of 64 rows, fp32) against bf16 keys: one wave
// per (row, 64-unit tile, 64-key block c), on the MFMA. Unit u sees the whole
// block c when c <= u (keys below n), none of it otherwise. The fp32 unit
// vector is split into bf16 hi + lo (x - hi - lo below 2^-17 |x|) and both
// halves are multiplied with the bf16 keys (exact products, fp32
// accumulation): S = Qu K^T as A = 16 units x 32 dims, B = 32 dims x 16 keys,
// two MFMAs per k-step. A lane then holds four units' scores of one key; the
// block maximum is a per-lane maximum over the block's four 16-key tiles and
// then over the 16 key lanes.
template <int D>
__global__ __launch_bounds__(64) void prune_prefill_blockmax_kernel(PruneArgs a) {
  constexpr int DS = D / 32;
  const int32_t c = blockIdx.x, ut = blockIdx.y, row = blockIdx.z;
  if (c > 64 * ut + 63) return;  // no unit of the tile sees this block
  const int32_t lane = threadIdx.x, l16 = lane & 15, grp = lane >> 4;
  const uint16_t* ks = static_cast<const uint16_t*>(a.k) + a.hm.kv_slab(row, a.n, D);
  u32x4 kop[4][DS];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int32_t key = min(c * 64 + 16 * t + l16, a.n - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(ks + (size_t)key * D + 8 * grp);
#pragma unroll
    for (int s = 0; s < DS; ++s) kop[t][s] = src[4 * s];
  }
  const float* qrow = static_cast<const float*>(a.qu) + (size_t)row * a.units * D;
  float* out = a.fine + (size_t)row * a.units * a.nbf + c;
#pragma unroll 1
  for (int ub = 0; ub < 4; ++ub) {
    const int32_t u0 = 64 * ut + 16 * ub;
    if (u0 >= a.units || u0 + 15 < c) continue;  // units past the end, or all before block c
    // A operands: unit u0 + l16, dims 8 grp + 32 s .. + 7, split into hi / lo
    const float* qv = qrow + (size_t)min(u0 + l16, a.units - 1) * D + 8 * grp;
    u32x4 ah[DS], al[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(qv + 32 * s);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(qv + 32 * s + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h = pack_bf16x2(x[2 * e], x[2 * e + 1]);
        ah[s][e] = h;
        al[s][e] = pack_bf16x2(x[2 * e] - __uint_as_float(h << 16), x[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
      }
    }
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        acc = mfma_bf16(ah[s], kop[t][s], acc);
        acc = mfma_bf16(al[s], kop[t][s], acc);
      }
      const bool ok = c * 64 + 16 * t + l16 < a.n;
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], ok ? acc[i] * a.scale : -INFINITY);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) mx[i] = xor_max(mx[i], m);
    }
    if (l16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t u = u0 + 4 * grp + i;
        if (u < a.units && c <= u) out[(size_t)u * a.nbf] = mx[i];
      }
    }
  }
}

// order-preserving key of an fp32 score: NaN ranks as -inf, -0 as +0
__device__ __forceinline__ uint32_t pr_score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int PR_THREADS = 256;

// block-wide sum (all threads get it); red has PR_THREADS / 64 entries
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < PR_THREADS / 64; ++w) s += red[w];
  return s;
}

// exclusive prefix of v over the threads (in thread order); returns the total
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t& excl, uint32_t* buf) {
  __syncthreads();
  buf[threadIdx.x] = v;
  __syncthreads();
  for (int off = 1; off < PR_THREADS; off <<= 1) {
    const uint32_t t = threadIdx.x >= (uint32_t)off ? buf[threadIdx.x - off] : 0u;
    __syncthreads();
    buf[threadIdx.x] += t;
    __syncthreads();
  }
  excl = buf[threadIdx.x] - v;
  return buf[PR_THREADS - 1];
}

// CAP: candidates one stage may hold (the host picks the smallest instance
// that fits the stage list, so small lists leave room for more work-groups).
template <int CAP>
__global__ __launch_bounds__(PR_THREADS) void prune_select_kernel(PruneArgs a) {
  __shared__ uint64_t key[CAP];
  __shared__ uint32_t sk[CAP];  // a candidate's score key, then its kept flag
  __shared__ int32_t cid[CAP];
  __shared__ int32_t kept[CAP];
  __shared__ uint32_t buf[PR_THREADS];
  __shared__ uint32_t red[PR_THREADS / 64];
  const int32_t u = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int32_t limit = unit_limit(a, u);
  const int32_t nvis = (limit + 63) / 64;  // visible 64-key blocks
  const float* fm = a.fine + ((size_t)row * a.units + u) * a.nbf;
  int32_t m = (nvis + a.chunk_blocks[0] - 1) / a.chunk_blocks[0];
  for (int32_t i = tid; i < m; i += PR_THREADS) cid[i] = i;
  int32_t nk = 0;
  for (int32_t s = 0; s < a.n_stages; ++s) {
    const int32_t cb = a.chunk_blocks[s];
    const int32_t forced = (nvis - 1) / cb;
    __syncthreads();
    for (int32_t i = tid; i < m; i += PR_THREADS) sk[i] = 0u;  // below every score key
    __syncthreads();
    // a candidate's score is its largest block maximum: every (candidate,
    // block) pair in parallel (consecutive pairs read consecutive blocks),
    // combined by an LDS maximum on order-preserving keys
    for (int32_t p = tid; p < m * cb; p += PR_THREADS) {
      const int32_t i = p / cb, b = cid[i] * cb + (p - i * cb);
      if (b < nvis) atomicMax(&sk[i], pr_score_key(fm[b]));
    }
    __syncthreads();
    for (int32_t i = tid; i < m; i += PR_THREADS)
      key[i] = cid[i] == forced ? ~0ull : ((uint64_t)sk[i] << 31) | (uint64_t)(0x7fffffff - cid[i]);
    __syncthreads();
    const int32_t keep = min(a.keep[s], m);
    if (keep >= m) {
      for (int32_t i = tid; i < m; i += PR_THREADS) sk[i] = 1u;
    } else if (m <= PR_THREADS) {
      // one candidate per thread: kept iff fewer than keep keys rank above it
      if (tid < m) {
        const uint64_t kt = key[tid];
        int32_t r = 0;
        for (int32_t j = 0; j < m; ++j) r += key[j] > kt;
        sk[tid] = r < keep ? 1u : 0u;
      }
    } else {
      // the keep-th largest key: largest T with #{key >= T} >= keep
      uint64_t T = 0;
      for (int bit = 63; bit >= 0; --bit) {
        const uint64_t t2 = T | (1ull << bit);
        uint32_t c = 0;
        for (int32_t i = tid; i < m; i += PR_THREADS) c += key[i] >= t2;
        if (block_sum(c, red) >= (uint32_t)keep) T = t2;
      }
      for (int32_t i = tid; i < m; i += PR_THREADS) sk[i] = key[i] >= T ? 1u : 0u;
    }
    __syncthreads();
    // compact the kept candidates in ascending order (each thread a run)
    const int32_t per = (m + PR_THREADS - 1) / PR_THREADS;
    const int32_t i0 = min(m, tid * per), i1 = min(m, i0 + per);
    uint32_t c = 0;
    for (int32_t i = i0; i < i1; ++i) c += sk[i];
    uint32_t pos;
    block_scan(c, pos, buf);
    for (int32_t i = i0; i < i1; ++i)
      if (sk[i]) kept[pos++] = cid[i];
    nk = keep;
    __syncthreads();
    if (s + 1 < a.n_stages) {
      // sub-chunks of the kept chunks, ascending; all but the last kept chunk
      // (the forced one, the highest id) lie wholly below the limit
      const int32_t r = cb / a.chunk_blocks[s + 1], cb2 = a.chunk_blocks[s + 1];
      const int32_t last_vis = (nvis + cb2 - 1) / cb2;  // sub-chunk ids below this hold visible keys
      m = (nk - 1) * r + (last_vis - kept[nk - 1] * r);
      for (int32_t i = tid; i < nk * r; i += PR_THREADS) {
        const int32_t y = kept[i / r] * r + i % r;
        if (i < m) cid[i] = y;
      }
    }
  }
  int32_t* dst = a.sel + ((size_t)row * a.units + u) * a.max_sel;
  for (int32_t i = tid; i < nk; i += PR_THREADS) dst[i] = kept[i];
  if (tid == 0) a.n_sel[(size_t)row * a.units + u] = nk;
}

// keys[row][i * chunk + t] = sel[row][i] * chunk + t, for the n_sel[row]
// chunks; n_keys = the keys below seq_len (only the last chunk can be cut).
__global__ __launch_bounds__(256) void chunks_to_keys_kernel(const int32_t* __restrict__ sel,
                                                             const int32_t* __restrict__ n_sel, int32_t max_sel,
                                                             int32_t chunk, int32_t n, int32_t* __restrict__ keys,
                                                             int32_t* __restrict__ n_keys) {
  const int32_t row = blockIdx.y;
  const int32_t cnt = min(n_sel[row], max_sel);
  const int32_t total = cnt * chunk;
  const int32_t* s = sel + (size_t)row * max_sel;
  int32_t* k = keys + (size_t)row * max_sel * chunk;
  for (int32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256)
    k[i] = min(s[i / chunk] * chunk + i % chunk, n - 1);
  if (blockIdx.x == 0 && threadIdx.x == 0)
    n_keys[row] = cnt == 0 ? 0 : (cnt - 1) * chunk + min(chunk, n - s[cnt - 1] * chunk);
}

}  // namespace

hipError_t launch_prune(PruneArgs a, hipStream_t s) {
  if (a.rows == 0 || a.units == 0 || a.n == 0) return hipSuccess;
  a.nbf = (a.n + 63) / 64;
  a.ntiles = (a.n + PR_TILE - 1) / PR_TILE;
  const bool kb = a.k_dtype == BF16, qb = a.qu_dtype == BF16, d64 = a.head_dim == 64;
  auto bm = kb ? (qb ? (d64 ? prune_blockmax_kernel<uint16_t, uint16_t, 64> : prune_blockmax_kernel<uint16_t, uint16_t, 128>)
                     : (d64 ? prune_blockmax_kernel<uint16_t, float, 64> : prune_blockmax_kernel<uint16_t, float, 128>))
               : (qb ? (d64 ? prune_blockmax_kernel<float, uint16_t, 64> : prune_blockmax_kernel<float, uint16_t, 128>)
                     : (d64 ? prune_blockmax_kernel<float, float, 64> : prune_blockmax_kernel<float, float, 128>));
  if (a.unit_rows == BLOCK && kb && !qb && !a.qu_full) {
    // pooled query blocks against bf16 keys: block maxima on the MFMA
    auto pk = d64 ? prune_prefill_blockmax_kernel<64> : prune_prefill_blockmax_kernel<128>;
    hipLaunchKernelGGL(pk, dim3(a.nbf, (a.units + 63) / 64, a.rows), dim3(64), 0, s, a);
  } else if (a.units == 1 && a.unit_rows == 0 && kb && qb) {
    // decode rows: one pass over K per kv group
    auto dk = d64 ? prune_decode_blockmax_kernel<64> : prune_decode_blockmax_kernel<128>;
    const long long items = (long long)(a.rows / a.hm.n) * a.wo.n_groups * a.ntiles;
    hipLaunchKernelGGL(dk, dim3((unsigned)items), dim3(PR_TILE), 0, s, a);
  } else {
    hipLaunchKernelGGL(bm, dim3((unsigned)((long long)a.ntiles * a.rows)), dim3(PR_TILE), 0, s, a);
  }
  // the largest candidate count of any stage picks the select's LDS size
  int64_t cand = (a.nbf + a.chunk_blocks[0] - 1) / a.chunk_blocks[0];
  for (int32_t st = 1; st < a.n_stages; ++st) {
    const int64_t c2 = (int64_t)a.keep[st - 1] * (a.chunk_blocks[st - 1] / a.chunk_blocks[st]);
    cand = c2 > cand ? c2 : cand;
  }
  hipLaunchKernelGGL(cand <= 1024 ? prune_select_kernel<1024> : prune_select_kernel<PR_MAX_CAND>,
                     dim3(a.units, a.rows), dim3(PR_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_chunks_to_keys(const int32_t* sel, const int32_t* n_sel, int32_t rows, int32_t max_sel,
                                 int32_t chunk, int32_t n, int32_t* keys, int32_t* n_keys, hipStream_t s) {
  if (rows == 0 || max_sel == 0) return hipSuccess;
  const long long blocks = ((long long)max_sel * chunk + 255) / 256;
  const unsigned gx = (unsigned)(blocks < 64 ? blocks : 64);
  hipLaunchKernelGGL(chunks_to_keys_kernel, dim3(gx, rows), dim3(256), 0, s, sel, n_sel, max_sel, chunk, n,
                     keys, n_keys);
  return hipGetLastError();
}

}  // namespace dsa
