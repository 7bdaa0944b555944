// Block-sparse flash-style attention over a per-query-block key set, gfx950.
//
// Computes, for every row i of query block a, softmax over the block's allowed
// keys j <= i of scale * q_i . k_j, times v_j [MInference 1.0 article, §1
// Problem Formulation, with masked entries excluded exactly]. The key set of a
// block is a list of contiguous key ranges followed by a list of gathered key
// columns (the vertical-slash sparse format of §2.2), or a list of 64-key blocks
// (block-sparse heads, §2.2), or the closed-form sink + local window of the
// streaming pattern (usage listing, streaming_forward). Online softmax with a
// deferred rescale is used instead of the two-pass form; both give the same
// result [Novita blog, §2 Modificación de Atención, FlashAttention one-pass
// description].
//
// Work decomposition: one wave64 work-group per (row = batch x listed head,
// query block of 64 rows). The wave keeps the 64 queries in registers and walks
// the key set in tiles of two 16-key sub-blocks:
//   S^T (keys x queries) = K_tile * Q^T      MFMA, K rows loaded straight from
//                                            global memory (gathers and
//                                            unaligned ranges cost nothing extra)
//   P = exp2(S * scale*log2e - m)            fp32, per query column per lane
//   O^T (dims x queries) += V_tile^T * P^T   MFMA; V_tile^T is transposed
//                                            through LDS (bf16) or read row-wise
//                                            (fp32, whose MFMA takes one k per
//                                            lane)
// In the MFMA output layout a lane holds one query column, so the running max,
// the sum and the rescale of O^T need no data from other query columns.
#include "kernels.hpp"

namespace dsa {
namespace {

struct SubBlock {
  int32_t start;        // first key (ranges)
  int32_t count;        // keys in this sub-block, 0..16
  const int32_t* list;  // gathered keys, or nullptr for a range
};

// Key of a slot; gathered entries are clamped into [0, n) so that a bad index
// can never address memory outside k or v.
__device__ __forceinline__ int32_t sb_key(const SubBlock& s, int32_t slot, int32_t n) {
  int32_t sl = slot < s.count ? slot : 0;
  return s.list ? min(max(s.list[sl], 0), n - 1) : s.start + sl;
}
__device__ __forceinline__ int32_t sb_last_key(const SubBlock& s) {
  return s.count == 0 ? -1 : (s.list ? s.list[s.count - 1] : s.start + s.count - 1);
}

// ---- key-range sources (all state is wave-uniform) ----
struct VsRanges {
  const int32_t* iv; int32_t n_iv; int32_t t; int32_t r0; int32_t n;
  __device__ bool next(int32_t& lo, int32_t& hi) {
    while (t < n_iv) {
      int32_t d_lo = iv[2 * t], d_hi = iv[2 * t + 1];
      ++t;
      if (d_lo >= r0 + BLOCK) { t = n_iv; return false; }  // intervals ascending
      lo = max(0, r0 - d_hi);
      hi = min(n, r0 + BLOCK - d_lo);
      if (lo < hi) return true;
    }
    return false;
  }
};
struct BlockRanges {
  const int32_t* sel; int32_t n_sel; int32_t t; int32_t n;
  __device__ bool next(int32_t& lo, int32_t& hi) {
    while (t < n_sel) {
      int32_t c = sel[t++];
      if (c < 0) continue;
      lo = c * BLOCK;
      hi = min(n, lo + BLOCK);
      if (lo < hi) return true;
    }
    return false;
  }
};
struct StreamRanges {
  int32_t a, init_blocks, local_blocks, t, n;
  __device__ bool next(int32_t& lo, int32_t& hi) {
    int32_t sink_end = min(init_blocks, a + 1);
    if (t == 0) {
      t = 1;
      if (sink_end > 0) { lo = 0; hi = min(n, sink_end * BLOCK); return true; }
    }
    if (t == 1) {
      t = 2;
      int32_t c0 = max(a - local_blocks + 1, sink_end);
      if (c0 <= a) { lo = c0 * BLOCK; hi = min(n, (a + 1) * BLOCK); return lo < hi; }
    }
    return false;
  }
};

template <class R>
struct KeyGen {
  R ranges;
  const int32_t* cols; int32_t n_cols;
  int32_t p, hi, cp;
  __device__ SubBlock next() {
    while (true) {
      if (p < hi) {
        int32_t c = min(16, hi - p);
        SubBlock s{p, c, nullptr};
        p += c;
        return s;
      }
      int32_t lo2, hi2;
      if (!ranges.next(lo2, hi2)) break;
      p = lo2;
      hi = hi2;
    }
    if (cp < n_cols) {
      int32_t c = min(16, n_cols - cp);
      SubBlock s{0, c, cols + cp};
      cp += c;
      return s;
    }
    return SubBlock{0, 0, nullptr};
  }
};

// Work-group -> (row, query block). Blocks of one row go to consecutive
// work-groups, latest (largest key set) first.
__device__ __forceinline__ void work_item(int32_t nb, int32_t& row, int32_t& a) {
  int32_t w = blockIdx.x;
  row = w / nb;
  a = nb - 1 - (w - row * nb);
}

// ---------------------------------------------------------------------------
// shared softmax step on a tile of S^T values st[sub-block][query block][i]
// lane holds query column (l & 15) + 16*qb, key slots 4*(l >> 4) + i
// ---------------------------------------------------------------------------
struct SoftmaxState {
  float m[4];     // running max in log2 units (scale*log2e folded in)
  float lsum[4];  // this lane's part of the row sums
};

__device__ __forceinline__ void mask_tile(f32x4 (&st)[2][4], const SubBlock (&sb)[2], int32_t r0,
                                          int32_t n, int32_t lane) {
  const int32_t g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    // only partial sub-blocks and those reaching the diagonal need a mask
    if (sb[s2].count < 16 || sb_last_key(sb[s2]) > r0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int32_t slot = 4 * g + i;
        bool valid = slot < sb[s2].count;
        int32_t key = sb_key(sb[s2], slot, n);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          int32_t row = r0 + 16 * qb + l16;
          if (!valid || key > row) st[s2][qb][i] = -INFINITY;
        }
      }
    }
  }
}

// Online softmax update; returns whether any rescale factor differs from 1.
// The running max is only raised when a new row max exceeds it by more than
// 2^8, so P stays <= 256 and the O rescale runs rarely; the final O / l is
// unchanged by the choice of reference max. SUM: add P to the row sums here
// (the bf16 kernel instead sums P after rounding it to bf16, so that O / l
// divides by the sum of exactly the weights the PV product used).
template <bool SUM>
__device__ __forceinline__ bool softmax_tile(f32x4 (&st)[2][4], SoftmaxState& ss,
                                             float scale_log2, float (&alpha)[4]) {
  float mt[4];
  bool upd[4];
  bool any_upd = false;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    float mx = fmaxf(fmaxf(fmaxf(st[0][qb][0], st[0][qb][1]), fmaxf(st[0][qb][2], st[0][qb][3])),
                     fmaxf(fmaxf(st[1][qb][0], st[1][qb][1]), fmaxf(st[1][qb][2], st[1][qb][3])));
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    mt[qb] = mx * scale_log2;
    upd[qb] = mt[qb] > ss.m[qb] + 8.0f;
    any_upd |= upd[qb];
  }
  bool wave_upd = __any(any_upd);
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    alpha[qb] = 1.0f;
    if (wave_upd && upd[qb]) {
      alpha[qb] = fast_exp2(ss.m[qb] - mt[qb]);
      ss.m[qb] = mt[qb];
      ss.lsum[qb] *= alpha[qb];
    }
  }
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = fast_exp2(fmaf(st[s2][qb][i], scale_log2, -ss.m[qb]));
        st[s2][qb][i] = p;
        if (SUM) ss.lsum[qb] += p;
      }
  return wave_upd;
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
template <int D, class R>
__device__ void attend_bf16(const uint16_t* __restrict__ qs, const uint16_t* __restrict__ ks,
                            const uint16_t* __restrict__ vs, uint16_t* __restrict__ os,
                            int32_t n, int32_t r0, float scale_log2, KeyGen<R> gen) {
  constexpr int DS = D / 32;      // MFMA k-steps of Q.K
  constexpr int DB = D / 16;      // 16-dim output blocks
  constexpr int VTS = 32 + 4;     // bf16 per transposed-V row (72 B, 8-B aligned)
  constexpr int NCH = D / 64;     // 8-dim chunks of V per lane per tile
  __shared__ __align__(16) uint16_t vt[D * VTS];

  const int32_t lane = threadIdx.x, g = lane >> 4, l16 = lane & 15;

  // Q^T operands: query row r0 + 16qb + l16, dims (D/4)g + 8s .. + 7
  u32x4 qop[4][DS];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    int32_t row = min(r0 + 16 * qb + l16, n - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(qs + (size_t)row * D + (D / 4) * g);
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[qb][s] = src[s];
  }

  f32x4 oacc[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  SoftmaxState ss;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) { ss.m[qb] = NEG_BIG; ss.lsum[qb] = 0.f; }

  const int32_t quad = lane & 7;         // V slots 4quad .. 4quad+3 of the tile
  while (true) {
    SubBlock sb[2];
    sb[0] = gen.next();
    if (sb[0].count == 0) break;
    sb[1] = gen.next();

    // K operands: key slot l16 of each sub-block
    u32x4 kop[2][DS];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      int32_t key = sb_key(sb[s2], l16, n);
      const u32x4* src = reinterpret_cast<const u32x4*>(ks + (size_t)key * D + (D / 4) * g);
#pragma unroll
      for (int s = 0; s < DS; ++s) kop[s2][s] = src[s];
    }
    // V rows for the transpose: 4 slots x 8 dims per chunk
    u32x4 vraw[NCH][4];
    {
      const SubBlock& vsb = sb[quad >> 2];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int32_t slot = 4 * (quad & 3) + t;
        bool valid = slot < vsb.count;
        int32_t key = sb_key(vsb, slot, n);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          int32_t chunk = (lane >> 3) + 8 * c;
          u32x4 x = *reinterpret_cast<const u32x4*>(vs + (size_t)key * D + 8 * chunk);
          vraw[c][t] = valid ? x : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }

    f32x4 st[2][4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s) acc = mfma_bf16(kop[s2][s], qop[qb][s], acc);
        st[s2][qb] = acc;
      }

    __syncthreads();  // previous tile's reads of vt are done
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int32_t chunk = (lane >> 3) + 8 * c;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int w = e >> 1;
        uint32_t a0 = vraw[c][0][w], a1 = vraw[c][1][w], a2 = vraw[c][2][w], a3 = vraw[c][3][w];
        uint32_t lo, hi;
        if (e & 1) {
          lo = (a0 >> 16) | (a1 & 0xffff0000u);
          hi = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
          lo = (a0 & 0xffffu) | (a1 << 16);
          hi = (a2 & 0xffffu) | (a3 << 16);
        }
        *reinterpret_cast<u32x2*>(&vt[(8 * chunk + e) * VTS + 4 * quad]) = u32x2{lo, hi};
      }
    }

    mask_tile(st, sb, r0, n, lane);
    float alpha[4];
    if (softmax_tile<false>(st, ss, scale_log2, alpha)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) oacc[db][qb] *= alpha[qb];
    }
    // P^T operands: slots 4g..4g+3 of sub-block 0, then of sub-block 1; the
    // row sums add the rounded values
    u32x4 pop[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      pop[qb] = u32x4{pack_bf16x2(st[0][qb][0], st[0][qb][1]), pack_bf16x2(st[0][qb][2], st[0][qb][3]),
                      pack_bf16x2(st[1][qb][0], st[1][qb][1]), pack_bf16x2(st[1][qb][2], st[1][qb][3])};
      ss.lsum[qb] += (packed_pair_sum(pop[qb][0]) + packed_pair_sum(pop[qb][1])) +
                     (packed_pair_sum(pop[qb][2]) + packed_pair_sum(pop[qb][3]));
    }

    __syncthreads();  // vt written
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* rowp = &vt[(16 * db + l16) * VTS];
      u32x2 x0 = *reinterpret_cast<const u32x2*>(rowp + 4 * g);
      u32x2 x1 = *reinterpret_cast<const u32x2*>(rowp + 16 + 4 * g);
      u32x4 aop = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) oacc[db][qb] = mfma_bf16(aop, pop[qb], oacc[db][qb]);
    }
  }

  // O = O^T / l: lane writes dims 16db + 4g .. +3 of query r0 + 16qb + l16
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    float lt = xor_sum(xor_sum(ss.lsum[qb], 16), 32);
    float inv = lt > 0.f ? 1.0f / lt : 0.f;
    int32_t row = r0 + 16 * qb + l16;
    if (row < n) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 x = oacc[db][qb] * inv;
        *reinterpret_cast<u32x2*>(os + (size_t)row * D + 16 * db + 4 * g) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (MFMA 16x16x4 f32: one k value per lane, so V needs no transpose)
// ---------------------------------------------------------------------------
template <int D, class R>
__device__ void attend_f32(const float* __restrict__ qs, const float* __restrict__ ks,
                           const float* __restrict__ vs, float* __restrict__ os, int32_t n,
                           int32_t r0, float scale_log2, KeyGen<R> gen) {
  constexpr int DK = D / 4;   // k-steps of Q.K; lane group g holds dims DK*g .. DK*g + DK-1
  constexpr int DB = D / 16;
  const int32_t lane = threadIdx.x, g = lane >> 4, l16 = lane & 15;

  float qop[4][DK];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    int32_t row = min(r0 + 16 * qb + l16, n - 1);
    const f32x4* src = reinterpret_cast<const f32x4*>(qs + (size_t)row * D + DK * g);
#pragma unroll
    for (int s = 0; s < DK / 4; ++s) {
      f32x4 x = src[s];
      qop[qb][4 * s] = x[0]; qop[qb][4 * s + 1] = x[1]; qop[qb][4 * s + 2] = x[2]; qop[qb][4 * s + 3] = x[3];
    }
  }
  f32x4 oacc[DB][4];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  SoftmaxState ss;
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) { ss.m[qb] = NEG_BIG; ss.lsum[qb] = 0.f; }

  while (true) {
    SubBlock sb[2];
    sb[0] = gen.next();
    if (sb[0].count == 0) break;
    sb[1] = gen.next();

    f32x4 st[2][4];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      int32_t key = sb_key(sb[s2], l16, n);
      const f32x4* src = reinterpret_cast<const f32x4*>(ks + (size_t)key * D + DK * g);
      float kop[DK];
#pragma unroll
      for (int s = 0; s < DK / 4; ++s) {
        f32x4 x = src[s];
        kop[4 * s] = x[0]; kop[4 * s + 1] = x[1]; kop[4 * s + 2] = x[2]; kop[4 * s + 3] = x[3];
      }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DK; ++s) acc = mfma_f32(kop[s], qop[qb][s], acc);
        st[s2][qb] = acc;
      }
    }

    mask_tile(st, sb, r0, n, lane);
    float alpha[4];
    if (softmax_tile<true>(st, ss, scale_log2, alpha)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) oacc[db][qb] *= alpha[qb];
    }
    // O^T += V^T P^T, one MFMA per (sub-block, i): lane group g carries key
    // slot 4g + i, whose V row the lane reads at dim 16db + l16.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int32_t slot = 4 * g + i;
        bool valid = slot < sb[s2].count;
        int32_t key = sb_key(sb[s2], slot, n);
        const float* vrow = vs + (size_t)key * D + l16;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float a = valid ? vrow[16 * db] : 0.f;
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) oacc[db][qb] = mfma_f32(a, st[s2][qb][i], oacc[db][qb]);
        }
      }
  }

#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    float lt = xor_sum(xor_sum(ss.lsum[qb], 16), 32);
    float inv = lt > 0.f ? 1.0f / lt : 0.f;
    int32_t row = r0 + 16 * qb + l16;
    if (row < n) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(os + (size_t)row * D + 16 * db + 4 * g) = oacc[db][qb] * inv;
    }
  }
}

// ---------------------------------------------------------------------------
// kernels per index mode
// ---------------------------------------------------------------------------
template <typename T, int D, class R>
__device__ __forceinline__ void attend(const AttnArgs& a, int32_t row, int32_t r0, KeyGen<R> gen) {
  const size_t qoff = a.hm.q_slab(row, a.seq_len, D);
  const size_t kvoff = a.hm.kv_slab(row, a.seq_len, D);
  if constexpr (sizeof(T) == 2) {
    attend_bf16<D, R>(static_cast<const uint16_t*>(a.q) + qoff,
                      static_cast<const uint16_t*>(a.k) + kvoff,
                      static_cast<const uint16_t*>(a.v) + kvoff,
                      static_cast<uint16_t*>(a.o) + qoff, a.seq_len, r0, a.scale_log2, gen);
  } else {
    attend_f32<D, R>(static_cast<const float*>(a.q) + qoff, static_cast<const float*>(a.k) + kvoff,
                     static_cast<const float*>(a.v) + kvoff, static_cast<float*>(a.o) + qoff,
                     a.seq_len, r0, a.scale_log2, gen);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_vs_kernel(AttnArgs a, VsIndex ix) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  int32_t row, blk;
  work_item(nb, row, blk);
  const int32_t r0 = blk * BLOCK;
  KeyGen<VsRanges> gen;
  gen.ranges = VsRanges{ix.iv + (size_t)row * ix.max_iv * 2, min(ix.n_iv[row], ix.max_iv), 0, r0,
                        a.seq_len};
  const size_t cb = (size_t)row * nb + blk;
  gen.cols = ix.cols + cb * ix.max_cols;
  gen.n_cols = min(ix.n_cols[cb], ix.max_cols);
  gen.p = gen.hi = gen.cp = 0;
  attend<T, D>(a, row, r0, gen);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_blocks_kernel(AttnArgs a, BlockIndex ix) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  int32_t row, blk;
  work_item(nb, row, blk);
  const size_t cb = (size_t)row * nb + blk;
  KeyGen<BlockRanges> gen;
  gen.ranges = BlockRanges{ix.sel + cb * ix.max_sel, min(ix.n_sel[cb], ix.max_sel), 0, a.seq_len};
  gen.cols = nullptr;
  gen.n_cols = 0;
  gen.p = gen.hi = gen.cp = 0;
  attend<T, D>(a, row, blk * BLOCK, gen);
}

template <typename T, int D>
__global__ __launch_bounds__(64) void attn_stream_kernel(AttnArgs a, StreamIndex ix) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  int32_t row, blk;
  work_item(nb, row, blk);
  KeyGen<StreamRanges> gen;
  gen.ranges = StreamRanges{blk, ix.init_blocks, ix.local_blocks, 0, a.seq_len};
  gen.cols = nullptr;
  gen.n_cols = 0;
  gen.p = gen.hi = gen.cp = 0;
  attend<T, D>(a, row, blk * BLOCK, gen);
}

}  // namespace

hipError_t launch_attention_vs(const AttnArgs& a, const VsIndex& ix, hipStream_t s) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.rows * nb;
  if (grid == 0) return hipSuccess;
  auto fn = a.dtype == BF16 ? (a.head_dim == 64 ? attn_vs_kernel<uint16_t, 64> : attn_vs_kernel<uint16_t, 128>)
                            : (a.head_dim == 64 ? attn_vs_kernel<float, 64> : attn_vs_kernel<float, 128>);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64), 0, s, a, ix);
  return hipGetLastError();
}

hipError_t launch_attention_blocks(const AttnArgs& a, const BlockIndex& ix, hipStream_t s) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.rows * nb;
  if (grid == 0) return hipSuccess;
  auto fn = a.dtype == BF16 ? (a.head_dim == 64 ? attn_blocks_kernel<uint16_t, 64> : attn_blocks_kernel<uint16_t, 128>)
                            : (a.head_dim == 64 ? attn_blocks_kernel<float, 64> : attn_blocks_kernel<float, 128>);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64), 0, s, a, ix);
  return hipGetLastError();
}

hipError_t launch_attention_stream(const AttnArgs& a, const StreamIndex& ix, hipStream_t s) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.rows * nb;
  if (grid == 0) return hipSuccess;
  auto fn = a.dtype == BF16 ? (a.head_dim == 64 ? attn_stream_kernel<uint16_t, 64> : attn_stream_kernel<uint16_t, 128>)
                            : (a.head_dim == 64 ? attn_stream_kernel<float, 64> : attn_stream_kernel<float, 128>);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64), 0, s, a, ix);
  return hipGetLastError();
}

}  // namespace dsa
