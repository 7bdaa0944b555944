// Block-sparse flash-style attention over a per-query-block key set, gfx950.
//
// Computes, for every row i of query block a, softmax over the block's allowed
// keys j <= i of scale * q_i . k_j, times v_j [MInference 1.0 article, §1
// Problem Formulation, with masked entries excluded exactly]. The key set of a
// block is a list of contiguous key ranges followed by a list of gathered key
// columns (the vertical-slash sparse format of §2.2), or a list of 64-key blocks
// (block-sparse heads, §2.2), or the closed-form sink + local window of the
// streaming pattern (usage listing, streaming_forward). Online softmax with a
// deferred rescale replaces the two-pass form; both give the same result
// [Novita blog, §2 Modificación de Atención, FlashAttention one-pass
// description].
//
// Work decomposition: one work-group per (row = batch x listed head, query
// block of 64 rows); the bf16 kernel splits the block's queries over two waves,
// the fp32 kernel keeps all 64 in one wave. A prologue cuts the block's key set into 16-key sub-blocks and writes their
// descriptors (first key or list position, count, flags) to LDS, so the hot
// loop is straight-line code over tiles of two sub-blocks:
//   S^T (keys x queries) = K_tile * Q^T      MFMA; K rows come straight from
//                                            global memory (gathers and
//                                            unaligned ranges cost nothing extra)
//   P = exp2(S * scale*log2e - m)            fp32, one query column per lane
//   O^T (dims x queries) += V_tile^T * P^T   MFMA; V_tile^T is transposed
//                                            through LDS (bf16) or read row-wise
//                                            (fp32, whose MFMA takes one k per
//                                            lane)
// In the MFMA output layout a lane holds one query column, so the running max
// and the rescale of O^T need no data from other query columns. In the bf16
// kernel the softmax denominator is one more MFMA block whose A operand is all
// ones: it sums exactly the bf16-rounded P the PV product used.
#include "kernels.hpp"

namespace dsa {
namespace {

// ---- 16-key sub-block descriptors ----
constexpr int32_t SB_CAP = 1024;        // descriptors per refill (8 KiB of LDS)
constexpr int32_t F_LIST = 1 << 8;      // keys come from the column list
constexpr int32_t F_MASK = 1 << 9;      // partial, or reaches the diagonal: mask
struct Desc {
  int32_t a;  // first key (range) or position in the column list
  int32_t b;  // count (0..16) | flags
  __device__ int32_t count() const { return b & 0xff; }
};

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

// Fills up to SB_CAP descriptors per call, resuming where the last call
// stopped: first the ranges, then the column list.
template <class R>
struct DescGen {
  R ranges;
  const int32_t* cols; int32_t n_cols;
  int32_t p, hi, cp, r0, n;
  __device__ int32_t fill(Desc* d, int32_t tid, int32_t nthreads) {
    int32_t cnt = 0;
    while (cnt < SB_CAP) {
      if (p >= hi) {
        int32_t lo2, hi2;
        if (!ranges.next(lo2, hi2)) break;
        p = lo2;
        hi = hi2;
        continue;
      }
      const int32_t take = min((hi - p + 15) >> 4, SB_CAP - cnt);
      for (int32_t t = tid; t < take; t += nthreads) {
        int32_t s = p + 16 * t, c = min(16, hi - s);
        d[cnt + t] = Desc{s, c | ((c < 16 || s + c - 1 > r0) ? F_MASK : 0)};
      }
      cnt += take;
      p = min(hi, p + 16 * take);
    }
    if (cnt < SB_CAP && cp < n_cols) {
      const int32_t take = min((n_cols - cp + 15) >> 4, SB_CAP - cnt);
      for (int32_t t = tid; t < take; t += nthreads) {
        int32_t s = cp + 16 * t, c = min(16, n_cols - s);
        bool m = c < 16 || cols[s + c - 1] > r0;
        d[cnt + t] = Desc{s, c | F_LIST | (m ? F_MASK : 0)};
      }
      cnt += take;
      cp = min(n_cols, cp + 16 * take);
    }
    return cnt;
  }
};

// Descriptor t as wave-uniform values; past the end an empty sub-block, which
// must carry the mask flag so that its slots are masked out.
__device__ __forceinline__ Desc uniform_desc(const Desc* d, int32_t t, int32_t cnt) {
  Desc x = t < cnt ? d[t] : Desc{0, F_MASK};
  return Desc{__builtin_amdgcn_readfirstlane(x.a), __builtin_amdgcn_readfirstlane(x.b)};
}

// Key of a slot; gathered entries are clamped into [0, n) so that a bad index
// can never address memory outside k or v. Empty slots read the first key.
__device__ __forceinline__ int32_t desc_key(const Desc& d, const int32_t* cols, int32_t slot,
                                            int32_t n) {
  int32_t sl = slot < d.count() ? slot : 0;
  return (d.b & F_LIST) ? min(max(cols[d.a + sl], 0), n - 1) : d.a + sl;
}

// Work-group -> (row, query block). The hardware deals consecutive work-group
// ids round-robin over the 8 XCDs, each with its own L2. Work items, ordered
// by WorkOrder, are cut into chunks of XCD_CHUNK and the chunks are dealt
// round-robin to the XCDs: the work-groups an XCD runs at one time then share
// K/V rows in its L2, and every XCD still gets a mix of all kv groups and block
// positions (whose costs differ). A tail shorter than NUM_XCD chunks keeps the
// identity mapping.
constexpr int32_t NUM_XCD = 8;
constexpr int32_t XCD_CHUNK = 32;
__device__ __forceinline__ void work_item(const AttnArgs& ar, int32_t nb, int32_t& row, int32_t& a) {
  const int32_t N = gridDim.x, i = blockIdx.x;
  const int32_t T = (N / (NUM_XCD * XCD_CHUNK)) * (NUM_XCD * XCD_CHUNK);
  int32_t w = i;
  if (i < T) {
    const int32_t xcd = i % NUM_XCD, k = i / NUM_XCD;
    w = ((k / XCD_CHUNK) * NUM_XCD + xcd) * XCD_CHUNK + k % XCD_CHUNK;
  }
  const int32_t n = ar.hm.n, per_b = nb * n;
  const int32_t b = w / per_b, w2 = w - b * per_b;
  int32_t gi = 0;
  while (gi + 1 < ar.wo.n_groups && ar.wo.gstart[gi + 1] * nb <= w2) ++gi;
  const int32_t g0 = ar.wo.gstart[gi], size = ar.wo.gstart[gi + 1] - g0;
  const int32_t off = w2 - g0 * nb;
  const int32_t a_idx = off / size, j = off - a_idx * size;
  row = b * n + ar.wo.order[g0 + j];
  a = nb - 1 - a_idx;
}

// ---------------------------------------------------------------------------
// softmax pieces on a tile of S^T values st[sub-block][query block][i]:
// lane holds query column (l & 15) + 16*qb and key slots 4*(l >> 4) + i
// ---------------------------------------------------------------------------
template <int QB>
__device__ __forceinline__ void mask_tile(f32x4 (&st)[2][QB], const Desc (&d)[2], const int32_t* cols,
                                          int32_t q0, int32_t n, int32_t lane) {
  const int32_t g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    if (d[s2].b & F_MASK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int32_t slot = 4 * g + i;
        bool valid = slot < d[s2].count();
        int32_t key = desc_key(d[s2], cols, slot, n);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          int32_t row = q0 + 16 * qb + l16;
          if (!valid || key > row) st[s2][qb][i] = -INFINITY;
        }
      }
    }
  }
}

template <int QB>
__device__ __forceinline__ void mask_tile_lds(f32x4 (&st)[2][QB], const Desc (&d)[2], const int32_t* lcols,
                                              int32_t q0, int32_t lane);

// New reference maxima: raised only when a row max exceeds the current one by
// more than 2^8 (P then stays <= 256 and the O rescale runs rarely; O / l does
// not depend on the reference). Returns whether any lane raised one; alpha
// holds the factors to apply to O and l.
template <int QB>
__device__ __forceinline__ bool update_max(const f32x4 (&st)[2][QB], float (&m)[QB], float scale_log2,
                                           float (&alpha)[QB]) {
  float mt[QB];
  bool any_upd = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float mx = fmaxf(fmaxf(fmaxf(st[0][qb][0], st[0][qb][1]), fmaxf(st[0][qb][2], st[0][qb][3])),
                     fmaxf(fmaxf(st[1][qb][0], st[1][qb][1]), fmaxf(st[1][qb][2], st[1][qb][3])));
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    mt[qb] = mx * scale_log2;
    any_upd |= mt[qb] > m[qb] + 8.0f;
  }
  if (!__any(any_upd)) return false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const bool up = mt[qb] > m[qb] + 8.0f;
    alpha[qb] = up ? fast_exp2(m[qb] - mt[qb]) : 1.0f;
    m[qb] = up ? mt[qb] : m[qb];
  }
  return true;
}

template <int QB>
__device__ __forceinline__ void exp_tile(f32x4 (&st)[2][QB], const float (&m)[QB], float scale_log2) {
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) st[s2][qb][i] = fast_exp2(fmaf(st[s2][qb][i], scale_log2, -m[qb]));
}

// ---------------------------------------------------------------------------
// bf16 kernel: two waves per query block, wave w owns queries r0 + 32w .. +31.
//
// K and V tiles (32 keys) travel global -> LDS with global_load_lds_dwordx4
// (no registers involved), into a two-stage ring: the loads of tile t+1 are
// in flight while tile t is computed, and one barrier per tile separates them.
// Each wave loads one of the two 16-key sub-blocks of a tile. Both matrices
// are row-major in LDS with the 16-byte chunks of row r XOR-swizzled by r, so
// that the operand reads below are free of bank conflicts:
//   K operand (MFMA A, 8 dims of one key per lane): ds_read_b128
//   V^T operand (MFMA A, 8 keys of one dim per lane): two ds_read_b64_tr_b16,
//     the gfx950 transposing LDS read (each 16-lane group reads a 16 x 4 block
//     of b16 and lane i receives element (4j + i/4, i%4) for j = 0..3).
// The block's column-list entries are staged in LDS together with the
// sub-block descriptors, so gathered keys cost no global round trip.
// ---------------------------------------------------------------------------
constexpr int BF16_WAVES = 2;
constexpr int32_t BF16_SB_CAP = 512;   // descriptors per refill
constexpr int32_t COLS_CAP = 1024;     // column-list entries staged per refill

template <int D>
struct TileLds {
  static constexpr int ROW = D * 2;           // bytes per key row
  static constexpr int UNITS = ROW / 16;      // 16-byte chunks per row
  static constexpr int MAT = 32 * ROW;        // one 32-key matrix
  static constexpr int STAGE = 2 * MAT;       // K then V
  static constexpr int RPI = 64 / UNITS;      // rows per global_load_lds_dwordx4
  static constexpr int INSTR = 16 / RPI;      // instructions per 16-row sub-block
  // byte offset of logical chunk c of row r
  __device__ static int off(int r, int c) { return r * ROW + 16 * (c ^ (r & (UNITS - 1))); }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Key of a slot for the bf16 kernel: gathered entries come from the staged
// copy of the column list in LDS.
__device__ __forceinline__ int32_t desc_key_lds(const Desc& d, const int32_t* lcols, int32_t slot) {
  int32_t sl = slot < d.count() ? slot : 0;
  return (d.b & F_LIST) ? lcols[d.a + sl] : d.a + sl;
}

// Fills descriptors like DescGen::fill, but list sub-blocks refer to a copy of
// the column list staged in LDS (positions relative to that copy), and at most
// COLS_CAP entries are staged per call. Entries are clamped into [0, n).
template <class R>
__device__ int32_t fill_bf16(DescGen<R>& gen, Desc* d, int32_t* lcols, int32_t tid, int32_t nthreads) {
  int32_t cnt = 0;
  while (cnt < BF16_SB_CAP) {
    if (gen.p >= gen.hi) {
      int32_t lo2, hi2;
      if (!gen.ranges.next(lo2, hi2)) break;
      gen.p = lo2;
      gen.hi = hi2;
      continue;
    }
    const int32_t take = min((gen.hi - gen.p + 15) >> 4, BF16_SB_CAP - cnt);
    for (int32_t t = tid; t < take; t += nthreads) {
      int32_t s = gen.p + 16 * t, c = min(16, gen.hi - s);
      d[cnt + t] = Desc{s, c | ((c < 16 || s + c - 1 > gen.r0) ? F_MASK : 0)};
    }
    cnt += take;
    gen.p = min(gen.hi, gen.p + 16 * take);
  }
  if (cnt < BF16_SB_CAP && gen.cp < gen.n_cols) {
    const int32_t ncol = min(gen.n_cols - gen.cp, min(COLS_CAP, 16 * (BF16_SB_CAP - cnt)));
    for (int32_t t = tid; t < ncol; t += nthreads) lcols[t] = min(max(gen.cols[gen.cp + t], 0), gen.n - 1);
    const int32_t take = (ncol + 15) >> 4;
    for (int32_t t = tid; t < take; t += nthreads) {
      int32_t s = 16 * t, c = min(16, ncol - s);
      bool m = c < 16 || gen.cols[gen.cp + s + c - 1] > gen.r0;
      d[cnt + t] = Desc{s, c | F_LIST | (m ? F_MASK : 0)};
    }
    cnt += take;
    gen.cp += ncol;
  }
  return cnt;
}

template <int QB>
__device__ __forceinline__ void mask_tile_lds(f32x4 (&st)[2][QB], const Desc (&d)[2], const int32_t* lcols,
                                              int32_t q0, int32_t lane) {
  const int32_t g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    if (d[s2].b & F_MASK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t slot = 4 * g + i;
        const bool valid = slot < d[s2].count();
        const int32_t key = desc_key_lds(d[s2], lcols, slot);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int32_t row = q0 + 16 * qb + l16;
          if (!valid || key > row) st[s2][qb][i] = -INFINITY;
        }
      }
    }
  }
}

// Row max over the four lane groups (lanes l, l^16, l^32, l^48 hold the same
// query column): gfx950 permlane swaps exchange 16-lane rows without LDS.
__device__ __forceinline__ float group_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const uint32_t v = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __attribute__((address_space(3))) void lds_void;

template <int D, class R>
__device__ void attend_bf16(const uint16_t* __restrict__ qs, const uint16_t* __restrict__ ks,
                            const uint16_t* __restrict__ vs, uint16_t* __restrict__ os,
                            int32_t n, int32_t r0, float scale_log2, DescGen<R> gen) {
  using L = TileLds<D>;
  constexpr int DS = D / 32;      // MFMA k-steps of Q.K
  constexpr int DB = D / 16;      // 16-dim output blocks
  // two ring stages in distinct arrays: the compiler can then prove that the
  // loads in flight into one stage do not alias the reads of the other
  __shared__ __align__(16) char ring0[L::STAGE];
  __shared__ __align__(16) char ring1[L::STAGE];
  __shared__ Desc desc[BF16_SB_CAP];
  __shared__ int32_t lcols[COLS_CAP];

  const int32_t tid = threadIdx.x, lane = tid & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int32_t g = lane >> 4, l16 = lane & 15;
  const int32_t q0 = r0 + 32 * wave;

  // Q^T operands: query row q0 + 16qb + l16, dims (D/4)g + 8s .. + 7
  u32x4 qop[2][DS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    int32_t row = min(q0 + 16 * qb + l16, n - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(qs + (size_t)row * D + (D / 4) * g);
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[qb][s] = src[s];
  }

  // per-lane LDS offsets within a stage
  // K operand of step s: row l16 (+16 per sub-block), chunk (D/32)g + s
  int32_t koff[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) koff[s] = L::off(l16, (D / 32) * g + s);
  // V^T operand of dim block db: row 4g + (l16 >> 2) (+16 for the second
  // sub-block), dims 16db + 4(l16 & 3) .. +3
  int32_t voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int32_t r = 4 * g + (l16 >> 2), dim = 16 * db + 4 * (l16 & 3);
    voff[db] = L::MAT + L::off(r, dim >> 3) + 2 * (dim & 7);
  }
  // global -> LDS load k of this wave's sub-block: lane takes row rr(k) of the
  // sub-block at logical chunk c(k), landing at LDS byte 16*lane of the load
  int32_t ld_row[L::INSTR], ld_off[L::INSTR];
#pragma unroll
  for (int k = 0; k < L::INSTR; ++k) {
    ld_row[k] = k * L::RPI + lane / L::UNITS;
    const int32_t c = (lane % L::UNITS) ^ ((16 * wave + ld_row[k]) & (L::UNITS - 1));
    ld_off[k] = ld_row[k] * L::ROW + 16 * c;    // + first key * ROW for a range
  }
  const uint32_t slab_bytes = (uint32_t)n * L::ROW;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)ks, (short)0, slab_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vs, (short)0, slab_bytes, 0x00020000);

  // O^T blocks 0..DB-1, and block DB = row sums of P (A operand all ones)
  f32x4 oacc[DB + 1][2];
#pragma unroll
  for (int db = 0; db <= DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {NEG_BIG, NEG_BIG};
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

  // loads of this wave's sub-block dw into a stage. Range sub-blocks use the
  // first key as the scalar offset; slots past the count read the rows that
  // follow (or zeros past the end of the slab) and are masked out later.
  auto issue_loads = [&](const Desc& dw, char* stage) {
    char* dst = stage + 16 * wave * L::ROW;
    if (dw.b & F_LIST) {
#pragma unroll
      for (int k = 0; k < L::INSTR; ++k) {
        const int32_t key = lcols[dw.a + min(ld_row[k], max(dw.count() - 1, 0))];
        const int32_t vo = ld_off[k] + (key - ld_row[k]) * L::ROW;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(dst + k * 1024), 16, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + L::MAT + k * 1024), 16, vo, 0, 0, 0);
      }
    } else {
      const int32_t so = dw.a * L::ROW;
#pragma unroll
      for (int k = 0; k < L::INSTR; ++k) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(dst + k * 1024), 16, ld_off[k], so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + L::MAT + k * 1024), 16, ld_off[k], so, 0, 0);
      }
    }
  };

  // one tile: wait for its loads, start the next tile's, compute
  auto tile = [&](int32_t tt, int32_t ntiles, int32_t cnt, const char* cur, char* nxt) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile tt have landed
    __syncthreads();                 // ... and the other wave's; tile tt-1 is consumed
    if (tt + 1 < ntiles) issue_loads(uniform_desc(desc, 2 * (tt + 1) + wave, cnt), nxt);
    const Desc d[2] = {uniform_desc(desc, 2 * tt, cnt), uniform_desc(desc, 2 * tt + 1, cnt)};

    // S^T = K Q^T
    f32x4 st[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 kop[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s)
        kop[s] = *reinterpret_cast<const u32x4*>(cur + koff[s] + s2 * 16 * L::ROW);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DS; ++s) acc = mfma_bf16(kop[s], qop[qb][s], acc);
        st[s2][qb] = acc;
      }
    }

    if ((d[0].b | d[1].b) & F_MASK) mask_tile_lds<2>(st, d, lcols, q0, lane);
    // running max (raised only past a 2^8 margin), rescale when raised
    float mt[2];
    bool up_any = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = fmaxf(__builtin_fmaxf(fmaxf(st[0][qb][0], st[0][qb][1]), fmaxf(st[0][qb][2], st[0][qb][3])),
                       fmaxf(fmaxf(st[1][qb][0], st[1][qb][1]), fmaxf(st[1][qb][2], st[1][qb][3])));
      mt[qb] = group_max4(mx) * scale_log2;
      up_any |= mt[qb] > m[qb] + 8.0f;
    }
    if (__any(up_any)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bool up = mt[qb] > m[qb] + 8.0f;
        const float alpha = up ? fast_exp2(m[qb] - mt[qb]) : 1.0f;
        m[qb] = up ? mt[qb] : m[qb];
#pragma unroll
        for (int db = 0; db <= DB; ++db) oacc[db][qb] *= alpha;
      }
    }
    exp_tile<2>(st, m, scale_log2);
    // P^T operands: slots 4g..4g+3 of sub-block 0, then of sub-block 1
    u32x4 pop[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      pop[qb] = u32x4{pack_bf16x2(st[0][qb][0], st[0][qb][1]), pack_bf16x2(st[0][qb][2], st[0][qb][3]),
                      pack_bf16x2(st[1][qb][0], st[1][qb][1]), pack_bf16x2(st[1][qb][2], st[1][qb][3])};

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 x0 = lds_read_tr16(cur + voff[db]);
      const u32x2 x1 = lds_read_tr16(cur + voff[db] + 16 * L::ROW);
      const u32x4 aop = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = mfma_bf16(aop, pop[qb], oacc[db][qb]);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[DB][qb] = mfma_bf16(ones, pop[qb], oacc[DB][qb]);
  };

  while (true) {
    __syncthreads();               // previous refill fully consumed
    const int32_t cnt = fill_bf16(gen, desc, lcols, tid, BF16_WAVES * 64);
    if (cnt == 0) break;
    __syncthreads();
    const int32_t ntiles = (cnt + 1) >> 1;
    issue_loads(uniform_desc(desc, wave, cnt), ring0);
    for (int32_t tt = 0; tt < ntiles; tt += 2) {
      tile(tt, ntiles, cnt, ring0, ring1);
      if (tt + 1 < ntiles) tile(tt + 1, ntiles, cnt, ring1, ring0);
    }
  }

  // O = O^T / l: lane writes dims 16db + 4g .. +3 of query q0 + 16qb + l16
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = oacc[DB][qb][0];
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int32_t row = q0 + 16 * qb + l16;
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
                           int32_t r0, float scale_log2, DescGen<R> gen) {
  constexpr int DK = D / 4;   // k-steps of Q.K; lane group g holds dims DK*g .. DK*g + DK-1
  constexpr int DB = D / 16;
  __shared__ Desc desc[SB_CAP];
  const int32_t lane = threadIdx.x, g = lane >> 4, l16 = lane & 15;
  const int32_t* cols = gen.cols;

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
  float m[4] = {NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};

  while (true) {
    __syncthreads();
    const int32_t cnt = gen.fill(desc, lane, 64);
    if (cnt == 0) break;
    __syncthreads();
    for (int32_t t = 0; t < cnt; t += 2) {
      const Desc d[2] = {uniform_desc(desc, t, cnt), uniform_desc(desc, t + 1, cnt)};
      f32x4 st[2][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        int32_t key = desc_key(d[s2], cols, l16, n);
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
      if ((d[0].b | d[1].b) & F_MASK) mask_tile<4>(st, d, cols, r0, n, lane);
      float alpha[4];
      if (update_max<4>(st, m, scale_log2, alpha)) {
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          lsum[qb] *= alpha[qb];
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha[qb];
        }
      }
      exp_tile<4>(st, m, scale_log2);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) lsum[qb] += (st[s2][qb][0] + st[s2][qb][1]) + (st[s2][qb][2] + st[s2][qb][3]);
      // O^T += V^T P^T, one MFMA per (sub-block, i): lane group g carries key
      // slot 4g + i, whose V row the lane reads at dim 16db + l16.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int32_t slot = 4 * g + i;
          bool valid = slot < d[s2].count();
          int32_t key = desc_key(d[s2], cols, slot, n);
          const float* vrow = vs + (size_t)key * D + l16;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            float a = valid ? vrow[16 * db] : 0.f;
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) oacc[db][qb] = mfma_f32(a, st[s2][qb][i], oacc[db][qb]);
          }
        }
    }
  }

#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    float lt = xor_sum(xor_sum(lsum[qb], 16), 32);
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
__device__ __forceinline__ void attend(const AttnArgs& a, int32_t row, int32_t r0, DescGen<R> gen) {
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

template <class R>
__device__ __forceinline__ DescGen<R> make_gen(R r, const int32_t* cols, int32_t n_cols, int32_t r0,
                                               int32_t n) {
  DescGen<R> g;
  g.ranges = r;
  g.cols = cols;
  g.n_cols = n_cols;
  g.p = g.hi = g.cp = 0;
  g.r0 = r0;
  g.n = n;
  return g;
}

template <typename T> constexpr int threads_of() { return sizeof(T) == 2 ? 64 * BF16_WAVES : 64; }
template <typename T> constexpr int waves_per_eu() { return sizeof(T) == 2 ? 2 : 1; }

template <typename T, int D>
__global__ __launch_bounds__(threads_of<T>()) __attribute__((amdgpu_waves_per_eu(waves_per_eu<T>(), waves_per_eu<T>()))) void attn_vs_kernel(AttnArgs a, VsIndex ix) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  int32_t row, blk;
  work_item(a, nb, row, blk);
  const int32_t r0 = blk * BLOCK;
  const size_t cb = (size_t)row * nb + blk;
  VsRanges rg{ix.iv + (size_t)row * ix.max_iv * 2, min(ix.n_iv[row], ix.max_iv), 0, r0, a.seq_len};
  attend<T, D>(a, row, r0,
               make_gen(rg, ix.cols + cb * ix.max_cols, min(ix.n_cols[cb], ix.max_cols), r0, a.seq_len));
}

template <typename T, int D>
__global__ __launch_bounds__(threads_of<T>()) __attribute__((amdgpu_waves_per_eu(waves_per_eu<T>(), waves_per_eu<T>()))) void attn_blocks_kernel(AttnArgs a, BlockIndex ix) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  int32_t row, blk;
  work_item(a, nb, row, blk);
  const size_t cb = (size_t)row * nb + blk;
  BlockRanges rg{ix.sel + cb * ix.max_sel, min(ix.n_sel[cb], ix.max_sel), 0, a.seq_len};
  attend<T, D>(a, row, blk * BLOCK, make_gen(rg, (const int32_t*)nullptr, 0, blk * BLOCK, a.seq_len));
}

template <typename T, int D>
__global__ __launch_bounds__(threads_of<T>()) __attribute__((amdgpu_waves_per_eu(waves_per_eu<T>(), waves_per_eu<T>()))) void attn_stream_kernel(AttnArgs a, StreamIndex ix) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  int32_t row, blk;
  work_item(a, nb, row, blk);
  StreamRanges rg{blk, ix.init_blocks, ix.local_blocks, 0, a.seq_len};
  attend<T, D>(a, row, blk * BLOCK, make_gen(rg, (const int32_t*)nullptr, 0, blk * BLOCK, a.seq_len));
}

}  // namespace

hipError_t launch_attention_vs(const AttnArgs& a, const VsIndex& ix, hipStream_t s) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.rows * nb;
  if (grid == 0) return hipSuccess;
  auto fn = a.dtype == BF16 ? (a.head_dim == 64 ? attn_vs_kernel<uint16_t, 64> : attn_vs_kernel<uint16_t, 128>)
                            : (a.head_dim == 64 ? attn_vs_kernel<float, 64> : attn_vs_kernel<float, 128>);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(a.dtype == BF16 ? 64 * BF16_WAVES : 64), 0, s, a, ix);
  return hipGetLastError();
}

hipError_t launch_attention_blocks(const AttnArgs& a, const BlockIndex& ix, hipStream_t s) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.rows * nb;
  if (grid == 0) return hipSuccess;
  auto fn = a.dtype == BF16 ? (a.head_dim == 64 ? attn_blocks_kernel<uint16_t, 64> : attn_blocks_kernel<uint16_t, 128>)
                            : (a.head_dim == 64 ? attn_blocks_kernel<float, 64> : attn_blocks_kernel<float, 128>);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(a.dtype == BF16 ? 64 * BF16_WAVES : 64), 0, s, a, ix);
  return hipGetLastError();
}

hipError_t launch_attention_stream(const AttnArgs& a, const StreamIndex& ix, hipStream_t s) {
  const int32_t nb = (a.seq_len + BLOCK - 1) / BLOCK;
  const long long grid = (long long)a.rows * nb;
  if (grid == 0) return hipSuccess;
  auto fn = a.dtype == BF16 ? (a.head_dim == 64 ? attn_stream_kernel<uint16_t, 64> : attn_stream_kernel<uint16_t, 128>)
                            : (a.head_dim == 64 ? attn_stream_kernel<float, 64> : attn_stream_kernel<float, 128>);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(a.dtype == BF16 ? 64 * BF16_WAVES : 64), 0, s, a, ix);
  return hipGetLastError();
}

}  // namespace dsa
