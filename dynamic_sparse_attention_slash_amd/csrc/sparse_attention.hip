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
// block of 64 rows) for the vertical-slash and block-sparse patterns (bf16:
// two waves of 32 queries; fp32: one wave of 64), and one per panel of two
// query blocks for the streaming pattern (bf16: four waves). A prologue cuts
// the key set into 16-key sub-blocks and writes their descriptors to LDS, so
// the hot loop is straight-line code over tiles of sub-blocks:
//   S^T (keys x queries) = K_tile * Q^T      MFMA; bf16 K/V tiles go global
//                                            -> LDS by DMA (gathered rows and
//                                            unaligned ranges alike); fp32 K
//                                            rows are read straight to registers
//   P = exp2(S * scale*log2e - m)            fp32, one query column per lane
//   O^T (dims x queries) += V_tile^T * P^T   MFMA; V_tile^T comes from a
//                                            transposing LDS read (bf16) or is
//                                            read row-wise (fp32, whose MFMA
//                                            takes one k per lane)
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
      // ids outside [0, nb) name no key block (and would overflow c * 64)
      if (c < 0 || c > (n - 1) / BLOCK) continue;
      lo = c * BLOCK;
      hi = min(n, lo + BLOCK);
      if (lo < hi) return true;
    }
    return false;
  }
};
struct StreamRanges {
  int32_t a, init_blocks, local_blocks, t, n;
  __device__ void stage_into(int32_t*) {}  // closed form: nothing staged
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
// bf16 panel kernel (streaming heads): a work-group takes a panel of PANEL = 2
// consecutive query blocks (rows r0 .. r0 + 127) with four waves; wave w owns
// the 32 queries starting at r0 + 64 (w >> 1) + 32 (w & 1).
//
// The key sets of the two blocks are walked together as one stream of 16-key
// sub-blocks, each carrying, per block, a mask of the slots that belong to that
// block's key set. Each window (the sink, the local window) is cut as the union
// of the two blocks' windows, which overlap in all but one key block, so the
// keys are loaded once for both blocks. A tile is 64 keys (4 sub-blocks). K and V tiles travel global -> LDS with
// buffer_load_dwordx4 ... lds (no registers involved) into a two-stage ring:
// the loads of tile t+1 are in flight while tile t is computed, and one
// barrier per tile separates them. Wave w loads sub-block w of a tile; each
// wave then computes on the tile's two 32-key halves, skipping a half that
// holds no key of its block. Both matrices are row-major in LDS with the
// 16-byte chunks of row r XOR-swizzled by r, so that the operand reads are free
// of bank conflicts:
//   K operand (MFMA A, 8 dims of one key per lane): ds_read_b128
//   V^T operand (MFMA A, 8 keys of one dim per lane): two ds_read_b64_tr_b16,
//     the gfx950 transposing LDS read (each 16-lane group reads a 16 x 4 block
//     of b16 and lane i receives element (4j + i/4, i%4) for j = 0..3).
// ---------------------------------------------------------------------------
constexpr int PANEL = 2;                // query blocks per work-group
constexpr int PANEL_WAVES = 2 * PANEL;  // 32 queries per wave
constexpr int32_t P_SB_CAP = 512;       // sub-block descriptors per refill (128 tiles)
constexpr int32_t P_LIST = 1;           // keys come from the staged column list
constexpr int32_t P_DIAG = 2;           // << j: may hold a key above block j's first row

struct PDesc {
  int32_t a;    // first key (range) or position in the staged column list
  uint32_t vm;  // valid slots: bits 0-15 for block 0 of the panel, 16-31 for block 1
  int32_t f;    // P_LIST | P_DIAG << j | (entries to load, for a list) << 8
};

__device__ __forceinline__ PDesc uniform_pdesc(const PDesc* d, int32_t t) {
  const PDesc x = d[t];
  return PDesc{__builtin_amdgcn_readfirstlane(x.a), (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)x.vm),
               __builtin_amdgcn_readfirstlane(x.f)};
}

// Slots s + i (i < 16) that lie in [lo, hi).
__device__ __forceinline__ uint32_t slot_mask(int32_t s, int32_t lo, int32_t hi) {
  const int32_t b0 = min(max(lo - s, 0), 16), b1 = min(max(hi - s, 0), 16);
  return b1 > b0 ? ((1u << b1) - 1u) & ~((1u << b0) - 1u) : 0u;
}

// ---- window sources: next() gives one interval's key window per block of
// the panel ([lo, hi) within [0, n), empty when lo >= hi); state is uniform ----
struct StreamPanelRanges {
  int32_t a0, nb, init_blocks, local_blocks, t, n;
  __device__ bool next(int32_t (&lo)[PANEL], int32_t (&hi)[PANEL]) {
    while (t < 2) {
      const int32_t which = t++;
      bool any = false;
#pragma unroll
      for (int j = 0; j < PANEL; ++j) {
        const int32_t aj = a0 + j;
        lo[j] = hi[j] = 0;
        if (aj < nb) {
          const int32_t sink_end = min(init_blocks, aj + 1);
          if (which == 0) {
            hi[j] = min(n, sink_end * BLOCK);
          } else {
            const int32_t c0 = max(aj - local_blocks + 1, sink_end);
            if (c0 <= aj) { lo[j] = c0 * BLOCK; hi[j] = min(n, (aj + 1) * BLOCK); }
          }
        }
        any |= lo[j] < hi[j];
      }
      if (any) return true;
    }
    return false;
  }
};

// Cuts the union of each interval's windows into sub-blocks, resuming where
// the last call stopped. Each interval starts on an even sub-block, so that a
// half tile never mixes the tail of one interval with the head of the next.
struct PanelCut {
  int32_t p, hi, lo_j[PANEL], hi_j[PANEL];
  bool exhausted;
};

__device__ __forceinline__ void empty_desc(PDesc* d, int32_t t, int32_t tid) {
  if (tid == 0) d[t] = PDesc{0, 0u, 0};
}

template <class R>
__device__ int32_t cut_ranges(R& src, PanelCut& c, PDesc* d, int32_t cnt, int32_t r0, int32_t tid,
                              int32_t nth) {
  while (cnt < P_SB_CAP) {
    if (c.p >= c.hi) {
      int32_t lo[PANEL], hi[PANEL];
      if (!src.next(lo, hi)) { c.exhausted = true; break; }
      int32_t ulo = 0x7fffffff, uhi = 0;
#pragma unroll
      for (int j = 0; j < PANEL; ++j) {
        if (lo[j] < hi[j]) { ulo = min(ulo, lo[j]); uhi = max(uhi, hi[j]); }
        c.lo_j[j] = lo[j];
        c.hi_j[j] = hi[j];
      }
      c.p = ulo;
      c.hi = uhi;
      if (cnt & 1) empty_desc(d, cnt++, tid);
      continue;
    }
    const int32_t take = min((c.hi - c.p + 15) >> 4, P_SB_CAP - cnt);
    for (int32_t t = tid; t < take; t += nth) {
      const int32_t s = c.p + 16 * t;
      uint32_t vm = 0;
      int32_t f = 0;
#pragma unroll
      for (int j = 0; j < PANEL; ++j) {
        const uint32_t m = slot_mask(s, c.lo_j[j], c.hi_j[j]);
        vm |= m << (16 * j);
        if (m && s + 15 > r0 + BLOCK * j) f |= P_DIAG << j;
      }
      d[cnt + t] = PDesc{s, vm, f};
    }
    cnt += take;
    c.p = min(c.hi, c.p + 16 * take);
  }
  return cnt;
}

__device__ __forceinline__ int32_t pad_tiles(PDesc* d, int32_t cnt, int32_t tid) {
  while (cnt & 3) empty_desc(d, cnt++, tid);
  return cnt;
}

struct StreamPanelSrc {
  static constexpr int32_t COLS = 1;
  StreamPanelRanges rg;
  PanelCut cut;
  int32_t r0;
  __device__ int32_t fill(PDesc* d, int32_t*, int32_t tid, int32_t nth) {
    const int32_t cnt = cut.exhausted ? 0 : cut_ranges(rg, cut, d, 0, r0, tid, nth);
    return pad_tiles(d, cnt, tid);
  }
};

template <int D>
struct TileLds {
  static constexpr int ROW = D * 2;           // bytes per key row
  static constexpr int UNITS = ROW / 16;      // 16-byte chunks per row
  static constexpr int MAT = 32 * ROW;        // one 32-key matrix
  static constexpr int HALF = 2 * MAT;        // K then V of a 32-key half tile
  static constexpr int STAGE = 2 * HALF;      // a 64-key tile
  static constexpr int RPI = 64 / UNITS;      // rows per buffer_load_dwordx4 ... lds
  static constexpr int INSTR = 16 / RPI;      // instructions per 16-row sub-block
  // Chunk swizzle of row r: an XOR-linear map of r's low four bits (table
  // below, one nibble per r) under which every operand read is free of bank
  // conflicts, for D = 64 and 128. gfx950 LDS has 64 four-byte banks and, as
  // measured with the bank-conflict counter, serves a ds_read_b128 in four
  // passes of 16 lanes (each half-wave's lane quads q = l >> 2 split by the
  // parity of q & 7: lanes 0-3, 12-15, 20-23, 24-27 form the first pass) and a
  // ds_read_b64 / ds_read_b64_tr_b16 in two passes of 32 lanes. The K reads (16
  // rows at one logical chunk per 16 lanes) and the V^T reads (4 rows x 2
  // chunks per 16 lanes) touch distinct banks in every pass.
  __device__ static int swz(int r) { return lds_chunk_swz(r) & (UNITS - 1); }
  // byte offset of logical chunk c of row r
  __device__ static int off(int r, int c) { return r * ROW + 16 * (c ^ swz(r)); }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Max of the eight scores a lane holds for query block qb of a 32-key tile.
// This file is compiled without NaN semantics (-fno-honor-nans; a masked
// score is -inf, never NaN), so fmaxf needs no operand quieting and the
// compiler forms v_max3_f32 itself, with the wait states that a VALU read of
// an MFMA result needs in front of it.
template <int QB>
__device__ __forceinline__ float tile_max(const f32x4 (&st)[2][QB], int qb) {
  const float a = fmaxf(fmaxf(st[0][qb][0], st[0][qb][1]), st[0][qb][2]);
  const float b = fmaxf(fmaxf(a, st[0][qb][3]), st[1][qb][0]);
  const float c = fmaxf(fmaxf(b, st[1][qb][1]), st[1][qb][2]);
  return fmaxf(c, st[1][qb][3]);
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

template <int D, class Src>
__device__ void attend_panel(const uint16_t* __restrict__ qs, const uint16_t* __restrict__ ks,
                             const uint16_t* __restrict__ vs, uint16_t* __restrict__ os,
                             int32_t n, int32_t r0, float scale_log2, Src src) {
  using L = TileLds<D>;
  constexpr int DS = D / 32;      // MFMA k-steps of Q.K
  constexpr int DB = D / 16;      // 16-dim output blocks
  constexpr int NTH = 64 * PANEL_WAVES;
  // two ring stages in distinct arrays: the compiler can then prove that the
  // loads in flight into one stage do not alias the reads of the other
  __shared__ __align__(16) char ring0[L::STAGE];
  __shared__ __align__(16) char ring1[L::STAGE];
  __shared__ PDesc desc[P_SB_CAP];
  __shared__ int32_t lcols[Src::COLS];

  const int32_t tid = threadIdx.x, lane = tid & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int32_t blk = wave >> 1;                                  // block of the panel
  const int32_t g = lane >> 4, l16 = lane & 15;
  const int32_t q0 = r0 + BLOCK * blk + 32 * (wave & 1);

  // Q^T operands: query row q0 + 16qb + l16, dims (D/4)g + 8s .. + 7
  u32x4 qop[2][DS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int32_t row = min(q0 + 16 * qb + l16, n - 1);
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(qs + (size_t)row * D + (D / 4) * g);
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[qb][s] = qsrc[s];
  }

  // per-lane LDS offsets within a half tile
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
  // global -> LDS load k of this wave's sub-block: lane takes row ld_row[k] of
  // the sub-block at logical chunk c(k), landing at LDS byte 16*lane of the load
  int32_t ld_row[L::INSTR], ld_off[L::INSTR];
#pragma unroll
  for (int k = 0; k < L::INSTR; ++k) {
    ld_row[k] = k * L::RPI + lane / L::UNITS;
    const int32_t c = (lane % L::UNITS) ^ L::swz(16 * (wave & 1) + ld_row[k]);
    ld_off[k] = ld_row[k] * L::ROW + 16 * c;
  }
  // The whole key offset goes into the per-lane offset, which the buffer
  // range check covers: rows past the end of the head's slab read as zeros.
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
  // a raw logit above raise[qb] lifts the row's reference past the margin
  const float inv_scale_log2 = 1.0f / scale_log2;
  float raise[2] = {(NEG_BIG + 8.0f) * inv_scale_log2, (NEG_BIG + 8.0f) * inv_scale_log2};
  // row + 1 - 4g for query qb of this lane: keys up to the row, counted from
  // the lane's first slot
  int32_t rp1[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) rp1[qb] = q0 + 16 * qb + l16 + 1 - 4 * g;
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

  // loads of sub-block dw into this wave's quarter of a stage. Slots past a
  // range's end read the rows that follow (zeros past the slab) and slots past
  // a list's count repeat its last entry; the masks drop them.
  auto issue_loads = [&](const PDesc& dw, char* stage) {
    char* dst = stage + blk * L::HALF + 16 * (wave & 1) * L::ROW;
    if (dw.f & P_LIST) {
      const int32_t last = max(((dw.f >> 8) & 31) - 1, 0);
#pragma unroll
      for (int k = 0; k < L::INSTR; ++k) {
        const int32_t key = lcols[dw.a + min(ld_row[k], last)];
        const int32_t vo = ld_off[k] + (key - ld_row[k]) * L::ROW;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(dst + k * 1024), 16, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + L::MAT + k * 1024), 16, vo, 0, 0, 0);
      }
    } else {
      const int32_t base = dw.a * L::ROW;
#pragma unroll
      for (int k = 0; k < L::INSTR; ++k) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(dst + k * 1024), 16, base + ld_off[k], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + L::MAT + k * 1024), 16, base + ld_off[k], 0, 0, 0);
      }
    }
  };

  // one 32-key half tile (sub-blocks d0, d1) for this wave's queries
  auto half = [&](const char* cur, const PDesc& d0, const PDesc& d1) {
    const uint32_t m0 = (d0.vm >> (16 * blk)) & 0xffffu, m1 = (d1.vm >> (16 * blk)) & 0xffffu;
    if ((m0 | m1) == 0u) return;
    // S^T = K Q^T: K operands of both sub-blocks in one batch of LDS reads,
    // the MFMAs at raised wave priority (as in the single-block kernel)
    u32x4 kop[2][DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        kop[s2][s] = *reinterpret_cast<const u32x4*>(cur + koff[s] + s2 * 16 * L::ROW);
    f32x4 st[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) st[s2][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_setprio(1);
    // k-step major: the four accumulator chains interleave
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) st[s2][qb] = mfma_bf16(kop[s2][s], qop[qb][s], st[s2][qb]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if ((m0 & m1) != 0xffffu || ((d0.f | d1.f) & (P_DIAG << blk))) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const PDesc& dd = s2 ? d1 : d0;
        const uint32_t ms = s2 ? m1 : m0;
        if (dd.f & P_LIST) {
          // gathered keys: slot validity and key <= row, element by element
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int32_t slot = 4 * g + i;
            const bool valid = (ms >> slot) & 1u;
            const int32_t key = lcols[dd.a + slot];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              if (!valid || key > q0 + 16 * qb + l16) st[s2][qb][i] = -INFINITY;
          }
        } else {
          // a range: the valid slots are one run [lo, hi), and key <= row
          // keeps slots below row + 1 - a; lane slot 4g + i is kept when
          // i < min(hi, row + 1 - a) - 4g (and i >= lo - 4g)
          const int32_t lo = ms ? __builtin_ctz(ms) : 16;
          const int32_t hi = ms ? 32 - __builtin_clz(ms) : 0;
          if (dd.f & (P_DIAG << blk)) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              const int32_t ub = min(hi - 4 * g, rp1[qb] - dd.a);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (i >= ub) st[s2][qb][i] = -INFINITY;
            }
          } else if (hi < 16) {
            // below the diagonal only the run's end bounds the slots
            const int32_t ub = hi - 4 * g;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool drop = i >= ub;
#pragma unroll
              for (int qb = 0; qb < 2; ++qb)
                if (drop) st[s2][qb][i] = -INFINITY;
            }
          }
          if (lo > 0) {
            const int32_t lb = lo - 4 * g;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (i < lb) st[s2][qb][i] = -INFINITY;
          }
        }
      }
    }
    // running max, raised only past a 2^8 margin: a lane compares its own
    // part of the row with the raise threshold; only when some row crosses it
    // are the row maxima gathered and O rescaled
    float mx[2];
    bool up_any = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      mx[qb] = tile_max<2>(st, qb);
      up_any |= mx[qb] > raise[qb];
    }
    if (__any(up_any)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mt = group_max4(mx[qb]) * scale_log2;
        const bool up = mt > m[qb] + 8.0f;
        const float alpha = up ? fast_exp2(m[qb] - mt) : 1.0f;
        m[qb] = up ? mt : m[qb];
        raise[qb] = (m[qb] + 8.0f) * inv_scale_log2;
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
    u32x4 vop[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 x0 = lds_read_tr16(cur + voff[db]);
      const u32x2 x1 = lds_read_tr16(cur + voff[db] + 16 * L::ROW);
      vop[db] = u32x4{x0[0], x0[1], x1[0], x1[1]};
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = mfma_bf16(vop[db], pop[qb], oacc[db][qb]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[DB][qb] = mfma_bf16(ones, pop[qb], oacc[DB][qb]);
    __builtin_amdgcn_s_setprio(0);
  };

  // one tile: wait for its loads, start the next tile's, compute both halves
  auto tile = [&](int32_t tt, int32_t ntiles, const char* cur, char* nxt) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's loads of tile tt have landed
    __syncthreads();                 // ... and the other waves'; tile tt-1 is consumed
    if (tt + 1 < ntiles) issue_loads(uniform_pdesc(desc, 4 * (tt + 1) + wave), nxt);
    half(cur, uniform_pdesc(desc, 4 * tt), uniform_pdesc(desc, 4 * tt + 1));
    half(cur + L::HALF, uniform_pdesc(desc, 4 * tt + 2), uniform_pdesc(desc, 4 * tt + 3));
  };

  while (true) {
    __syncthreads();               // previous refill fully consumed
    const int32_t cnt = src.fill(desc, lcols, tid, NTH);   // a multiple of 4
    if (cnt == 0) break;
    __syncthreads();
    const int32_t ntiles = cnt >> 2;
    issue_loads(uniform_pdesc(desc, wave), ring0);
    for (int32_t tt = 0; tt < ntiles; tt += 2) {
      tile(tt, ntiles, ring0, ring1);
      if (tt + 1 < ntiles) tile(tt + 1, ntiles, ring1, ring0);
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
        const f32x4 x = oacc[db][qb] * inv;
        *reinterpret_cast<u32x2*>(os + (size_t)row * D + 16 * db + 4 * g) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 single-block kernel: one work-group per (row, query block), two waves
// of 32 queries, over the block's own key set cut into 16-key sub-blocks
// (first key or list position, count, flags) by DescGen. 32-key tiles go
// global -> LDS through a two-stage ring as in the panel kernel (same
// swizzle, masks and softmax); a work-group needs 40 KB of LDS, so four are
// resident per CU.
// ---------------------------------------------------------------------------
// A global int32 list read through an LDS window: get(i) is called with the
// same i by every thread of the work-group; when i leaves the window, the
// threads load the next `cap` entries together (one round trip instead of one
// per entry).
struct StagedList {
  const int32_t* src; int32_t n;
  int32_t* buf; int32_t cap;
  int32_t base, cnt;
  int32_t tid, nth;
  __device__ int32_t get(int32_t i) {
    if (i >= base + cnt) {
      __syncthreads();   // the window's last entries are consumed
      base = i;
      cnt = min(cap, n - i);
      for (int32_t j = tid; j < cnt; j += nth) buf[j] = src[i + j];
      __syncthreads();
    }
    return buf[i - base];
  }
};

// VsRanges and BlockRanges over staged lists (the interval pairs, the block ids)
struct VsRangesStaged {
  StagedList iv; int32_t n_iv, t, r0, n;
  __device__ void stage_into(int32_t* buf) { iv.buf = buf; }
  __device__ bool next(int32_t& lo, int32_t& hi) {
    while (t < n_iv) {
      const int32_t d_lo = iv.get(2 * t), d_hi = iv.get(2 * t + 1);
      ++t;
      if (d_lo >= r0 + BLOCK) { t = n_iv; return false; }  // intervals ascend
      lo = max(0, r0 - d_hi);
      hi = min(n, r0 + BLOCK - d_lo);
      if (lo < hi) return true;
    }
    return false;
  }
};
struct BlockRangesStaged {
  StagedList sel; int32_t n_sel, t, n;
  __device__ void stage_into(int32_t* buf) { sel.buf = buf; }
  __device__ bool next(int32_t& lo, int32_t& hi) {
    while (t < n_sel) {
      const int32_t c = sel.get(t++);
      if (c < 0 || c > (n - 1) / BLOCK) continue;  // outside [0, nb): no key block
      lo = c * BLOCK;
      hi = min(n, lo + BLOCK);
      if (lo < hi) return true;
    }
    return false;
  }
};
constexpr int SB_WAVES = 2;
constexpr int32_t SB1_CAP = 512;       // descriptors per refill
constexpr int32_t SB1_COLS = 1024;     // column-list entries staged per refill

// Fills descriptors like DescGen::fill, but list sub-blocks refer to a copy of
// the column list staged in LDS (positions relative to that copy), at most
// SB1_COLS entries per call, clamped into [0, n).
template <class R>
__device__ int32_t fill_single(DescGen<R>& gen, Desc* d, int32_t* lcols, int32_t tid, int32_t nthreads) {
  int32_t cnt = 0;
  while (cnt < SB1_CAP) {
    if (gen.p >= gen.hi) {
      int32_t lo2, hi2;
      if (!gen.ranges.next(lo2, hi2)) break;
      gen.p = lo2;
      gen.hi = hi2;
      continue;
    }
    const int32_t take = min((gen.hi - gen.p + 15) >> 4, SB1_CAP - cnt);
    for (int32_t t = tid; t < take; t += nthreads) {
      const int32_t s = gen.p + 16 * t, c = min(16, gen.hi - s);
      d[cnt + t] = Desc{s, c | ((c < 16 || s + c - 1 > gen.r0) ? F_MASK : 0)};
    }
    cnt += take;
    gen.p = min(gen.hi, gen.p + 16 * take);
  }
  if (cnt < SB1_CAP && gen.cp < gen.n_cols) {
    const int32_t ncol = min(gen.n_cols - gen.cp, min(SB1_COLS, 16 * (SB1_CAP - cnt)));
    // the column buffer also holds the staged range lists: every thread is
    // done with them here (the ranges are exhausted)
    __syncthreads();
    constexpr int BATCH = 4;  // loads in flight per thread
    for (int32_t t0 = 0; t0 < ncol; t0 += BATCH * nthreads) {
      int32_t v[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int32_t t = t0 + u * nthreads + tid;
        v[u] = t < ncol ? gen.cols[gen.cp + t] : 0;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int32_t t = t0 + u * nthreads + tid;
        if (t < ncol) lcols[t] = min(max(v[u], 0), gen.n - 1);
      }
    }
    __syncthreads();
    const int32_t take = (ncol + 15) >> 4;
    for (int32_t t = tid; t < take; t += nthreads) {
      const int32_t s = 16 * t, c = min(16, ncol - s);
      const bool m = c < 16 || lcols[s + c - 1] > gen.r0;
      d[cnt + t] = Desc{s, c | F_LIST | (m ? F_MASK : 0)};
    }
    cnt += take;
    gen.cp += ncol;
  }
  return cnt;
}

// LDS of the single-block kernel: one object per head dimension, whatever
// the key-range source, so that a kernel with several sources (the mixed
// layer) holds it once.
template <int D>
struct SingleLds {
  __align__(16) char ring0[TileLds<D>::HALF];
  __align__(16) char ring1[TileLds<D>::HALF];
  Desc desc[SB1_CAP];
  int32_t lcols[SB1_COLS];
};
template <int D>
__device__ __forceinline__ SingleLds<D>& single_lds() {
  __shared__ SingleLds<D> lds;
  return lds;
}

// SHARED: the LDS comes from single_lds (a kernel with several range
// sources); otherwise it is declared here.
template <int D, class R, bool SHARED = false>
__device__ void attend_single(const uint16_t* __restrict__ qs, const uint16_t* __restrict__ ks,
                              const uint16_t* __restrict__ vs, uint16_t* __restrict__ os,
                              int32_t n, int32_t r0, float scale_log2, DescGen<R> gen) {
  using L = TileLds<D>;
  constexpr int DS = D / 32;
  constexpr int DB = D / 16;
  constexpr int NTH = 64 * SB_WAVES;
  char* ring0;
  char* ring1;
  Desc* desc;
  int32_t* lcols;
  if constexpr (SHARED) {
    SingleLds<D>& lds = single_lds<D>();
    ring0 = lds.ring0;
    ring1 = lds.ring1;
    desc = lds.desc;
    lcols = lds.lcols;
  } else {
    __shared__ __align__(16) char ring0_[L::HALF];
    __shared__ __align__(16) char ring1_[L::HALF];
    __shared__ Desc desc_[SB1_CAP];
    __shared__ int32_t lcols_[SB1_COLS];
    ring0 = ring0_;
    ring1 = ring1_;
    desc = desc_;
    lcols = lcols_;
  }

  const int32_t tid = threadIdx.x, lane = tid & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t g = lane >> 4, l16 = lane & 15;
  const int32_t q0 = r0 + 32 * wave;
  gen.ranges.stage_into(lcols);

  u32x4 qop[2][DS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int32_t row = min(q0 + 16 * qb + l16, n - 1);
    const u32x4* qsrc = reinterpret_cast<const u32x4*>(qs + (size_t)row * D + (D / 4) * g);
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[qb][s] = qsrc[s];
  }
  int32_t koff[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) koff[s] = L::off(l16, (D / 32) * g + s);
  int32_t voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int32_t r = 4 * g + (l16 >> 2), dim = 16 * db + 4 * (l16 & 3);
    voff[db] = L::MAT + L::off(r, dim >> 3) + 2 * (dim & 7);
  }
  // wave w loads sub-block w of a tile
  int32_t ld_row[L::INSTR], ld_off[L::INSTR];
#pragma unroll
  for (int k = 0; k < L::INSTR; ++k) {
    ld_row[k] = k * L::RPI + lane / L::UNITS;
    const int32_t c = (lane % L::UNITS) ^ L::swz(16 * wave + ld_row[k]);
    ld_off[k] = ld_row[k] * L::ROW + 16 * c;
  }
  const uint32_t slab_bytes = (uint32_t)n * L::ROW;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)ks, (short)0, slab_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vs, (short)0, slab_bytes, 0x00020000);

  f32x4 oacc[DB + 1][2];
#pragma unroll
  for (int db = 0; db <= DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {NEG_BIG, NEG_BIG};
  const float inv_scale_log2 = 1.0f / scale_log2;
  float raise[2] = {(NEG_BIG + 8.0f) * inv_scale_log2, (NEG_BIG + 8.0f) * inv_scale_log2};
  int32_t rp1[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) rp1[qb] = q0 + 16 * qb + l16 + 1 - 4 * g;
  const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

  auto issue_loads = [&](const Desc& dw, char* stage) {
    char* dst = stage + 16 * wave * L::ROW;
    if (dw.b & F_LIST) {
      const int32_t last = max(dw.count() - 1, 0);
#pragma unroll
      for (int k = 0; k < L::INSTR; ++k) {
        const int32_t key = lcols[dw.a + min(ld_row[k], last)];
        const int32_t vo = ld_off[k] + (key - ld_row[k]) * L::ROW;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(dst + k * 1024), 16, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + L::MAT + k * 1024), 16, vo, 0, 0, 0);
      }
    } else {
      const int32_t base = dw.a * L::ROW;
#pragma unroll
      for (int k = 0; k < L::INSTR; ++k) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(dst + k * 1024), 16, base + ld_off[k], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(dst + L::MAT + k * 1024), 16, base + ld_off[k], 0, 0, 0);
      }
    }
  };

  auto tile = [&](int32_t tt, int32_t ntiles, int32_t cnt, const char* cur, char* nxt) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tt + 1 < ntiles) issue_loads(uniform_desc(desc, 2 * (tt + 1) + wave, cnt), nxt);
    const Desc d[2] = {uniform_desc(desc, 2 * tt, cnt), uniform_desc(desc, 2 * tt + 1, cnt)};
    // K operands of both sub-blocks in one batch of LDS reads. The MFMA
    // blocks run at raised wave priority, so that the other wave on the SIMD
    // fills the gaps between them with its softmax work.
    u32x4 kop[2][DS];
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        kop[s2][s] = *reinterpret_cast<const u32x4*>(cur + koff[s] + s2 * 16 * L::ROW);
    f32x4 st[2][2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) st[s2][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_s_setprio(1);
    // k-step major: the four accumulator chains interleave
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) st[s2][qb] = mfma_bf16(kop[s2][s], qop[qb][s], st[s2][qb]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if ((d[0].b | d[1].b) & F_MASK) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const Desc& dd = d[s2];
        if (!(dd.b & F_MASK)) continue;
        const int32_t c = dd.count();
        if (dd.b & F_LIST) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int32_t sl = 4 * g + i;
            const bool valid = sl < c;
            const int32_t key = lcols[dd.a + min(sl, max(c - 1, 0))];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
              if (!valid || key > q0 + 16 * qb + l16) st[s2][qb][i] = -INFINITY;
          }
        } else {
          // a range: slots [0, c) valid and key = a + slot <= row
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            const int32_t ub = min(c - 4 * g, rp1[qb] - dd.a);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i >= ub) st[s2][qb][i] = -INFINITY;
          }
        }
      }
    }
    float mx[2];
    bool up_any = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      mx[qb] = tile_max<2>(st, qb);
      up_any |= mx[qb] > raise[qb];
    }
    if (__any(up_any)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mt = group_max4(mx[qb]) * scale_log2;
        const bool up = mt > m[qb] + 8.0f;
        const float alpha = up ? fast_exp2(m[qb] - mt) : 1.0f;
        m[qb] = up ? mt : m[qb];
        raise[qb] = (m[qb] + 8.0f) * inv_scale_log2;
#pragma unroll
        for (int db = 0; db <= DB; ++db) oacc[db][qb] *= alpha;
      }
    }
    exp_tile<2>(st, m, scale_log2);
    u32x4 pop[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      pop[qb] = u32x4{pack_bf16x2(st[0][qb][0], st[0][qb][1]), pack_bf16x2(st[0][qb][2], st[0][qb][3]),
                      pack_bf16x2(st[1][qb][0], st[1][qb][1]), pack_bf16x2(st[1][qb][2], st[1][qb][3])};
    // V^T operands in one batch of transposing LDS reads, then the P.V MFMAs
    u32x4 vop[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const u32x2 x0 = lds_read_tr16(cur + voff[db]);
      const u32x2 x1 = lds_read_tr16(cur + voff[db] + 16 * L::ROW);
      vop[db] = u32x4{x0[0], x0[1], x1[0], x1[1]};
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = mfma_bf16(vop[db], pop[qb], oacc[db][qb]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[DB][qb] = mfma_bf16(ones, pop[qb], oacc[DB][qb]);
    __builtin_amdgcn_s_setprio(0);
  };

  while (true) {
    __syncthreads();
    const int32_t cnt = fill_single(gen, desc, lcols, tid, NTH);
    if (cnt == 0) break;
    __syncthreads();
    const int32_t ntiles = (cnt + 1) >> 1;
    issue_loads(uniform_desc(desc, wave, cnt), ring0);
    for (int32_t tt = 0; tt < ntiles; tt += 2) {
      tile(tt, ntiles, cnt, ring0, ring1);
      if (tt + 1 < ntiles) tile(tt + 1, ntiles, cnt, ring1, ring0);
    }
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lt = oacc[DB][qb][0];
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int32_t row = q0 + 16 * qb + l16;
    if (row < n) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 x = oacc[db][qb] * inv;
        *reinterpret_cast<u32x2*>(os + (size_t)row * D + 16 * db + 4 * g) =
            u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (MFMA 16x16x4 f32: one k value per lane, so V needs no transpose)
//
// f32_waves(D) waves share a query block: they fill the descriptor array
// together (the generator's state is the same in every wave). Even waves hold
// queries 0-31, odd waves queries 32-63, and the waves of each half split the
// sub-block pairs (wave w takes pairs w / 2, w / 2 + waves / 2, ...). At the
// end the partial (max, sum, O) of the waves of a half meet in LDS and the
// half's first wave merges them in wave order. A short sequence has few query
// blocks, so one wave per block would leave most of the chip idle: at D = 64
// a wave fits 256 VGPRs, and eight waves per work-group run two per SIMD; at
// D = 128 a wave takes more than 256 VGPRs (one per SIMD), so four.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int f32_waves(int D) { return D >= 128 ? 4 : 8; }
template <int D, class R>
__device__ void attend_f32(const float* __restrict__ qs, const float* __restrict__ ks,
                           const float* __restrict__ vs, float* __restrict__ os, int32_t n,
                           int32_t r0, float scale_log2, DescGen<R> gen) {
  constexpr int DK = D / 4;   // k-steps of Q.K; lane group g holds dims DK*g .. DK*g + DK-1
  constexpr int DB = D / 16;
  // 16-query blocks per wave: a wave's Q and O take 2 * QPW * D / 4 VGPRs per
  // lane, so the waves split the 64 queries in two halves
  constexpr int NW = f32_waves(D);
  constexpr int QPW = 2;
  constexpr int QH = 4 / QPW;            // query groups of the work-group
  constexpr int KW = NW / QH;            // waves splitting the keys of a group
  constexpr int MW = DB * 4 * QPW + 2 * QPW;  // merged floats per lane: max, sum, O
  __shared__ Desc desc[SB_CAP];
  __shared__ float mbuf[(NW - QH) * MW * 64];
  const int32_t lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
  const int32_t qh = wave % QH, kw = wave / QH;
  const int32_t q0 = r0 + 16 * QPW * qh;   // first query of this wave
  const int32_t* cols = gen.cols;

  float qop[QPW][DK];
#pragma unroll
  for (int qb = 0; qb < QPW; ++qb) {
    int32_t row = min(q0 + 16 * qb + l16, n - 1);
    const f32x4* src = reinterpret_cast<const f32x4*>(qs + (size_t)row * D + DK * g);
#pragma unroll
    for (int s = 0; s < DK / 4; ++s) {
      f32x4 x = src[s];
      qop[qb][4 * s] = x[0]; qop[qb][4 * s + 1] = x[1]; qop[qb][4 * s + 2] = x[2]; qop[qb][4 * s + 3] = x[3];
    }
  }
  f32x4 oacc[DB][QPW];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < QPW; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[QPW], lsum[QPW];
#pragma unroll
  for (int qb = 0; qb < QPW; ++qb) { m[qb] = NEG_BIG; lsum[qb] = 0.f; }

  while (true) {
    __syncthreads();
    const int32_t cnt = gen.fill(desc, (int32_t)threadIdx.x, 64 * NW);
    if (cnt == 0) break;
    __syncthreads();
    for (int32_t t = 2 * kw; t < cnt; t += 2 * KW) {
      const Desc d[2] = {uniform_desc(desc, t, cnt), uniform_desc(desc, t + 1, cnt)};
      f32x4 st[2][QPW];
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
        for (int qb = 0; qb < QPW; ++qb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < DK; ++s) acc = mfma_f32(kop[s], qop[qb][s], acc);
          st[s2][qb] = acc;
        }
      }
      if ((d[0].b | d[1].b) & F_MASK) mask_tile<QPW>(st, d, cols, q0, n, lane);
      float alpha[QPW];
      if (update_max<QPW>(st, m, scale_log2, alpha)) {
#pragma unroll
        for (int qb = 0; qb < QPW; ++qb) {
          lsum[qb] *= alpha[qb];
#pragma unroll
          for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha[qb];
        }
      }
      exp_tile<QPW>(st, m, scale_log2);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int qb = 0; qb < QPW; ++qb) lsum[qb] += (st[s2][qb][0] + st[s2][qb][1]) + (st[s2][qb][2] + st[s2][qb][3]);
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
            for (int qb = 0; qb < QPW; ++qb) oacc[db][qb] = mfma_f32(a, st[s2][qb][i], oacc[db][qb]);
          }
        }
    }
  }

  // The waves of a query group hold the same query columns lane by lane (the
  // max is per column, the sums and O per lane), so the merge is lane by lane:
  // element e of a lane of wave w >= QH at mbuf[(w - QH) * MW * 64 + e * 64 + lane].
  // Wave qh (kw = 0) merges waves qh + QH, qh + 2 QH, ... in that order.
  if (kw > 0) {
    float* dst = mbuf + (size_t)(wave - QH) * MW * 64 + lane;
#pragma unroll
    for (int qb = 0; qb < QPW; ++qb) {
      dst[qb * 64] = m[qb];
      dst[(QPW + qb) * 64] = lsum[qb];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < QPW; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(2 * QPW + 4 * QPW * db + 4 * qb + i) * 64] = oacc[db][qb][i];
  }
  __syncthreads();
  if (kw > 0) return;
  for (int32_t k = 1; k < KW; ++k) {
    const float* src = mbuf + (size_t)(qh + QH * k - QH) * MW * 64 + lane;
    float a0[QPW], a1[QPW];
#pragma unroll
    for (int qb = 0; qb < QPW; ++qb) {
      const float mw = src[qb * 64], mx = fmaxf(m[qb], mw);
      a0[qb] = fast_exp2(m[qb] - mx);
      a1[qb] = fast_exp2(mw - mx);
      m[qb] = mx;
      lsum[qb] = lsum[qb] * a0[qb] + src[(QPW + qb) * 64] * a1[qb];
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < QPW; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[db][qb][i] = oacc[db][qb][i] * a0[qb] + src[(2 * QPW + 4 * QPW * db + 4 * qb + i) * 64] * a1[qb];
  }
#pragma unroll
  for (int qb = 0; qb < QPW; ++qb) {
    float lt = xor_sum(xor_sum(lsum[qb], 16), 32);
    float inv = lt > 0.f ? 1.0f / lt : 0.f;
    int32_t row = q0 + 16 * qb + l16;
    if (row < n) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(os + (size_t)row * D + 16 * db + 4 * g) = oacc[db][qb] * inv;
    }
  }
}

// ---------------------------------------------------------------------------
// kernels per index mode
// fp32: one work-group (f32_waves(D) waves) per (row, query block)
// bf16: one work-group (four waves) per (row, panel of two query blocks)
// ---------------------------------------------------------------------------
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

template <int D, class R>
__device__ __forceinline__ void attend_block_f32(const AttnArgs& a, int32_t row, int32_t r0, DescGen<R> gen) {
  const size_t qoff = a.hm.q_slab(row, a.seq_len, D);
  const size_t kvoff = a.hm.kv_slab(row, a.seq_len, D);
  attend_f32<D, R>(static_cast<const float*>(a.q) + qoff, static_cast<const float*>(a.k) + kvoff,
                   static_cast<const float*>(a.v) + kvoff, static_cast<float*>(a.o) + qoff,
                   a.seq_len, r0, a.scale_log2, gen);
}

template <int D, class Src>
__device__ __forceinline__ void attend_panel_bf16(const AttnArgs& a, int32_t row, int32_t r0, const Src& src) {
  const size_t qoff = a.hm.q_slab(row, a.seq_len, D);
  const size_t kvoff = a.hm.kv_slab(row, a.seq_len, D);
  attend_panel<D, Src>(static_cast<const uint16_t*>(a.q) + qoff, static_cast<const uint16_t*>(a.k) + kvoff,
                       static_cast<const uint16_t*>(a.v) + kvoff, static_cast<uint16_t*>(a.o) + qoff,
                       a.seq_len, r0, a.scale_log2, src);
}

__device__ __forceinline__ int32_t num_blocks(int32_t n) { return (n + BLOCK - 1) / BLOCK; }
__device__ __forceinline__ int32_t num_panels(int32_t n) { return (num_blocks(n) + PANEL - 1) / PANEL; }

template <int D>
__global__ __launch_bounds__(64 * f32_waves(D)) void attn_vs_f32_kernel(AttnArgs a, VsIndex ix) {
  const int32_t nb = num_blocks(a.seq_len);
  int32_t row, blk;
  work_item(a.hm, a.wo, nb, row, blk);
  const int32_t r0 = blk * BLOCK;
  const size_t cb = (size_t)row * nb + blk;
  VsRanges rg{ix.iv + (size_t)row * ix.max_iv * 2, min(ix.n_iv[row], ix.max_iv), 0, r0, a.seq_len};
  attend_block_f32<D>(a, row, r0,
                      make_gen(rg, ix.cols + cb * ix.max_cols, min(ix.n_cols[cb], ix.max_cols), r0, a.seq_len));
}

template <int D>
__global__ __launch_bounds__(64 * f32_waves(D)) void attn_blocks_f32_kernel(AttnArgs a, BlockIndex ix) {
  const int32_t nb = num_blocks(a.seq_len);
  int32_t row, blk;
  work_item(a.hm, a.wo, nb, row, blk);
  const size_t cb = (size_t)row * nb + blk;
  BlockRanges rg{ix.sel + cb * ix.max_sel, min(ix.n_sel[cb], ix.max_sel), 0, a.seq_len};
  attend_block_f32<D>(a, row, blk * BLOCK, make_gen(rg, (const int32_t*)nullptr, 0, blk * BLOCK, a.seq_len));
}

template <int D>
__global__ __launch_bounds__(64 * f32_waves(D)) void attn_stream_f32_kernel(AttnArgs a, StreamIndex ix) {
  const int32_t nb = num_blocks(a.seq_len);
  int32_t row, blk;
  work_item(a.hm, a.wo, nb, row, blk);
  StreamRanges rg{blk, ix.init_blocks, ix.local_blocks, 0, a.seq_len};
  attend_block_f32<D>(a, row, blk * BLOCK, make_gen(rg, (const int32_t*)nullptr, 0, blk * BLOCK, a.seq_len));
}

#define PANEL_KERNEL __global__ __launch_bounds__(64 * PANEL_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))

template <int D>
PANEL_KERNEL void attn_stream_bf16_kernel(AttnArgs a, StreamIndex ix) {
  const int32_t nb = num_blocks(a.seq_len);
  int32_t row, p;
  work_item(a.hm, a.wo, num_panels(a.seq_len), row, p);
  const int32_t a0 = PANEL * p;
  StreamPanelSrc src;
  src.rg = StreamPanelRanges{a0, nb, ix.init_blocks, ix.local_blocks, 0, a.seq_len};
  src.cut = PanelCut{};
  src.r0 = a0 * BLOCK;
  attend_panel_bf16<D>(a, row, a0 * BLOCK, src);
}


#define SINGLE_KERNEL __global__ __launch_bounds__(64 * SB_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))

template <int D, class R, bool SHARED = false>
__device__ __forceinline__ void attend_single_bf16(const AttnArgs& a, int32_t row, int32_t r0, DescGen<R> gen) {
  const size_t qoff = a.hm.q_slab(row, a.seq_len, D);
  const size_t kvoff = a.hm.kv_slab(row, a.seq_len, D);
  attend_single<D, R, SHARED>(static_cast<const uint16_t*>(a.q) + qoff, static_cast<const uint16_t*>(a.k) + kvoff,
                      static_cast<const uint16_t*>(a.v) + kvoff, static_cast<uint16_t*>(a.o) + qoff,
                      a.seq_len, r0, a.scale_log2, gen);
}

template <int D>
SINGLE_KERNEL void attn_vs_single_kernel(AttnArgs a, VsIndex ix) {
  const int32_t nb = num_blocks(a.seq_len);
  int32_t row, blk;
  work_item(a.hm, a.wo, nb, row, blk);
  const int32_t r0 = blk * BLOCK;
  const size_t cb = (size_t)row * nb + blk;
  const int32_t niv = max(0, min(ix.n_iv[row], ix.max_iv));
  VsRangesStaged rg{StagedList{ix.iv + (size_t)row * ix.max_iv * 2, 2 * niv, nullptr, SB1_COLS, 0, 0,
                               (int32_t)threadIdx.x, 64 * SB_WAVES},
                    niv, 0, r0, a.seq_len};
  attend_single_bf16<D>(a, row, r0,
                        make_gen(rg, ix.cols + cb * ix.max_cols, max(0, min(ix.n_cols[cb], ix.max_cols)), r0, a.seq_len));
}

template <int D>
SINGLE_KERNEL void attn_blocks_single_kernel(AttnArgs a, BlockIndex ix) {
  const int32_t nb = num_blocks(a.seq_len);
  int32_t row, blk;
  work_item(a.hm, a.wo, nb, row, blk);
  const size_t cb = (size_t)row * nb + blk;
  const int32_t ns = max(0, min(ix.n_sel[cb], ix.max_sel));
  BlockRangesStaged rg{StagedList{ix.sel + cb * ix.max_sel, ns, nullptr, SB1_COLS, 0, 0, (int32_t)threadIdx.x,
                                  64 * SB_WAVES},
                       ns, 0, a.seq_len};
  attend_single_bf16<D>(a, row, blk * BLOCK, make_gen(rg, (const int32_t*)nullptr, 0, blk * BLOCK, a.seq_len));
}

// All heads of a mixed layer in one grid: the work item's head picks its
// pattern, and each pattern runs the single-block attention with its own
// key-range source (the per-pattern kernels' sources), sharing one LDS
// layout.
template <int D>
SINGLE_KERNEL void attn_mixed_single_kernel(AttnArgs a, MixedIndex ix) {
  const int32_t nb = num_blocks(a.seq_len);
  int32_t row, blk;
  work_item(a.hm, a.wo, nb, row, blk);
  const int32_t r0 = blk * BLOCK;
  const int32_t t = row % a.hm.n, b = row / a.hm.n;
  const int32_t kind = ix.kind[t];
  if (kind == PAT_VS) {
    const int32_t prow = b * ix.n_vs + ix.slot[t];
    const size_t cb = (size_t)prow * nb + blk;
    const int32_t niv = max(0, min(ix.vs.n_iv[prow], ix.vs.max_iv));
    VsRangesStaged rg{StagedList{ix.vs.iv + (size_t)prow * ix.vs.max_iv * 2, 2 * niv, nullptr, SB1_COLS, 0, 0,
                                 (int32_t)threadIdx.x, 64 * SB_WAVES},
                      niv, 0, r0, a.seq_len};
    attend_single_bf16<D, VsRangesStaged, true>(a, row, r0,
                          make_gen(rg, ix.vs.cols + cb * ix.vs.max_cols,
                                   max(0, min(ix.vs.n_cols[cb], ix.vs.max_cols)), r0, a.seq_len));
  } else if (kind == PAT_BS) {
    const int32_t prow = b * ix.n_bs + ix.slot[t];
    const size_t cb = (size_t)prow * nb + blk;
    const int32_t ns = max(0, min(ix.bs.n_sel[cb], ix.bs.max_sel));
    BlockRangesStaged rg{StagedList{ix.bs.sel + cb * ix.bs.max_sel, ns, nullptr, SB1_COLS, 0, 0,
                                    (int32_t)threadIdx.x, 64 * SB_WAVES},
                         ns, 0, a.seq_len};
    attend_single_bf16<D, BlockRangesStaged, true>(a, row, r0, make_gen(rg, (const int32_t*)nullptr, 0, r0, a.seq_len));
  } else {
    StreamRanges rg{blk, ix.st.init_blocks, ix.st.local_blocks, 0, a.seq_len};
    attend_single_bf16<D, StreamRanges, true>(a, row, r0, make_gen(rg, (const int32_t*)nullptr, 0, r0, a.seq_len));
  }
}

// grid: rows x query blocks (or x panels of two blocks for the panel kernel)
dim3 attn_grid(const AttnArgs& a, bool panels) {
  const long long nb = (a.seq_len + BLOCK - 1) / BLOCK;
  const long long units = panels ? (nb + PANEL - 1) / PANEL : nb;
  return dim3((unsigned)((long long)a.rows * units));
}

}  // namespace

// Vertical-slash and block-sparse heads run the single-block bf16 kernel:
// their key sets differ between neighbouring query blocks in many narrow
// pieces, and four independent work-groups per CU beat the panel's sharing
// there (measured on MI355X: 6% at 128K, 3-14% on the mixed layers).
// Streaming heads, whose windows two blocks share almost whole, run the panel.
hipError_t launch_attention_vs(const AttnArgs& a, const VsIndex& ix, hipStream_t s) {
  const dim3 grid = attn_grid(a, false);
  if (grid.x == 0) return hipSuccess;
  if (a.dtype == BF16)
    hipLaunchKernelGGL(a.head_dim == 64 ? attn_vs_single_kernel<64> : attn_vs_single_kernel<128>, grid,
                       dim3(64 * SB_WAVES), 0, s, a, ix);
  else
    hipLaunchKernelGGL(a.head_dim == 64 ? attn_vs_f32_kernel<64> : attn_vs_f32_kernel<128>, grid,
                       dim3(64 * f32_waves(a.head_dim)), 0, s, a, ix);
  return hipGetLastError();
}

hipError_t launch_attention_blocks(const AttnArgs& a, const BlockIndex& ix, hipStream_t s) {
  const dim3 grid = attn_grid(a, false);
  if (grid.x == 0) return hipSuccess;
  if (a.dtype == BF16)
    hipLaunchKernelGGL(a.head_dim == 64 ? attn_blocks_single_kernel<64> : attn_blocks_single_kernel<128>, grid,
                       dim3(64 * SB_WAVES), 0, s, a, ix);
  else
    hipLaunchKernelGGL(a.head_dim == 64 ? attn_blocks_f32_kernel<64> : attn_blocks_f32_kernel<128>, grid,
                       dim3(64 * f32_waves(a.head_dim)), 0, s, a, ix);
  return hipGetLastError();
}

// bf16: one grid over every listed head in the order a.wo gives. The library
// passes the pattern-by-pattern order (make_work_order with kinds): the items
// of one pattern stay together as in the per-pattern launches, each pattern's
// query blocks latest first. Putting the heads of a kv group side by side
// whatever their pattern measured up to 20% slower on MI355X for long
// vertical-slash and block-sparse items (Llama-3-8B shapes, 128K-1M). fp32
// runs one launch per pattern over that pattern's heads.
hipError_t launch_attention_mixed(const AttnArgs& a, const MixedIndex& ix, hipStream_t s) {
  if (a.rows == 0 || a.seq_len == 0) return hipSuccess;
  if (a.dtype == BF16) {
    hipLaunchKernelGGL(a.head_dim == 64 ? attn_mixed_single_kernel<64> : attn_mixed_single_kernel<128>,
                       attn_grid(a, false), dim3(64 * SB_WAVES), 0, s, a, ix);
    return hipGetLastError();
  }
  const int32_t batch = a.rows / a.hm.n;
  for (int8_t kind : {PAT_VS, PAT_BS, PAT_STREAM}) {
    AttnArgs p = a;
    p.hm.n = 0;
    for (int32_t t = 0; t < a.hm.n; ++t)
      if (ix.kind[t] == kind) p.hm.h[p.hm.n++] = a.hm.h[t];
    if (p.hm.n == 0) continue;
    p.rows = batch * p.hm.n;
    p.wo = make_work_order(p.hm);
    hipError_t e = kind == PAT_VS   ? launch_attention_vs(p, ix.vs, s)
                   : kind == PAT_BS ? launch_attention_blocks(p, ix.bs, s)
                                    : launch_attention_stream(p, ix.st, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_attention_stream(const AttnArgs& a, const StreamIndex& ix, hipStream_t s) {
  const bool bf16 = a.dtype == BF16;
  const dim3 grid = attn_grid(a, bf16);
  if (grid.x == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(a.head_dim == 64 ? attn_stream_bf16_kernel<64> : attn_stream_bf16_kernel<128>, grid,
                       dim3(64 * PANEL_WAVES), 0, s, a, ix);
  else
    hipLaunchKernelGGL(a.head_dim == 64 ? attn_stream_f32_kernel<64> : attn_stream_f32_kernel<128>, grid,
                       dim3(64 * f32_waves(a.head_dim)), 0, s, a, ix);
  return hipGetLastError();
}

}  // namespace dsa
