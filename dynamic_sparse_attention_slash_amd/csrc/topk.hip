// Exact top-k with a fixed tie order, gfx950.
//
// Selects the vertical / slash indices and the key blocks of the sparse
// patterns [MInference 1.0 article, §2.2: top-k vertical lines and slash lines;
// top-k blocks of the pooled block scores]. The rank order is: the forced entry
// first, then larger score, then smaller index; -0.0 ranks as +0.0 and NaN as
// -inf. Output indices are ascending.
//
// Method: scores map to order-preserving 32-bit keys (the forced entry gets
// the maximum key, which no canonical float reaches). Rows shorter than 64K
// entries and the block lists are selected by one work-group each, which
// first tries a two-read select over 12-bit key bins (described at
// select_bins below; its kept entries come out in index order from an LDS
// bitmap); rows it cannot take use the radix select: a 4-pass
// MSB-first radix select (8 bits per pass) finds the k-th largest key T and
// how many entries equal to T must be kept (need_eq). Each pass counts
// digits into LDS histograms, one copy per wave and lane group so that the
// few bins a float exponent range fills are not hit by a whole wave at once;
// the bin holding the k-th largest key comes from a parallel suffix scan over
// the 256 bins. A compaction pass then walks the entries in index order, each
// wave owning one contiguous segment (which it also visits in the counting
// passes): an entry is kept when key > T, or key == T and fewer than need_eq
// equal keys precede it. Ballot prefix counts give each kept entry its output
// slot, so the result comes out ascending with no sort.
// Rows of 64K entries or more spread the same steps over many work-groups
// (the row-parallel passes further down): row histograms in global memory
// give T 12 + 12 + 8 bits at a time, then every 16K-entry chunk of the row
// counts and writes its kept entries at offsets summed from the earlier
// chunks' counts.
#include "kernels.hpp"

namespace dsa {
namespace {

__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN -> -inf
  if (u == 0x80000000u) u = 0u;                           // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
constexpr uint32_t FORCED_KEY = 0xffffffffu;

template <int NW, int NC>
struct SelectShared {
  uint32_t hist[NW * NC][256];  // per wave and lane group
  uint32_t scan[256];           // wave-local suffix sums of the bin totals
  uint32_t wsum[4];             // bin totals per 64-bin wave slice
  uint32_t wcnt[NW][2];
  uint32_t digit, rem;
};

// The keys of one wave's segment [s0, s1) of the candidates, visited in
// ascending position order 64 at a time: visit(f) calls f(j, key, valid) for
// position s0 + 64 j + lane, j < trips (trips is uniform over the wave).
// The trips' loads are issued VISIT_LOADS at a time ahead of their callbacks
// (which still run in trip order), so that a pass over a long segment is not
// one memory latency per trip.
constexpr int VISIT_LOADS = 8;
struct GlobalSeg {
  const float* x; int32_t forced, s0, s1, trips, lane;
  int32_t base;  // index of x[0] in the output
  template <class F>
  __device__ __forceinline__ void visit(F&& f) const {
    for (int32_t j0 = 0; j0 < trips; j0 += VISIT_LOADS) {
      float xv[VISIT_LOADS];
#pragma unroll
      for (int u = 0; u < VISIT_LOADS; ++u) {
        const int32_t i = s0 + 64 * (j0 + u) + lane;
        xv[u] = (j0 + u < trips && i < s1) ? x[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < VISIT_LOADS; ++u) {
        const int32_t j = j0 + u;
        if (j >= trips) break;
        const int32_t i = s0 + 64 * j + lane;
        const bool valid = i < s1;
        f(j, valid ? (i == forced ? FORCED_KEY : score_key(xv[u])) : 0u, valid);
      }
    }
  }
  __device__ __forceinline__ int32_t index(int32_t j) const { return base + s0 + 64 * j + lane; }
};
// Wave w's segment of m candidates: [w * seg, (w + 1) * seg) clipped to m.
template <int NW>
__device__ __forceinline__ void wave_segment(int32_t m, int32_t& s0, int32_t& s1, int32_t& trips) {
  const int32_t wave = threadIdx.x >> 6;
  const int32_t seg = ((m + NW * 64 - 1) / (NW * 64)) * 64;
  s0 = min(m, wave * seg);
  s1 = min(m, s0 + seg);
  trips = (s1 - s0 + 63) >> 6;
}

// Top kk (1 <= kk < m) of the m candidates, each wave visiting its segment
// through `seg`, written ascending to out[0..kk) (and their keys to
// out_key[0..kk) when out_key is not null). NC histogram copies per wave
// (lane groups of 64 / NC lanes).
template <int NW, int NC, class Seg>
__device__ __forceinline__ void select_topk(const Seg& seg, int32_t kk, int32_t* __restrict__ out,
                                            uint32_t* __restrict__ out_key, SelectShared<NW, NC>& sh) {
  static_assert(NW >= 4, "the digit scan uses the first four waves");
  const int32_t tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int NT = NW * 64;
  uint32_t* hist = &sh.hist[wave * NC + lane / (64 / NC)][0];
  uint32_t prefix = 0, pmask = 0;
  uint32_t rem = (uint32_t)kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < NW * NC * 256; i += NT) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    seg.visit([&](int32_t, uint32_t key, bool valid) {
      if (valid && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    // the digit: the largest bin b whose suffix count S(b) (entries with a
    // digit >= b) reaches rem; thread b of the first four waves owns bin b
    uint32_t t = 0, s = 0;
    if (tid < 256) {
#pragma unroll
      for (int c = 0; c < NW * NC; ++c) t += sh.hist[c][tid];
      s = t;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_down(s, d);
        if (lane + d < 64) s += o;
      }
      sh.scan[tid] = s;
      if (lane == 0) sh.wsum[wave] = s;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t above = 0;
      for (int w = wave + 1; w < 4; ++w) above += sh.wsum[w];
      const uint32_t S = s + above, S1 = S - t;  // S(b), S(b + 1)
      if (S >= rem && S1 < rem) {
        sh.digit = (uint32_t)tid;
        sh.rem = rem - S1;
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= 255u << shift;
    rem = sh.rem;
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = rem;

  // compaction in index order over the waves' segments
  uint32_t n_gt = 0, n_eq = 0;
  seg.visit([&](int32_t, uint32_t key, bool valid) {
    n_gt += __popcll(__ballot(valid && key > T));
    n_eq += __popcll(__ballot(valid && key == T));
  });
  if (lane == 0) { sh.wcnt[wave][0] = n_gt; sh.wcnt[wave][1] = n_eq; }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) { gt_before += sh.wcnt[w][0]; eq_before += sh.wcnt[w][1]; }
  uint32_t eq_seen = eq_before;
  uint32_t pos = gt_before + min(eq_before, need_eq);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  seg.visit([&](int32_t j, uint32_t key, bool valid) {
    const bool eq = valid && key == T;
    const uint64_t eq_mask = __ballot(eq);
    const uint32_t eq_rank = eq_seen + __popcll(eq_mask & lt_mask);
    const bool keep = valid && (key > T || (eq && eq_rank < need_eq));
    const uint64_t keep_mask = __ballot(keep);
    const uint32_t slot = pos + __popcll(keep_mask & lt_mask);
    if (keep && slot < (uint32_t)kk) {
      out[slot] = seg.index(j);
      if (out_key) out_key[slot] = key;
    }
    pos += __popcll(keep_mask);
    eq_seen += __popcll(eq_mask);
  });
}

// Two-read select. Read 1 counts the top BIN_BITS bits of every key into LDS
// bins; a suffix scan over the bins finds the bin b that holds the kk-th
// largest key and how many keys lie in higher bins (all of them are kept).
// Read 2 collects those keys' indices and the (key, index) pairs of bin b in
// LDS. Each bin-b entry's rank among the bin-b entries, in the rank order
// (larger key, then smaller index), decides whether it fills one of the
// remaining places; the kk kept entries are then sorted by index in LDS. A
// row whose bin b holds more than CAND entries (many keys sharing their top
// bits: constant or heavily tied rows), or with kk > KEEP, is left to the
// radix select: the function then returns false having written nothing.
// Either way the result is the unique exact top kk.
constexpr int BIN_BITS = 12, BINS = 1 << BIN_BITS;
constexpr int BIN_LOADS = 8;  // keys loaded ahead per thread
constexpr int BM_WORDS = 2048;  // kept-entry bitmap: rows of up to 65536 entries
template <int NW, int CAND, int KEEP, bool KEYS>
struct BinShared {
  union {
    uint32_t hist[BINS];
    struct {
      // boundary-bin candidates as (key << 32 | ~index): a larger value
      // ranks first (larger key, then smaller index)
      alignas(16) uint64_t cand[CAND];
      union {
        int32_t kidx[KEEP];
        uint32_t bm[BM_WORDS];  // bit i: entry i kept
      };
      uint32_t kkey[KEYS ? KEEP : 1];
    } l;
  } u;
  uint32_t wsum[NW];
  uint32_t bin, above, in_bin, n_c, n_k;
};

// raw_at(i) loads entry i < m (as 32 bits), key_of(i, raw) maps it to its
// key, idx_at(i) gives its output index (distinct values in [0, m)). Entries
// are visited in any order, BIN_LOADS loads issued before their keys are
// formed. Writes out[0..kk) ascending (and their keys to out_key when KEYS).
// Without keys and for rows of up to 32 * BM_WORDS entries, the kept
// entries are marked in an LDS bitmap and written out in index order by a
// popcount prefix sum; otherwise they are gathered and bitonic-sorted.
template <int NW, int CAND, int KEEP, bool KEYS, class RawAt, class KeyOf, class IdxAt>
__device__ bool select_bins(RawAt raw_at, KeyOf key_of, IdxAt idx_at, int32_t m, int32_t kk,
                            int32_t* __restrict__ out, uint32_t* __restrict__ out_key,
                            BinShared<NW, CAND, KEEP, KEYS>& f) {
  constexpr int NT = NW * 64;
  constexpr int PER = BINS / NT;  // bins per thread in the scan
  static_assert(PER * NT == BINS, "bins per thread");
  if (kk > KEEP) return false;    // the kept entries would not fit
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto each_key = [&](auto&& fn) {
    for (int32_t i0 = 0; i0 < m; i0 += BIN_LOADS * NT) {
      uint32_t rv[BIN_LOADS];
#pragma unroll
      for (int u = 0; u < BIN_LOADS; ++u) {
        const int32_t i = i0 + u * NT + tid;
        rv[u] = i < m ? raw_at(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < BIN_LOADS; ++u) {
        const int32_t i = i0 + u * NT + tid;
        if (i < m) fn(i, key_of(i, rv[u]));
      }
    }
  };

  // read 1: bin counts of the top BIN_BITS key bits
  for (int i = tid; i < BINS; i += NT) f.u.hist[i] = 0;
  if (tid == 0) { f.n_c = 0; f.n_k = 0; }
  __syncthreads();
  each_key([&](int32_t, uint32_t key) { atomicAdd(&f.u.hist[key >> (32 - BIN_BITS)], 1u); });
  __syncthreads();
  // thread t owns bins [PER t, PER t + PER); suffix sums over the threads
  uint32_t loc[PER], tsum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { loc[j] = f.u.hist[PER * tid + j]; tsum += loc[j]; }
  uint32_t s = tsum;  // inclusive suffix sum within the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t x = __shfl_down(s, d);
    if (lane + d < 64) s += x;
  }
  if (lane == 0) f.wsum[wave] = s;
  __syncthreads();
  uint32_t higher = s - tsum;  // entries in bins above this thread's
  for (int w = wave + 1; w < NW; ++w) higher += f.wsum[w];
  if (higher < (uint32_t)kk && higher + tsum >= (uint32_t)kk) {
    uint32_t acc = higher;
    for (int j = PER - 1; j >= 0; --j) {
      if (acc + loc[j] >= (uint32_t)kk) {
        f.bin = (uint32_t)(PER * tid + j);
        f.above = acc;
        f.in_bin = loc[j];
        break;
      }
      acc += loc[j];
    }
  }
  __syncthreads();
  const uint32_t bin = f.bin, above = f.above, in_bin = f.in_bin;
  if (in_bin > (uint32_t)CAND) {
    __syncthreads();  // every thread has read the bin before LDS is reused
    return false;
  }
  const bool use_bm = !KEYS && m <= 32 * BM_WORDS;
  const int32_t nw = (m + 31) >> 5;
  if (use_bm) {
    // the bitmap may overlay the bin counts, which every thread copied to
    // registers before the barrier above
    for (int32_t i = tid; i < nw; i += NT) f.u.l.bm[i] = 0u;
    __syncthreads();
  }
  auto keep = [&](int32_t ix, uint32_t key) {
    if (use_bm) {
      atomicOr(&f.u.l.bm[ix >> 5], 1u << (ix & 31));
    } else {
      const uint32_t p = atomicAdd(&f.n_k, 1u);
      f.u.l.kidx[p] = ix;
      if (KEYS) f.u.l.kkey[p] = key;
    }
  };

  // read 2: keys above bin b are kept; bin b entries become candidates
  each_key([&](int32_t i, uint32_t key) {
    const uint32_t hb = key >> (32 - BIN_BITS);
    if (hb > bin) {
      keep(idx_at(i), key);
    } else if (hb == bin) {
      const uint32_t p = atomicAdd(&f.n_c, 1u);
      f.u.l.cand[p] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)idx_at(i);
    }
  });
  __syncthreads();
  // candidate c is kept when fewer than kk - above candidates rank before it
  const uint32_t places = (uint32_t)kk - above;
  for (uint32_t c = tid; c < in_bin; c += NT) {
    const uint64_t cc = f.u.l.cand[c];
    uint32_t rank = 0, e = 0;
    for (; e + 1 < in_bin; e += 2) {  // two candidates per 16-byte LDS read
      const uint64_t* pe = &f.u.l.cand[e];
      rank += (pe[0] > cc ? 1u : 0u) + (pe[1] > cc ? 1u : 0u);
    }
    if (e < in_bin) rank += f.u.l.cand[e] > cc ? 1u : 0u;
    if (rank < places) keep((int32_t)~(uint32_t)cc, (uint32_t)(cc >> 32));
  }
  if (use_bm) {
    // thread t owns bitmap words [wpt t, wpt t + wpt); its set bits go out
    // after those of the threads before it (block prefix of the popcounts)
    __syncthreads();
    const int32_t wpt = (nw + NT - 1) / NT, w0 = tid * wpt, w1 = min(nw, w0 + wpt);
    uint32_t cnt = 0;
    for (int32_t wi = w0; wi < w1; ++wi) cnt += __popc(f.u.l.bm[wi]);
    uint32_t sc = cnt;  // inclusive prefix within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t x = __shfl_up(sc, d);
      if (lane >= d) sc += x;
    }
    if (lane == 63) f.wsum[wave] = sc;
    __syncthreads();
    uint32_t pos = sc - cnt;
    for (int w = 0; w < wave; ++w) pos += f.wsum[w];
    for (int32_t wi = w0; wi < w1; ++wi) {
      uint32_t b = f.u.l.bm[wi];
      while (b) {
        out[pos++] = 32 * wi + __builtin_ctz(b);
        b &= b - 1u;
      }
    }
    return true;
  }
  // ascending indices: bitonic sort of the kk kept entries, padded to a power of two
  int32_t P = 1;
  while (P < kk) P <<= 1;
  __syncthreads();
  for (int32_t i = kk + tid; i < P; i += NT) f.u.l.kidx[i] = 0x7fffffff;
  __syncthreads();
  for (int32_t size = 2; size <= P; size <<= 1) {
    for (int32_t stride = size >> 1; stride > 0; stride >>= 1) {
      for (int32_t t = tid; t < (P >> 1); t += NT) {
        const int32_t i = 2 * t - (t & (stride - 1));  // lower element of the pair
        const int32_t jx = i + stride;
        const bool up = (i & size) == 0;
        const int32_t x = f.u.l.kidx[i], y = f.u.l.kidx[jx];
        if ((x > y) == up) {
          f.u.l.kidx[i] = y;
          f.u.l.kidx[jx] = x;
          if (KEYS) {
            const uint32_t kx = f.u.l.kkey[i];
            f.u.l.kkey[i] = f.u.l.kkey[jx];
            f.u.l.kkey[jx] = kx;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int32_t i = tid; i < kk; i += NT) {
    out[i] = f.u.l.kidx[i];
    if (KEYS) out_key[i] = f.u.l.kkey[i];
  }
  return true;
}

// Rows shorter than RP_MIN_N: one work-group per row, two-read select (kk up
// to 8192), else the radix select.
union RowTopkShared {
  BinShared<16, 2048, 8192, false> f;
  SelectShared<16, 2> r;
};
constexpr int ROW_WAVES = 16;
__global__ __launch_bounds__(ROW_WAVES * 64) void topk_rows_kernel(const float* __restrict__ scores,
                                                                   int32_t n, int32_t kk, int32_t forced,
                                                                   int32_t* __restrict__ out) {
  __shared__ RowTopkShared sh;
  const int32_t row = blockIdx.x;
  int32_t* o = out + (size_t)row * kk;
  if (kk >= n) {
    for (int32_t i = threadIdx.x; i < n; i += ROW_WAVES * 64) o[i] = i;
    return;
  }
  const float* x = scores + (size_t)row * n;
  auto raw_at = [&](int32_t i) { return __float_as_uint(x[i]); };
  auto key_of = [&](int32_t i, uint32_t r) { return i == forced ? FORCED_KEY : score_key(__uint_as_float(r)); };
  auto idx_at = [](int32_t i) { return i; };
  if (select_bins<ROW_WAVES>(raw_at, key_of, idx_at, n, kk, o, (uint32_t*)nullptr, sh.f)) return;
  GlobalSeg seg{x, forced, 0, 0, 0, (int32_t)(threadIdx.x & 63), 0};
  wave_segment<ROW_WAVES>(n, seg.s0, seg.s1, seg.trips);
  select_topk<ROW_WAVES, 2>(seg, kk, o, nullptr, sh.r);
}

// Long rows, row-parallel: every RP_CHUNK-long chunk of a row is one
// work-group of each pass.
//   Passes 1-3 find the row's kk-th largest key K exactly, 12 + 12 + 8 bits at
//   a time: each pass adds the bins of the keys that share K's bits found so
//   far to a row histogram, whose suffix scan then gives the next bits of K and
//   how many keys lie above them.
//   Pass 4 counts, per chunk, the keys above K (gt) and equal to K (eq).
//   Pass 5 writes each chunk's kept entries, in index order, straight to the
//   output: every key above K, and keys equal to K while fewer than
//   need = kk - (keys above K in the row) of them precede it in the row. The
//   chunk's first output slot is the earlier chunks' gt plus min(need, their
//   eq). This is the rank order (larger key, then smaller index) and the
//   output comes out ascending, as in the other selects.
constexpr int32_t RP_CHUNK = 16384;
constexpr int RP_WAVES = 4;
constexpr int RP_BINS2 = 256;  // last level: key bits 7-0

__host__ __device__ constexpr int32_t rp_chunks(int32_t n) { return (n + RP_CHUNK - 1) / RP_CHUNK; }
// Rows of at least RP_MIN_N entries take the row-parallel select (measured: at
// 32K entries one work-group per row is faster, from 64K on the row-parallel
// passes are)
constexpr int32_t RP_MIN_N = 65536;
__host__ __device__ constexpr bool row_parallel(int32_t n, int32_t kk) {
  return n >= RP_MIN_N && kk < n;
}

// workspace, per row: the three level histograms and (K, keys above K), then
// (gt, eq) per chunk and wave
constexpr int32_t RP_HIST_WORDS = 2 * BINS + RP_BINS2 + 2;
__host__ __device__ constexpr size_t rp_bytes(int32_t rows, int32_t nch) {
  return (size_t)rows * ((size_t)RP_HIST_WORDS + 2 * RP_WAVES * (size_t)nch) * sizeof(uint32_t);
}

// Over an NB-bin histogram h (global), the bin holding the r-th largest entry
// (1 <= r <= total) and the number of entries in the bins above it, for every
// thread of the work-group. Thread t owns bins [PER t, PER t + PER).
template <int NW, int NB>
__device__ void boundary_bin(const uint32_t* __restrict__ h, uint32_t r, uint32_t* wsum, uint32_t* res,
                             uint32_t& bin, uint32_t& above) {
  constexpr int NT = NW * 64, PER = NB / NT;
  static_assert(PER * NT == NB, "bins per thread");
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t loc[PER], tsum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { loc[j] = h[PER * tid + j]; tsum += loc[j]; }
  uint32_t s = tsum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t x = __shfl_down(s, d);
    if (lane + d < 64) s += x;
  }
  if (lane == 0) wsum[wave] = s;
  __syncthreads();
  uint32_t higher = s - tsum;
  for (int v = wave + 1; v < NW; ++v) higher += wsum[v];
  if (higher < r && higher + tsum >= r) {
    uint32_t acc = higher;
    for (int j = PER - 1; j >= 0; --j) {
      if (acc + loc[j] >= r) { res[0] = (uint32_t)(PER * tid + j); res[1] = acc; break; }
      acc += loc[j];
    }
  }
  __syncthreads();
  bin = res[0];
  above = res[1];
  __syncthreads();  // res and wsum are reused
}

struct RpBound { uint32_t key, above; };  // K, keys above K in the row (passes >= LEVEL)

// K's bits known before pass LEVEL (LEVEL 0: none; 1: bits 31-20; 2: bits 31-8;
// 3: all) and the count of keys above them.
template <int LEVEL>
__device__ RpBound rp_bound(const uint32_t* __restrict__ hr, int32_t kk, uint32_t* wsum, uint32_t* res) {
  RpBound b{0u, 0u};
  if (LEVEL >= 1) {
    uint32_t b0, a0;
    boundary_bin<RP_WAVES, BINS>(hr, (uint32_t)kk, wsum, res, b0, a0);
    b.key = b0 << 20;
    b.above = a0;
  }
  if (LEVEL >= 2) {
    uint32_t b1, a1;
    boundary_bin<RP_WAVES, BINS>(hr + BINS, (uint32_t)kk - b.above, wsum, res, b1, a1);
    b.key |= b1 << 8;
    b.above += a1;
  }
  if (LEVEL >= 3) {
    uint32_t b2, a2;
    boundary_bin<RP_WAVES, RP_BINS2>(hr + 2 * BINS, (uint32_t)kk - b.above, wsum, res, b2, a2);
    b.key |= b2;
    b.above += a2;
  }
  return b;
}

__global__ __launch_bounds__(256) void rp_zero_kernel(uint32_t* __restrict__ p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// Pass LEVEL + 1 (LEVEL 0, 1, 2): histogram of the next bits of the keys that
// share K's known bits.
template <int LEVEL>
__global__ __launch_bounds__(RP_WAVES * 64) void rp_hist_kernel(const float* __restrict__ scores, int32_t n,
                                                                 int32_t kk, int32_t forced, uint32_t* __restrict__ ws) {
  constexpr int NT = RP_WAVES * 64;
  constexpr int NB = LEVEL == 2 ? RP_BINS2 : BINS;
  __shared__ uint32_t h[NB];
  __shared__ uint32_t wsum[RP_WAVES], res[2];
  const int32_t c = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const int32_t c0 = c * RP_CHUNK, m = min(RP_CHUNK, n - c0), f = forced - c0;
  uint32_t* hr = ws + (size_t)row * RP_HIST_WORDS;
  const RpBound b = rp_bound<LEVEL>(hr, kk, wsum, res);
  for (int i = tid; i < NB; i += NT) h[i] = 0u;
  __syncthreads();
  const float* x = scores + (size_t)row * n + c0;
  for (int32_t i0 = 0; i0 < m; i0 += BIN_LOADS * NT) {
    float v[BIN_LOADS];
#pragma unroll
    for (int u = 0; u < BIN_LOADS; ++u) {
      const int32_t i = i0 + u * NT + tid;
      v[u] = i < m ? x[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < BIN_LOADS; ++u) {
      const int32_t i = i0 + u * NT + tid;
      if (i >= m) continue;
      const uint32_t key = i == f ? FORCED_KEY : score_key(v[u]);
      if (LEVEL == 0) atomicAdd(&h[key >> 20], 1u);
      else if (LEVEL == 1) { if ((key >> 20) == (b.key >> 20)) atomicAdd(&h[(key >> 8) & (BINS - 1)], 1u); }
      else if ((key >> 8) == (b.key >> 8)) atomicAdd(&h[key & (RP_BINS2 - 1)], 1u);
    }
  }
  __syncthreads();
  uint32_t* ho = hr + LEVEL * BINS;
  for (int i = tid; i < NB; i += NT)
    if (h[i]) atomicAdd(&ho[i], h[i]);
}

// K and the number of keys above it, once per row, for passes 4 and 5.
__global__ __launch_bounds__(RP_WAVES * 64) void rp_bound_kernel(int32_t kk, uint32_t* __restrict__ ws) {
  __shared__ uint32_t wsum[RP_WAVES], res[2];
  uint32_t* hr = ws + (size_t)blockIdx.x * RP_HIST_WORDS;
  const RpBound b = rp_bound<3>(hr, kk, wsum, res);
  if (threadIdx.x == 0) {
    hr[2 * BINS + RP_BINS2] = b.key;
    hr[2 * BINS + RP_BINS2 + 1] = b.above;
  }
}

// Pass 4: keys above K and equal to K in each wave's segment of each chunk.
__global__ __launch_bounds__(RP_WAVES * 64) void rp_count_kernel(const float* __restrict__ scores, int32_t n,
                                                                  int32_t forced, const uint32_t* __restrict__ ws,
                                                                  uint32_t* __restrict__ cnt) {
  const int32_t c = blockIdx.x, row = blockIdx.y, nch = gridDim.x;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t c0 = c * RP_CHUNK, m = min(RP_CHUNK, n - c0);
  const uint32_t K = ws[(size_t)row * RP_HIST_WORDS + 2 * BINS + RP_BINS2];
  GlobalSeg seg{scores + (size_t)row * n + c0, forced - c0, 0, 0, 0, lane, c0};
  wave_segment<RP_WAVES>(m, seg.s0, seg.s1, seg.trips);
  uint32_t gt = 0, eq = 0;
  seg.visit([&](int32_t, uint32_t key, bool valid) {
    gt += __popcll(__ballot(valid && key > K));
    eq += __popcll(__ballot(valid && key == K));
  });
  if (lane == 0) {
    uint32_t* cc = cnt + (((size_t)row * nch + c) * RP_WAVES + wave) * 2;
    cc[0] = gt;
    cc[1] = eq;
  }
}

// Pass 5: each chunk's kept entries to the output, ascending.
__global__ __launch_bounds__(RP_WAVES * 64) void rp_write_kernel(const float* __restrict__ scores, int32_t n,
                                                                  int32_t kk, int32_t forced, const uint32_t* __restrict__ ws,
                                                                  const uint32_t* __restrict__ cnt,
                                                                  int32_t* __restrict__ out) {
  constexpr int NT = RP_WAVES * 64;
  __shared__ uint32_t pre[RP_WAVES][2];
  const int32_t c = blockIdx.x, row = blockIdx.y, nch = gridDim.x;
  const int32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t c0 = c * RP_CHUNK, m = min(RP_CHUNK, n - c0);
  const uint32_t* hb = ws + (size_t)row * RP_HIST_WORDS + 2 * BINS + RP_BINS2;
  const uint32_t K = hb[0], need = (uint32_t)kk - hb[1];
  // keys above K (G) and equal to K (E) in the earlier chunks, and in this
  // chunk's earlier waves
  const uint32_t* cr = cnt + (size_t)row * nch * RP_WAVES * 2;
  uint32_t g = 0, e = 0;
  for (int32_t j = tid; j < c * RP_WAVES; j += NT) { g += cr[2 * j]; e += cr[2 * j + 1]; }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) { g += __shfl_xor(g, d); e += __shfl_xor(e, d); }
  if (lane == 0) { pre[wave][0] = g; pre[wave][1] = e; }
  __syncthreads();
  uint32_t G = 0, E = 0, gt_before = 0, eq_before = 0;
  for (int v = 0; v < RP_WAVES; ++v) { G += pre[v][0]; E += pre[v][1]; }
  for (int v = 0; v < wave; ++v) {
    gt_before += cr[2 * (c * RP_WAVES + v)];
    eq_before += cr[2 * (c * RP_WAVES + v) + 1];
  }
  GlobalSeg seg{scores + (size_t)row * n + c0, forced - c0, 0, 0, 0, lane, c0};
  wave_segment<RP_WAVES>(m, seg.s0, seg.s1, seg.trips);
  uint32_t eq_seen = E + eq_before;  // keys equal to K before this wave's segment
  uint32_t pos = G + min(need, E) + gt_before + min(need - min(need, E), eq_before);
  int32_t* o = out + (size_t)row * kk;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  seg.visit([&](int32_t j, uint32_t key, bool valid) {
    const bool is_eq = valid && key == K;
    const uint64_t eq_mask = __ballot(is_eq);
    const uint32_t eq_rank = eq_seen + __popcll(eq_mask & lt_mask);
    const bool keep = valid && (key > K || (is_eq && eq_rank < need));
    const uint64_t keep_mask = __ballot(keep);
    const uint32_t slot = pos + __popcll(keep_mask & lt_mask);
    if (keep && slot < (uint32_t)kk) o[slot] = seg.index(j);
    pos += __popcll(keep_mask);
    eq_seen += __popcll(eq_mask);
  });
}


// One work-group per (row, query block a): top min(topk, a+1) of
// logits[row][a][0..a] with entry a forced, by the two-read select (the
// row stays in cache between the reads), else by the radix select.
constexpr int BLK_WAVES = 4;
union BlockTopkShared {
  BinShared<BLK_WAVES, 1024, 1024, false> f;
  SelectShared<BLK_WAVES, 2> r;
};

__global__ __launch_bounds__(BLK_WAVES * 64) void block_topk_kernel(const float* __restrict__ logits,
                                                                    int32_t nb, int32_t topk,
                                                                    int32_t* __restrict__ sel,
                                                                    int32_t* __restrict__ n_sel) {
  __shared__ BlockTopkShared sh;
  constexpr int NT = BLK_WAVES * 64;
  const int32_t a = blockIdx.x, row = blockIdx.y;
  const int32_t m = a + 1;
  const int32_t kk = min(topk, m);
  const int32_t kstride = min(topk, nb);
  const size_t cb = (size_t)row * nb + a;
  int32_t* o = sel + cb * kstride;
  if (threadIdx.x == 0) n_sel[cb] = kk;
  if (kk >= m) {
    for (int32_t i = threadIdx.x; i < m; i += NT) o[i] = i;
    return;
  }
  const float* x = logits + cb * nb;
  auto raw_at = [&](int32_t i) { return __float_as_uint(x[i]); };
  auto key_of = [&](int32_t i, uint32_t r) { return i == a ? FORCED_KEY : score_key(__uint_as_float(r)); };
  auto idx_at = [](int32_t i) { return i; };
  if (select_bins<BLK_WAVES>(raw_at, key_of, idx_at, m, kk, o, (uint32_t*)nullptr, sh.f)) return;
  GlobalSeg seg{x, a, 0, 0, 0, (int32_t)(threadIdx.x & 63), 0};
  wave_segment<BLK_WAVES>(m, seg.s0, seg.s1, seg.trips);
  select_topk<BLK_WAVES, 2>(seg, kk, o, nullptr, sh.r);
}

}  // namespace

size_t topk_workspace_bytes(int32_t rows, int32_t n, int32_t k) {
  const int32_t kk = k < n ? k : n;
  if (rows <= 0 || !row_parallel(n, kk)) return 0;
  return rp_bytes(rows, rp_chunks(n));
}

hipError_t launch_topk_rows(const float* scores, int32_t rows, int32_t n, int32_t k,
                            int32_t forced, int32_t* out, void* ws, hipStream_t s) {
  const int32_t kk = k < n ? k : n;
  if (rows == 0 || kk == 0) return hipSuccess;
  if (row_parallel(n, kk)) {
    const int32_t nch = rp_chunks(n);
    uint32_t* hist = static_cast<uint32_t*>(ws);
    uint32_t* cnt = hist + (size_t)rows * RP_HIST_WORDS;
    const size_t words = (size_t)rows * RP_HIST_WORDS;
    const dim3 grid(nch, rows), block(RP_WAVES * 64);
    hipLaunchKernelGGL(rp_zero_kernel, dim3((unsigned)std::min<size_t>((words + 255) / 256, 1024)), dim3(256), 0, s,
                       hist, words);
    hipLaunchKernelGGL(rp_hist_kernel<0>, grid, block, 0, s, scores, n, kk, forced, hist);
    hipLaunchKernelGGL(rp_hist_kernel<1>, grid, block, 0, s, scores, n, kk, forced, hist);
    hipLaunchKernelGGL(rp_hist_kernel<2>, grid, block, 0, s, scores, n, kk, forced, hist);
    hipLaunchKernelGGL(rp_bound_kernel, dim3(rows), block, 0, s, kk, hist);
    hipLaunchKernelGGL(rp_count_kernel, grid, block, 0, s, scores, n, forced, hist, cnt);
    hipLaunchKernelGGL(rp_write_kernel, grid, block, 0, s, scores, n, kk, forced, hist, cnt, out);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(ROW_WAVES * 64), 0, s, scores, n, kk, forced, out);
  return hipGetLastError();
}

hipError_t launch_block_topk(const float* logits, int32_t rows, int32_t nb, int32_t topk,
                             int32_t* sel, int32_t* n_sel, hipStream_t s) {
  if (rows == 0 || nb == 0) return hipSuccess;
  hipLaunchKernelGGL(block_topk_kernel, dim3(nb, rows), dim3(BLK_WAVES * 64), 0, s, logits, nb,
                     topk, sel, n_sel);
  return hipGetLastError();
}

}  // namespace dsa
