// Vertical-slash score estimate, gfx950.
//
// For one query head and its kv head, with the window rows i_r = n - lq + r
// (r < lq = min(last_q, n)) and p[r][j] the causal softmax of row i_r:
//   v[j] = sum_r p[r][j]            (vertical / column scores)
//   s[d] = sum_r p[r][i_r - d]      (slash / diagonal scores)
// [MInference 1.0 article, §2.2 Vertical-Slash Head: the last queries times
// all keys give the estimated attention; Novita blog, §2 Modificación de
// Atención: rowmax and l of a first pass turn a second pass into softmax
// probabilities, restricted to the window's query rows.]
//
// Pass 1 (stats): per (row, chunk of a.chunk keys) one wave computes
//   S = Q_window K_chunk^T with MFMA (lane = one key column, 16 query rows) and
//   keeps a running (max, sum) per query row; partials go to workspace.
// Combine: per row, max / log-sum over the chunks -> F_r = m_r + log2 Z_r.
// Work-groups of both passes are mapped like the attention's: the heads of a
// kv group take the same key chunk on the same XCD at about the same time, so
// a chunk of K is fetched from memory once per group.
// Pass 2 (scores): recompute S, p = exp2(S*scale*log2e - F_r). Column sums are
//   register sums plus two cross-lane steps (the loop runs key-major, so a
//   key's scores stay in one lane column). Diagonal sums: per 32-key half
//   tile, each p goes to LDS at the row of its diagonal (a skewed tile whose
//   unused slots stay zero), each lane adds up whole rows, and a diagonal
//   still open at the half tile's end moves on to the lane that owns it in
//   the next one: no atomics, fixed order, bit-reproducible.
// S-combine: s[d] adds the (at most two) chunk partials covering offset d in
//   ascending chunk order.
#include "kernels.hpp"

namespace dsa {
namespace {

// Skewed probability tile of one 32-key half tile (64 window rows x 32 keys):
// element (r, c) sits at row r - c + 31 (its diagonal), column c. Rows 0..94
// hold the 95 diagonals, row 95 stays zero. Row stride 34 floats: the 64-bit
// row reads are free of bank conflicts, and the whole tile (13 KB) leaves
// room for three one-wave work-groups per SIMD.
constexpr int DG_ROWS = 96, DG_STRIDE = 34;
constexpr int WIN_WAVES = 4;              // window slices per work-group (column-score windows)

__device__ __forceinline__ int32_t wave_lane() { return (int32_t)(threadIdx.x & 63); }

struct Window {
  int32_t n, lq, start;
  __device__ int32_t pos(int32_t r) const { return start + r; }  // sequence row of window row r
};

// S tile for 16 keys [j0, j0+16): lane holds key column j0 + l16 and window
// rows 16qb + 4g + i. Returns the unscaled scores, -inf where masked; the
// consumers fold scale * log2(e) into one FMA per element.
template <typename T, int D>
struct Tile;

template <int D>
struct Tile<uint16_t, D> {
  static constexpr int DS = D / 32;
  u32x4 qop[4][DS];
  __device__ void load_q(const uint16_t* qs, const Window& w) {
    const int32_t lane = wave_lane(), g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      int32_t r = min(16 * qb + l16, w.lq - 1);
      const u32x4* src = reinterpret_cast<const u32x4*>(qs + (size_t)w.pos(r) * D + (D / 4) * g);
#pragma unroll
      for (int s = 0; s < DS; ++s) qop[qb][s] = src[s];
    }
  }
  // K operands of the 16 keys from j0 (clamped into [0, n): a load past the
  // end reads the last key, and its scores are never used)
  struct KReg { u32x4 v[DS]; };
  __device__ void load_k(const uint16_t* ks, int32_t j0, const Window& w, KReg& k) const {
    const int32_t lane = wave_lane(), g = lane >> 4, l16 = lane & 15;
    const int32_t key = min(j0 + l16, w.n - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(ks + (size_t)key * D + (D / 4) * g);
#pragma unroll
    for (int s = 0; s < DS; ++s) k.v[s] = src[s];
  }
  // unmasked scores: the MFMAs alone
  __device__ void scores_raw(const KReg& k, f32x4 (&out)[4]) const {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s) acc = mfma_bf16(qop[qb][s], k.v[s], acc);
      out[qb] = acc;
    }
  }
  __device__ void scores_k(const KReg& k, int32_t j0, const Window& w, f32x4 (&out)[4]) const {
    scores_raw(k, out);
    finish(out, j0, wave_lane() & 15, w);
  }
  // mask only a step that reaches the window's first row (or a window of
  // fewer than 64 rows): earlier keys precede every window row
  __device__ static void finish(f32x4 (&x)[4], int32_t j0, int32_t l16, const Window& w) {
    if (!(j0 + 15 <= w.start && w.lq == 64)) mask(x, j0 + l16, w);
  }
  // row r = 16 qb + 4 g + i is kept when r < lq and key <= start + r, i.e.
  // when lo <= 16 qb + i < hi for the lane values below (no per-row registers)
  __device__ static void mask(f32x4 (&x)[4], int32_t key, const Window& w) {
    const int32_t g4 = 4 * (wave_lane() >> 4);
    const int32_t lo = key - w.start - g4, hi = w.lq - g4;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = 16 * qb + i >= lo && 16 * qb + i < hi;
        x[qb][i] = ok ? x[qb][i] : -INFINITY;
      }
  }
};

template <int D>
struct Tile<float, D> {
  static constexpr int DK = D / 4;
  float qop[4][DK];
  __device__ void load_q(const float* qs, const Window& w) {
    const int32_t lane = wave_lane(), g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      int32_t r = min(16 * qb + l16, w.lq - 1);
      const f32x4* src = reinterpret_cast<const f32x4*>(qs + (size_t)w.pos(r) * D + DK * g);
#pragma unroll
      for (int s = 0; s < DK / 4; ++s) {
        f32x4 x = src[s];
        qop[qb][4 * s] = x[0]; qop[qb][4 * s + 1] = x[1]; qop[qb][4 * s + 2] = x[2]; qop[qb][4 * s + 3] = x[3];
      }
    }
  }
  struct KReg { f32x4 v[DK / 4]; };
  __device__ void load_k(const float* ks, int32_t j0, const Window& w, KReg& k) const {
    const int32_t lane = wave_lane(), g = lane >> 4, l16 = lane & 15;
    const int32_t key = min(j0 + l16, w.n - 1);
    const f32x4* src = reinterpret_cast<const f32x4*>(ks + (size_t)key * D + DK * g);
#pragma unroll
    for (int s = 0; s < DK / 4; ++s) k.v[s] = src[s];
  }
  __device__ void scores_k(const KReg& k, int32_t j0, const Window& w, f32x4 (&out)[4]) const {
    const int32_t l16 = wave_lane() & 15;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DK; ++s) acc = mfma_f32(qop[qb][s], k.v[s / 4][s % 4], acc);
      out[qb] = acc;
    }
    Tile<uint16_t, D>::finish(out, j0, l16, w);
  }
};

// Scores of consecutive 16-key steps. bf16 loads the next step's K while the
// current one computes (16 more VGPRs, still three waves per SIMD); fp32,
// whose K operands are twice as wide, loads each step's K at its start.
template <typename T, int D, bool PF = sizeof(T) == 2>
struct KStream {
  static constexpr bool PREFETCH = PF;
  typename Tile<T, D>::KReg kn;
  __device__ KStream(const Tile<T, D>& tile, const T* ks, int32_t j_begin, const Window& w) {
    if (PREFETCH) tile.load_k(ks, j_begin, w, kn);
  }
  __device__ void scores(const Tile<T, D>& tile, const T* ks, int32_t j0, const Window& w, f32x4 (&x)[4]) {
    if (PREFETCH) {
      const typename Tile<T, D>::KReg kc = kn;
      tile.load_k(ks, j0 + 16, w, kn);
      tile.scores_k(kc, j0, w, x);
    } else {
      tile.load_k(ks, j0, w, kn);
      tile.scores_k(kn, j0, w, x);
    }
  }
};

// bf16 K of 16-key steps through a ring of NS steps in LDS: each step goes
// global -> LDS by DMA (buffer_load ... lds, no registers) NS - 1 steps
// before it is used, into its own stage array (4 KB per step at D = 128).
// Rows are stored with the swizzle the attention tiles use, so the K operand
// reads are free of bank conflicts. Rows past the head's slab read as zeros
// (buffer range check); their scores are masked. One-wave work-groups take
// three stages (12 KB per wave: three waves per SIMD stay resident).
constexpr int KR_STAGES = 3;
// The window column-sum work-groups (four waves, each with its own ring and
// the chunk's per-slice column sums) take two stages: 48 KB of LDS instead
// of 64 KB, so three work-groups per CU, three waves per SIMD.
constexpr int WIN_RING_STAGES = 2;
template <int D, int NS = KR_STAGES>
struct KRing {
  static constexpr int ROW = D * 2;          // bytes per key
  static constexpr int UNITS = ROW / 16;     // 16-byte chunks per key
  static constexpr int STEP = 16 * ROW;      // bytes per 16-key step
  static constexpr int INSTR = STEP / 1024;  // DMA instructions per step
  static constexpr int RPI = 64 / UNITS;     // key rows per DMA instruction
  static constexpr int DS = D / 32;
  __amdgpu_buffer_rsrc_t rs;
  int32_t ld_off[INSTR];  // byte offset of this lane's 16 bytes within a step
  int32_t koff[DS];       // LDS offset of this lane's K operand of k-step s
  __device__ KRing(const uint16_t* ks, int32_t n) {
    const int32_t lane = wave_lane(), g = lane >> 4, l16 = lane & 15;
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)ks, (short)0, (uint32_t)n * ROW, 0x00020000);
#pragma unroll
    for (int k = 0; k < INSTR; ++k) {
      const int32_t r = k * RPI + lane / UNITS;
      ld_off[k] = r * ROW + 16 * ((lane % UNITS) ^ (lds_chunk_swz(r) & (UNITS - 1)));
    }
#pragma unroll
    for (int s = 0; s < DS; ++s) koff[s] = l16 * ROW + 16 * (((D / 32) * g + s) ^ (lds_chunk_swz(l16) & (UNITS - 1)));
  }
  // keys [j0, j0 + 16) into stage: lane L of instruction k lands at byte
  // k * 1024 + 16 L, i.e. row k * RPI + L / UNITS, chunk slot L % UNITS
  __device__ void issue(int32_t j0, char* stage) const {
#pragma unroll
    for (int k = 0; k < INSTR; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(stage + k * 1024), 16,
                                               j0 * ROW + ld_off[k], 0, 0, 0);
  }
  // Waits until this lane's DMA of the current step (issued NS - 1 steps
  // back) has landed, then reads the K operands. Every step issues
  // exactly INSTR DMA loads, so at least INSTR * (NS - 1) vector
  // memory operations follow the current step's; loads completing in order,
  // vmcnt of that count suffices (other loads and stores issued in between
  // only make it stricter).
  // The reads are one asm block that waits for its own results: the compiler
  // cannot tell which stage an LDS DMA writes, and would otherwise drain
  // every load in flight before each read.
  __device__ void read(const char* stage, typename Tile<uint16_t, D>::KReg& k) const {
    constexpr int ahead = INSTR * (NS - 1);  // DMA loads issued after this step's
    static_assert(ahead < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | ahead);     // vmcnt(ahead), no expcnt / lgkmcnt wait
    // the stage's LDS byte address (an address-space cast of the pointer)
    const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)stage;
    if constexpr (DS == 4) {
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %1, %5\n\t"
          "ds_read_b128 %2, %6\n\t"
          "ds_read_b128 %3, %7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k.v[0]), "=&v"(k.v[1]), "=&v"(k.v[2]), "=&v"(k.v[3])
          : "v"(base + koff[0]), "v"(base + koff[1]), "v"(base + koff[2]), "v"(base + koff[3])
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %2\n\t"
          "ds_read_b128 %1, %3\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(k.v[0]), "=&v"(k.v[1])
          : "v"(base + koff[0]), "v"(base + koff[1])
          : "memory");
    }
  }
};

// bf16: three waves per SIMD, so the prefetched K costs no occupancy.
// MULTI: a work-group of up to WIN_WAVES waves, wave t taking window slice t
// (64 rows from a.win_start + 64 t) over the same key chunk; each wave streams
// K through its own ring, so the work-group's waves fetch each K line once
// from memory and the other times from cache.
#define EST_KERNEL_1 \
  __global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 1, sizeof(T) == 2 ? 3 : 8)))
#define EST_WIN_KERNEL \
  __global__ __launch_bounds__(64 * WIN_WAVES) __attribute__((amdgpu_waves_per_eu(3, 3)))

// The wave's window: the launch's (one wave) or its 64-row slice (MULTI)
template <bool MULTI>
__device__ __forceinline__ Window wave_window(const EstArgs& a, int32_t slice) {
  if (!MULTI) return Window{a.seq_len, a.lq_eff(), a.win_start};
  const int32_t start = a.win_start + 64 * slice;
  return Window{a.seq_len, min(64, a.seq_len - start), start};
}

template <typename T, int D, bool MULTI>
__device__ __forceinline__ void est_stats(const EstArgs& a) {
  const int32_t C = a.chunk, nchunks = (a.seq_len + C - 1) / C;
  int32_t row, chunk;
  work_item(a.hm, a.wo, nchunks, row, chunk);
  const int32_t slice = MULTI ? __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6)) : 0;
  const int32_t nsl = MULTI ? (int32_t)(blockDim.x >> 6) : 1;
  const Window w = wave_window<MULTI>(a, slice);
  const T* qs = static_cast<const T*>(a.q) + a.hm.q_slab(row, a.seq_len, D);
  const T* ks = static_cast<const T*>(a.k) + a.hm.kv_slab(row, a.seq_len, D);
  Tile<T, D> tile;
  tile.load_q(qs, w);
  float m[4][4], z[4][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) { m[qb][i] = NEG_BIG; z[qb][i] = 0.f; }

  const int32_t j_begin = chunk * C, j_end = min(a.seq_len, j_begin + C);
  const float sc = a.scale_log2;
  // running (max, sum) with a deferred max, one step in two parts. pre:
  // d = x * scale * log2(e) - m in one FMA, and the reference m raised only
  // where d exceeds 8 (then d = 0); one compare per step, the largest d
  // against the margin (a v_max3 tree). post: the sums take 2^d.
  auto pre = [&](const f32x4 (&x)[4], f32x4 (&d)[4]) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) d[qb][i] = __builtin_fmaf(x[qb][i], sc, -m[qb][i]);
    const float dm = fmaxf(fmaxf(fmaxf(fmaxf(d[0][0], d[0][1]), fmaxf(d[0][2], d[0][3])),
                                 fmaxf(fmaxf(d[1][0], d[1][1]), fmaxf(d[1][2], d[1][3]))),
                           fmaxf(fmaxf(fmaxf(d[2][0], d[2][1]), fmaxf(d[2][2], d[2][3])),
                                 fmaxf(fmaxf(d[3][0], d[3][1]), fmaxf(d[3][2], d[3][3]))));
    if (__any(dm > 8.f)) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (d[qb][i] > 8.f) {
            const float xs = x[qb][i] * sc;
            z[qb][i] *= fast_exp2(m[qb][i] - xs);
            m[qb][i] = xs;
            d[qb][i] = 0.f;
          }
    }
  };
  auto post = [&](const f32x4 (&d)[4]) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) z[qb][i] += fast_exp2(d[qb][i]);
  };
  if constexpr (sizeof(T) == 2) {
    constexpr int NW = MULTI ? WIN_WAVES : 1;
    __shared__ __align__(16) char kr0[NW][KRing<D>::STEP], kr1[NW][KRing<D>::STEP], kr2[NW][KRing<D>::STEP];
    char* const stage[KR_STAGES] = {kr0[slice], kr1[slice], kr2[slice]};
    const KRing<D> ring(ks, a.seq_len);
    // every step issues its INSTR loads, past the chunk's end too (rows of
    // the next chunk, or zeros past the slab, into stages never read), so
    // that the wait count in ring.read is exact
    // One step of lag: the sums of step t take their 2^d in the same basic
    // block as the MFMAs of step t + 1, interleaved with them, so that the
    // exponentials issue while the matrix core works. The lagged d starts
    // at -inf, which adds exact zeros; the order of the updates is that of
    // the steps.
    f32x4 dp[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) dp[qb] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const int32_t l16 = wave_lane() & 15;
#pragma unroll
    for (int u = 0; u < KR_STAGES - 1; ++u) ring.issue(j_begin + 16 * u, stage[u]);
    for (int32_t t0 = j_begin; t0 < j_end; t0 += 16 * KR_STAGES) {
#pragma unroll
      for (int u = 0; u < KR_STAGES; ++u) {
        const int32_t j0 = t0 + 16 * u;
        // the stage of step u - 1 is consumed: refill it with step u + KR_STAGES - 1
        ring.issue(j0 + 16 * (KR_STAGES - 1), stage[(u + KR_STAGES - 1) % KR_STAGES]);
        if (j0 < j_end) {
          typename Tile<T, D>::KReg kc;
          ring.read(stage[u], kc);
          f32x4 x[4];
          tile.scores_raw(kc, x);
          post(dp);
#pragma unroll
          for (int r = 0; r < 4 * Tile<T, D>::DS; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two VALU
          }
          // the sums are formed here, in the MFMAs' block (not sunk past the
          // mask's branch)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb) asm volatile("" ::"v"(z[qb][0]), "v"(z[qb][1]), "v"(z[qb][2]), "v"(z[qb][3]));
          Tile<T, D>::finish(x, j0, l16, w);
          pre(x, dp);
        }
      }
    }
    post(dp);
    __builtin_amdgcn_s_waitcnt(0);  // no DMA into LDS outlives the loop
  } else {
    KStream<T, D> kst(tile, ks, j_begin, w);
    for (int32_t j0 = j_begin; j0 < j_end; j0 += 16) {
      f32x4 x[4], d[4];
      kst.scores(tile, ks, j0, w, x);
      pre(x, d);
      post(d);
    }
  }
  // merge the 16 key columns of each row (lanes with equal l >> 4)
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mm = m[qb][i], zz = z[qb][i];
#pragma unroll
      for (int msk = 1; msk < 16; msk <<= 1) {
        float mo = __shfl_xor(mm, msk, 64), zo = __shfl_xor(zz, msk, 64);
        float mn = fmaxf(mm, mo);
        zz = zz * fast_exp2(mm - mn) + zo * fast_exp2(mo - mn);
        mm = mn;
      }
      m[qb][i] = mm;
      z[qb][i] = zz;
    }
  const int32_t lane = wave_lane(), g = lane >> 4;
  if ((lane & 15) == 0) {
    float* dst = a.part_stats + ((size_t)(row * nsl + slice) * nchunks + chunk) * 64 * 2;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int r = 16 * qb + 4 * g + i;
        dst[2 * r] = m[qb][i];
        dst[2 * r + 1] = z[qb][i];
      }
  }
}

template <typename T, int D>
EST_KERNEL_1 void est_stats_kernel(EstArgs a) { est_stats<T, D, false>(a); }
template <int D>
EST_WIN_KERNEL void est_window_stats_kernel(EstArgs a) { est_stats<uint16_t, D, true>(a); }

// F_r = m_r + log2(Z_r) over all chunks. One work-group per row: thread t
// merges window row t % 64 over the chunks c = t / 64 (mod COMB_SPLIT) with a
// running (max, sum), then the COMB_SPLIT partials of each window row meet in
// LDS in a fixed order.
constexpr int COMB_SPLIT = 16;
__global__ __launch_bounds__(64 * COMB_SPLIT) void est_combine_kernel(EstArgs a, int32_t nchunks) {
  __shared__ float pm[COMB_SPLIT][64], pz[COMB_SPLIT][64];
  const int32_t row = blockIdx.x, r = threadIdx.x & 63, part = threadIdx.x >> 6;
  const float* src = a.part_stats + (size_t)row * nchunks * 128 + 2 * r;
  float mm = NEG_BIG, zz = 0.f;
  // eight chunks' loads in flight, then their merge in chunk order
  constexpr int B = 8;
  for (int32_t c0 = part; c0 < nchunks; c0 += B * COMB_SPLIT) {
    float mc[B], zc[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int32_t c = c0 + u * COMB_SPLIT;
      const bool ok = c < nchunks;
      mc[u] = ok ? src[(size_t)c * 128] : NEG_BIG;
      zc[u] = ok ? src[(size_t)c * 128 + 1] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (c0 + u * COMB_SPLIT >= nchunks) break;
      const float mn = fmaxf(mm, mc[u]);
      zz = zz * fast_exp2(mm - mn) + zc[u] * fast_exp2(mc[u] - mn);
      mm = mn;
    }
  }
  pm[part][r] = mm;
  pz[part][r] = zz;
  __syncthreads();
  if (part == 0) {
    float m2 = NEG_BIG;
#pragma unroll
    for (int t = 0; t < COMB_SPLIT; ++t) m2 = fmaxf(m2, pm[t][r]);
    float z2 = 0.f;
#pragma unroll
    for (int t = 0; t < COMB_SPLIT; ++t) z2 += pz[t][r] * fast_exp2(pm[t][r] - m2);
    a.row_stats[(size_t)row * 64 + r] = z2 > 0.f ? m2 + __log2f(z2) : INFINITY;
  }
}

// Column sums of one chunk (no slash scores) with K through the LDS ring as
// in the stats pass; the column-sum stores between the loads only make the
// ring's fixed wait count conservative. MULTI: each wave sums its window
// slice into LDS, and after the chunk the work-group adds the slices in slice
// order (a fixed order: the same bits on every run).
template <int D, bool MULTI>
__device__ void ring_column_sums(const EstArgs& a, const Tile<uint16_t, D>& tile, const uint16_t* ks,
                                 const Window& w, const float (&F)[4][4], float* vout, int32_t j_begin,
                                 int32_t j_end, int32_t slice, int32_t nsl) {
  using T = uint16_t;
  const int32_t g = wave_lane() >> 4, l16 = wave_lane() & 15;
  const float sc = a.scale_log2;
  constexpr int NW = MULTI ? WIN_WAVES : 1;
  constexpr int NS = MULTI ? WIN_RING_STAGES : KR_STAGES;
  constexpr int STEP = KRing<D, NS>::STEP;
  __shared__ __align__(16) char kr0[NW][STEP], kr1[NW][STEP], kr2[NS > 2 ? NW : 1][NS > 2 ? STEP : 16];
  __shared__ float cs[NW][MULTI ? EST_CHUNK : 1];
  char* const stage[3] = {kr0[slice], kr1[slice], kr2[NS > 2 ? slice : 0]};
  const KRing<D, NS> ring(ks, a.seq_len);
  // (one wave) the window slices after the first add into v: each step's
  // earlier v is loaded together with its K, so that waiting for it never
  // drains the loads issued after it
  const bool add_here = !MULTI && a.add_v;
  float vprev[NS];
  auto load_v = [&](int32_t j0) { return vout[min(j0 + l16, a.seq_len - 1)]; };
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) {
    vprev[u] = add_here ? load_v(j_begin + 16 * u) : 0.f;
    ring.issue(j_begin + 16 * u, stage[u]);
  }
  for (int32_t t0 = j_begin; t0 < j_end; t0 += 16 * NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int32_t j0 = t0 + 16 * u, jn = j0 + 16 * (NS - 1);
      const int un = (u + NS - 1) % NS;  // constant after unrolling
      vprev[un] = add_here ? load_v(jn) : 0.f;
      ring.issue(jn, stage[un]);
      if (j0 < j_end) {
        typename Tile<T, D>::KReg kc;
        ring.read(stage[u], kc);
        f32x4 x[4];
        tile.scores_k(kc, j0, w, x);
        float colsum = 0.f;
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) colsum += fast_exp2(__builtin_fmaf(x[qb][i], sc, -F[qb][i]));
        colsum = xor_sum(xor_sum(colsum, 16), 32);
        if (MULTI) {
          if (g == 0) cs[slice][j0 - j_begin + l16] = colsum;
        } else if (g == 0 && j0 + l16 < a.seq_len) {
          vout[j0 + l16] = add_here ? vprev[u] + colsum : colsum;
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA into LDS outlives the loop
  if constexpr (MULTI) {
    __syncthreads();
    for (int32_t jj = (int32_t)threadIdx.x; jj < j_end - j_begin; jj += 64 * nsl) {
      float sum = 0.f;
      for (int32_t t = 0; t < nsl; ++t) sum += cs[t][jj];
      float* dst = vout + j_begin + jj;
      *dst = a.add_v ? *dst + sum : sum;
    }
  }
}

// S: slash scores wanted (a.want_s); without them the probabilities never
// go through LDS
template <typename T, int D, bool S, bool MULTI>
__device__ __forceinline__ void est_scores(const EstArgs& a) {
  static_assert(!(MULTI && S), "window slices: column scores only");
  static_assert(!MULTI || sizeof(T) == 2, "window slices: bf16 only");
  __shared__ __align__(16) float dtile[S ? DG_ROWS * DG_STRIDE : 1];
  const int32_t C = a.chunk, nchunks = (a.seq_len + C - 1) / C;
  int32_t row, chunk;
  work_item(a.hm, a.wo, nchunks, row, chunk);
  const int32_t slice = MULTI ? __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6)) : 0;
  const int32_t nsl = MULTI ? (int32_t)(blockDim.x >> 6) : 1;
  const int32_t lane = wave_lane(), g = lane >> 4, l16 = lane & 15;
  const Window w = wave_window<MULTI>(a, slice);
  const T* qs = static_cast<const T*>(a.q) + a.hm.q_slab(row, a.seq_len, D);
  const T* ks = static_cast<const T*>(a.k) + a.hm.kv_slab(row, a.seq_len, D);
  Tile<T, D> tile;
  tile.load_q(qs, w);
  float F[4][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) F[qb][i] = a.row_stats[(size_t)(row * nsl + slice) * 64 + 16 * qb + 4 * g + i];

  float* vout = a.v_scores + (size_t)row * a.seq_len;
  const float sc = a.scale_log2;
  const int32_t j_begin = chunk * C, j_end = min(a.seq_len, j_begin + C);
  if constexpr (sizeof(T) == 2 && !S) {
    ring_column_sums<D, MULTI>(a, tile, ks, w, F, vout, j_begin, j_end, slice, nsl);
    return;
  }
  // The chunk's partial diagonal sums: entry (C - 1) - (J - j_begin) + e holds
  // the diagonal with r - c = e in the half tile starting at key J, i.e. the
  // entry of (window row r, key j) is r - j + j_begin + C - 1, in [0, C + 63).
  float* const spart = S ? a.s_part + ((size_t)row * nchunks + chunk) * (C + 63) : nullptr;
  // write slot of this lane's (r, c) = (16 qb + 4 g + i, 16 sb + l16): the
  // lane part (4 g - l16 + 15) * DG_STRIDE + l16 (never negative) plus the
  // constant (16 (qb - sb) + i + 16) * DG_STRIDE + 16 sb
  const int32_t wlane = (4 * g - l16 + 15) * DG_STRIDE + l16;
  // lane l sums diagonal e = l - 31 (row l) into da and, for l < 31, diagonal
  // e = l + 33 (row l + 64) into db; the other lanes read the zero row
  const float* const rda = dtile + lane * DG_STRIDE;
  const float* const rdb = dtile + (lane < 31 ? lane + 64 : DG_ROWS - 1) * DG_STRIDE;
  float da = 0.f, db = 0.f;
  if (S) {
    // slots no (r, c) maps to are never written: zero them once
    for (int32_t e = lane; e < DG_ROWS * DG_STRIDE; e += 64) dtile[e] = 0.f;
    __syncthreads();
  }
  KStream<T, D, (sizeof(T) == 2 && !(S && D == 128))> kst(tile, ks, j_begin, w);
  int32_t h0 = j_begin;
  for (; h0 < j_end; h0 += 32) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int32_t j0 = h0 + 16 * sb;
      f32x4 x[4];
      kst.scores(tile, ks, j0, w, x);
      float colsum = 0.f;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(__builtin_fmaf(x[qb][i], sc, -F[qb][i]));
          colsum += p;
          if (S) dtile[wlane + (16 * (qb - sb) + i + 16) * DG_STRIDE + 16 * sb] = p;
        }
      colsum = xor_sum(xor_sum(colsum, 16), 32);
      if (g == 0 && j0 + l16 < a.seq_len) {
        if (a.add_v) vout[j0 + l16] += colsum;
        else vout[j0 + l16] = colsum;
      }
    }
    if (!S) continue;
    __syncthreads();
    float sa[2] = {0.f, 0.f}, sbv[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 32; c += 2) {
      const float2 va = *reinterpret_cast<const float2*>(rda + c);
      const float2 vb = *reinterpret_cast<const float2*>(rdb + c);
      sa[(c >> 1) & 1] += va.x + va.y;
      sbv[(c >> 1) & 1] += vb.x + vb.y;
    }
    da += sa[0] + sa[1];
    db += sbv[0] + sbv[1];
    __syncthreads();
    // diagonals e in [32, 63] end in this half tile: e = l + 33 (lanes < 31)
    // and e = 32 (lane 63, its da)
    const int32_t base = (C - 1) - (h0 - j_begin);
    if (lane < 31) spart[base + lane + 33] = db;
    if (lane == 63) spart[base + 32] = da;
    // e <= 31 continues as e + 32 in the next half tile: lane l's da (e = l - 31)
    // becomes da of lane l + 32 (l < 32) or db of lane l - 32 (l >= 32)
    const float moved = __shfl_xor(da, 32, 64);
    da = lane >= 32 ? moved : 0.f;
    db = lane < 31 ? moved : 0.f;
  }
  if (!S) return;
  // diagonals still open, in the frame of the half tile after the last:
  // da of lanes >= 32 (e = l - 31), db of lanes < 31 (e = l + 33)
  const int32_t base = (C - 1) - (h0 - j_begin);
  if (lane >= 32) spart[base + lane - 31] = da;
  if (lane < 31) spart[base + lane + 33] = db;
  // a short last chunk leaves the entries below base + 1 untouched (no key
  // of this chunk lies on them): zero them, as a full chunk would have
  for (int32_t e = lane; e <= base; e += 64) spart[e] = 0.f;
}

template <typename T, int D, bool S>
EST_KERNEL_1 void est_scores_kernel(EstArgs a) { est_scores<T, D, S, false>(a); }
template <int D>
EST_WIN_KERNEL void est_window_scores_kernel(EstArgs a) { est_scores<uint16_t, D, false, true>(a); }

// s[d] = sum over chunks c covering d (ascending c) of s_part[c][e_c(d)],
// e_c(d) = d - (start - (c*C + C - 1)), start = the window's first row.
__global__ __launch_bounds__(256) void est_scombine_kernel(EstArgs a, int32_t nchunks) {
  const int32_t row = blockIdx.y;
  const int32_t d = blockIdx.x * 256 + threadIdx.x;
  if (d >= a.seq_len) return;
  const int32_t n = a.seq_len, lq = a.lq_eff(), start = a.win_start, C = a.chunk, SACC = C + 63;
  const int32_t cs = __builtin_ctz((uint32_t)C);  // the chunk is a power of two
  // keys of diagonal d: j in [start - d, start + lq - 1 - d] (clipped at 0)
  const int32_t j_lo = max(0, start - d), j_hi = start + lq - 1 - d;
  // a diagonal spans lq <= 64 <= C keys: at most two chunks, both loaded
  // before the add (in chunk order, as always)
  const float* sp = a.s_part + (size_t)row * nchunks * SACC;
  const int32_t c0 = j_lo >> cs, c1 = j_hi >> cs;
  float sum = 0.f;
  if (c0 <= c1) {
    const float x0 = sp[(size_t)c0 * SACC + d - (start - (c0 * C + C - 1))];
    const float x1 = c1 > c0 ? sp[(size_t)c1 * SACC + d - (start - (c1 * C + C - 1))] : 0.f;
    sum = c1 > c0 ? x0 + x1 : x0;
  }
  a.s_scores[(size_t)row * n + d] = sum;
}

}  // namespace

int32_t est_chunk_keys(int32_t seq_len) {
  // The chunk fixes the fp32 summation order of the row statistics and the
  // slash partials, so it depends on seq_len alone: a head's scores are then
  // the same bits whatever batch or head list it is computed with. Long rows
  // take the largest chunk (64+ chunks per row); shorter ones smaller chunks,
  // down to 64 keys, so that a row still spreads over about 64 work-groups.
  if (seq_len >= 65536) return EST_CHUNK;
  if (seq_len >= 32768) return 512;
  if (seq_len >= 16384) return 256;
  if (seq_len >= 8192) return 128;
  return 64;
}

size_t est_workspace_bytes(int32_t rows, int32_t seq_len) {
  if (rows == 0 || seq_len == 0) return 0;  // nothing is launched
  const int32_t C = est_chunk_keys(seq_len);
  const size_t nch = (size_t)(seq_len + C - 1) / C;
  const size_t part = (size_t)rows * nch * 128 * sizeof(float);
  const size_t stats = (size_t)rows * 64 * sizeof(float);
  const size_t spart = (size_t)rows * nch * (C + 63) * sizeof(float);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(part) + al(stats) + al(spart);
}

void est_carve(EstArgs& a, void* ws) {
  a.chunk = est_chunk_keys(a.seq_len);
  const size_t nch = (size_t)(a.seq_len + a.chunk - 1) / a.chunk;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = static_cast<char*>(ws);
  a.part_stats = reinterpret_cast<float*>(p);
  p += al((size_t)a.rows * nch * 128 * sizeof(float));
  a.row_stats = reinterpret_cast<float*>(p);
  p += al((size_t)a.rows * 64 * sizeof(float));
  a.s_part = reinterpret_cast<float*>(p);
}

hipError_t launch_vs_estimate(const EstArgs& a, hipStream_t s) {
  if (a.rows == 0 || a.seq_len == 0) return hipSuccess;
  const int32_t nch = (a.seq_len + a.chunk - 1) / a.chunk;
  const dim3 grid((unsigned)((long long)nch * a.rows));
  const bool bf = a.dtype == BF16, d64 = a.head_dim == 64;
  auto st = bf ? (d64 ? est_stats_kernel<uint16_t, 64> : est_stats_kernel<uint16_t, 128>)
               : (d64 ? est_stats_kernel<float, 64> : est_stats_kernel<float, 128>);
  auto sc = a.want_s ? (bf ? (d64 ? est_scores_kernel<uint16_t, 64, true> : est_scores_kernel<uint16_t, 128, true>)
                           : (d64 ? est_scores_kernel<float, 64, true> : est_scores_kernel<float, 128, true>))
                     : (bf ? (d64 ? est_scores_kernel<uint16_t, 64, false> : est_scores_kernel<uint16_t, 128, false>)
                           : (d64 ? est_scores_kernel<float, 64, false> : est_scores_kernel<float, 128, false>));
  hipLaunchKernelGGL(st, grid, dim3(64), 0, s, a);
  hipLaunchKernelGGL(est_combine_kernel, dim3(a.rows), dim3(64 * COMB_SPLIT), 0, s, a, nch);
  hipLaunchKernelGGL(sc, grid, dim3(64), 0, s, a);
  if (a.want_s)
    hipLaunchKernelGGL(est_scombine_kernel, dim3((a.seq_len + 255) / 256, a.rows), dim3(256), 0, s, a, nch);
  return hipGetLastError();
}

size_t est_window_workspace_bytes(int32_t rows, int32_t seq_len) {
  if (rows == 0 || seq_len == 0) return 0;  // nothing is launched
  const int32_t C = est_chunk_keys(seq_len);
  const size_t nch = (size_t)(seq_len + C - 1) / C;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  // per (row, window slice of a launch): chunk partials and row statistics
  return al((size_t)rows * WIN_WAVES * nch * 128 * sizeof(float)) +
         al((size_t)rows * WIN_WAVES * 64 * sizeof(float));
}

void est_window_carve(EstArgs& a, void* ws) {
  a.chunk = est_chunk_keys(a.seq_len);
  const size_t nch = (size_t)(a.seq_len + a.chunk - 1) / a.chunk;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const uintptr_t p = reinterpret_cast<uintptr_t>(ws);
  a.part_stats = reinterpret_cast<float*>(p);
  a.row_stats = reinterpret_cast<float*>(p + al((size_t)a.rows * WIN_WAVES * nch * 128 * sizeof(float)));
  a.s_part = nullptr;
}

hipError_t launch_window_column_scores(EstArgs a, int32_t window, hipStream_t s) {
  const int32_t n = a.seq_len;
  window = window < n ? window : n;
  if (a.rows == 0 || n == 0 || window <= 0) return hipSuccess;
  a.want_s = 0;
  if (a.dtype != BF16) {
    // fp32: one launch per 64-row slice (the first writes v, the others add)
    for (int32_t r0 = n - window; r0 < n; r0 += 64) {
      a.win_start = r0;
      a.last_q = n - r0 < 64 ? n - r0 : 64;
      a.add_v = r0 > n - window;
      const hipError_t e = launch_vs_estimate(a, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // bf16: up to WIN_WAVES slices per launch, one wave each
  const int32_t nch = (n + a.chunk - 1) / a.chunk;
  const dim3 grid((unsigned)((long long)nch * a.rows));
  const bool d64 = a.head_dim == 64;
  auto st = d64 ? est_window_stats_kernel<64> : est_window_stats_kernel<128>;
  auto sc = d64 ? est_window_scores_kernel<64> : est_window_scores_kernel<128>;
  const int32_t nslices = (window + 63) / 64;
  for (int32_t s0 = 0; s0 < nslices; s0 += WIN_WAVES) {
    const int32_t nsl = nslices - s0 < WIN_WAVES ? nslices - s0 : WIN_WAVES;
    a.win_start = n - window + 64 * s0;
    a.last_q = 64;
    a.add_v = s0 > 0;
    hipLaunchKernelGGL(st, grid, dim3(64 * nsl), 0, s, a);
    hipLaunchKernelGGL(est_combine_kernel, dim3(a.rows * nsl), dim3(64 * COMB_SPLIT), 0, s, a, nch);
    hipLaunchKernelGGL(sc, grid, dim3(64 * nsl), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsa
