// Exact top-k with a fixed tie order, gfx950.
//
// Selects the vertical / slash indices and the key blocks of the sparse
// patterns [MInference 1.0 article, §2.2: top-k vertical lines and slash lines;
// top-k blocks of the pooled block scores]. The rank order is: the forced entry
// first, then larger score, then smaller index; -0.0 ranks as +0.0 and NaN as
// -inf. Output indices are ascending.
//
// Method: scores map to order-preserving 32-bit keys (the forced entry gets
// the maximum key, which no canonical float reaches). A 4-pass MSB-first radix
// select (8 bits per pass, per-wave LDS histograms) finds the k-th largest key
// T and how many entries equal to T must be kept (need_eq). A compaction pass
// then walks the entries in index order, each wave owning one contiguous
// segment: an entry is kept when key > T, or key == T and fewer than need_eq
// equal keys precede it. Ballot prefix counts give each kept entry its output
// slot, so the result comes out ascending with no sort.
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

template <int NW>
struct SelectShared {
  uint32_t hist[NW][256];
  uint32_t tot[256];
  uint32_t wcnt[NW][2];
  uint32_t digit, rem;
};

// Top kk (1 <= kk < m) of the m keys get(i), written ascending to out[0..kk).
template <int NW, class Get>
__device__ void select_topk(const Get& get, int32_t m, int32_t kk, int32_t* __restrict__ out,
                            SelectShared<NW>& sh) {
  const int32_t tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int NT = NW * 64;
  uint32_t prefix = 0, pmask = 0;
  if (tid == 0) sh.rem = (uint32_t)kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < NW * 256; i += NT) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    for (int32_t i = tid; i < m; i += NT) {
      uint32_t key = get(i);
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    for (int b = tid; b < 256; b += NT) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += sh.hist[w][b];
      sh.tot[b] = t;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0, rem = sh.rem;
      int b = 255;
      for (; b > 0; --b) {
        if (cum + sh.tot[b] >= rem) break;
        cum += sh.tot[b];
      }
      sh.digit = (uint32_t)b;
      sh.rem = rem - cum;
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    pmask |= 255u << shift;
  }
  const uint32_t T = prefix;
  const uint32_t need_eq = sh.rem;

  // compaction in index order, wave w owns [w*seg, (w+1)*seg)
  const int32_t seg = ((m + NW * 64 - 1) / (NW * 64)) * 64;
  const int32_t s0 = min(m, wave * seg), s1 = min(m, s0 + seg);
  uint32_t n_gt = 0, n_eq = 0;
  for (int32_t i0 = s0; i0 < s1; i0 += 64) {
    int32_t i = i0 + lane;
    uint32_t key = i < s1 ? get(i) : 0u;
    n_gt += __popcll(__ballot(i < s1 && key > T));
    n_eq += __popcll(__ballot(i < s1 && key == T));
  }
  if (lane == 0) { sh.wcnt[wave][0] = n_gt; sh.wcnt[wave][1] = n_eq; }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) { gt_before += sh.wcnt[w][0]; eq_before += sh.wcnt[w][1]; }
  uint32_t eq_seen = eq_before;
  uint32_t pos = gt_before + min(eq_before, need_eq);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int32_t i0 = s0; i0 < s1; i0 += 64) {
    int32_t i = i0 + lane;
    uint32_t key = i < s1 ? get(i) : 0u;
    bool eq = i < s1 && key == T;
    uint64_t eq_mask = __ballot(eq);
    uint32_t eq_rank = eq_seen + __popcll(eq_mask & lt_mask);
    bool keep = i < s1 && (key > T || (eq && eq_rank < need_eq));
    uint64_t keep_mask = __ballot(keep);
    const uint32_t slot = pos + __popcll(keep_mask & lt_mask);
    if (keep && slot < (uint32_t)kk) out[slot] = i;
    pos += __popcll(keep_mask);
    eq_seen += __popcll(eq_mask);
  }
}

struct GlobalKeys {
  const float* x; int32_t forced;
  __device__ uint32_t operator()(int32_t i) const { return i == forced ? FORCED_KEY : score_key(x[i]); }
};
struct LdsKeys {
  const uint32_t* k;
  __device__ uint32_t operator()(int32_t i) const { return k[i]; }
};

constexpr int ROW_WAVES = 16;
__global__ __launch_bounds__(ROW_WAVES * 64) void topk_rows_kernel(const float* __restrict__ scores,
                                                                   int32_t n, int32_t kk, int32_t forced,
                                                                   int32_t* __restrict__ out) {
  __shared__ SelectShared<ROW_WAVES> sh;
  const int32_t row = blockIdx.x;
  int32_t* o = out + (size_t)row * kk;
  if (kk >= n) {
    for (int32_t i = threadIdx.x; i < n; i += ROW_WAVES * 64) o[i] = i;
    return;
  }
  select_topk<ROW_WAVES>(GlobalKeys{scores + (size_t)row * n, forced}, n, kk, o, sh);
}

// One work-group per (row, query block a): top min(topk, a+1) of
// logits[row][a][0..a] with entry a forced.
constexpr int BLK_WAVES = 4;
constexpr int LDS_KEYS = 16384;
__global__ __launch_bounds__(BLK_WAVES * 64) void block_topk_kernel(const float* __restrict__ logits,
                                                                    int32_t nb, int32_t topk,
                                                                    int32_t* __restrict__ sel,
                                                                    int32_t* __restrict__ n_sel) {
  __shared__ SelectShared<BLK_WAVES> sh;
  __shared__ uint32_t keys[LDS_KEYS];
  const int32_t a = blockIdx.x, row = blockIdx.y;
  const int32_t m = a + 1;
  const int32_t kk = min(topk, m);
  const int32_t kstride = min(topk, nb);
  const size_t cb = (size_t)row * nb + a;
  int32_t* o = sel + cb * kstride;
  if (threadIdx.x == 0) n_sel[cb] = kk;
  if (kk >= m) {
    for (int32_t i = threadIdx.x; i < m; i += BLK_WAVES * 64) o[i] = i;
    return;
  }
  const float* x = logits + cb * nb;
  if (m <= LDS_KEYS) {
    for (int32_t i = threadIdx.x; i < m; i += BLK_WAVES * 64) keys[i] = i == a ? FORCED_KEY : score_key(x[i]);
    __syncthreads();
    select_topk<BLK_WAVES>(LdsKeys{keys}, m, kk, o, sh);
  } else {
    select_topk<BLK_WAVES>(GlobalKeys{x, a}, m, kk, o, sh);
  }
}

}  // namespace

hipError_t launch_topk_rows(const float* scores, int32_t rows, int32_t n, int32_t k,
                            int32_t forced, int32_t* out, hipStream_t s) {
  const int32_t kk = k < n ? k : n;
  if (rows == 0 || kk == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_rows_kernel, dim3(rows), dim3(ROW_WAVES * 64), 0, s, scores, n, kk,
                     forced, out);
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
