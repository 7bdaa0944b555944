// Vertical-slash sparse format, gfx950 [MInference 1.0 article, §2.2
// Vertical-Slash Head: the top vertical and slash indices are converted to a
// sparse format that a block-sparse kernel consumes].
//
// Query block a (rows [64a, 64a+64)) meets slash offset d on the keys
// [64a - d, 64a + 64 - d); offsets whose gap is at most 64 give touching key
// ranges, so the slash offsets of a head are merged once into intervals
// [d_lo, d_hi] (kernel 1), and block a's ranges are
// [max(0, 64a - d_hi), min(n, 64a + 64 - d_lo)) for every interval with
// d_lo < 64a + 64 - computed on the fly by the attention kernel, so no
// per-block range list is stored. Kernel 2 builds each block's column list:
// the verticals below the block's end that no range covers. A vertical j is
// covered iff some interval has d_lo - 64 < 64a - j <= d_hi; the expanded
// intervals (d_lo - 64, d_hi] are disjoint, so a binary search on d_lo finds
// the only candidate.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int IV_THREADS = 256;

__global__ __launch_bounds__(IV_THREADS) void vs_intervals_kernel(const int32_t* __restrict__ S, int32_t ns,
                                                                  int32_t* __restrict__ iv,
                                                                  int32_t* __restrict__ n_iv) {
  __shared__ uint32_t wtot[IV_THREADS / 64];
  __shared__ int32_t base_sh;
  const int32_t row = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t* s = S + (size_t)row * ns;
  int32_t* o = iv + (size_t)row * ns * 2;
  if (tid == 0) base_sh = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int32_t i0 = 0; i0 < ns; i0 += IV_THREADS) {
    __syncthreads();
    const int32_t i = i0 + tid;
    const bool valid = i < ns;
    const int32_t d = valid ? s[i] : 0;
    const bool start = valid && (i == 0 || d - s[i - 1] > BLOCK);
    const bool end = valid && (i == ns - 1 || s[i + 1] - d > BLOCK);
    const uint64_t smask = __ballot(start);
    if (lane == 0) wtot[wave] = (uint32_t)__popcll(smask);
    __syncthreads();
    int32_t before = base_sh;
    for (int w = 0; w < wave; ++w) before += (int32_t)wtot[w];
    const int32_t starts_upto = before + (int32_t)__popcll(smask & lt_mask) + (start ? 1 : 0);
    if (start) o[2 * (starts_upto - 1)] = d;
    if (end) o[2 * (starts_upto - 1) + 1] = d;
    __syncthreads();
    if (tid == 0) {
      int32_t t = 0;
      for (int w = 0; w < IV_THREADS / 64; ++w) t += (int32_t)wtot[w];
      base_sh += t;
    }
  }
  __syncthreads();
  if (tid == 0) n_iv[row] = base_sh;
}

constexpr int COL_WAVES = 4;
constexpr int BLOCKS_PER_WG = 16;
constexpr int IV_LDS_CAP = 4096;  // intervals cached in LDS (32 KiB)

__device__ __forceinline__ bool covered(const int32_t* ivp, int32_t cnt, int32_t delta) {
  // largest t with d_lo[t] - 64 < delta
  int32_t lo = 0, hi = cnt;  // answer in [lo, hi) -> t = lo - 1 after search
  while (lo < hi) {
    int32_t mid = (lo + hi) >> 1;
    if (ivp[2 * mid] - BLOCK < delta) lo = mid + 1; else hi = mid;
  }
  return lo > 0 && delta <= ivp[2 * (lo - 1) + 1];
}

__global__ __launch_bounds__(COL_WAVES * 64) void vs_cols_kernel(
    const int32_t* __restrict__ V, int32_t nv, const int32_t* __restrict__ iv,
    const int32_t* __restrict__ n_iv, int32_t max_iv, int32_t n, int32_t nb,
    int32_t* __restrict__ cols, int32_t* __restrict__ n_cols) {
  __shared__ int32_t liv[2 * IV_LDS_CAP];
  const int32_t row = blockIdx.y, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t cnt = n_iv[row];
  const int32_t* giv = iv + (size_t)row * max_iv * 2;
  const bool use_lds = cnt <= IV_LDS_CAP;
  if (use_lds)
    for (int32_t i = tid; i < 2 * cnt; i += COL_WAVES * 64) liv[i] = giv[i];
  __syncthreads();
  const int32_t* ivp = use_lds ? liv : giv;
  const int32_t* vrow = V + (size_t)row * nv;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int32_t a_end = min(nb, (int32_t)(blockIdx.x + 1) * BLOCKS_PER_WG);
  for (int32_t a = blockIdx.x * BLOCKS_PER_WG + wave; a < a_end; a += COL_WAVES) {
    const int32_t r0 = a * BLOCK, end = min(n, r0 + BLOCK);
    int32_t* out = cols + ((size_t)row * nb + a) * nv;
    int32_t pos = 0;
    for (int32_t i0 = 0; i0 < nv; i0 += 64) {
      const int32_t i = i0 + lane;
      const int32_t j = i < nv ? vrow[i] : INT32_MAX;
      const bool keep = j < end && !covered(ivp, cnt, r0 - j);
      const uint64_t kmask = __ballot(keep);
      if (keep) out[pos + __popcll(kmask & lt_mask)] = j;
      pos += (int32_t)__popcll(kmask);
      if (__ballot(j >= end) != 0ull) break;  // V ascending: the rest is past the block
    }
    if (lane == 0) n_cols[(size_t)row * nb + a] = pos;
  }
}

}  // namespace

hipError_t launch_vs_build_index(const int32_t* V, int32_t nv, const int32_t* S, int32_t ns,
                                 int32_t rows, int32_t seq_len, int32_t* iv, int32_t* n_iv,
                                 int32_t* cols, int32_t* n_cols, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int32_t nb = (seq_len + BLOCK - 1) / BLOCK;
  hipLaunchKernelGGL(vs_intervals_kernel, dim3(rows), dim3(IV_THREADS), 0, s, S, ns, iv, n_iv);
  hipLaunchKernelGGL(vs_cols_kernel, dim3((nb + BLOCKS_PER_WG - 1) / BLOCKS_PER_WG, rows),
                     dim3(COL_WAVES * 64), 0, s, V, nv, iv, n_iv, ns, seq_len, nb, cols, n_cols);
  return hipGetLastError();
}

}  // namespace dsa
