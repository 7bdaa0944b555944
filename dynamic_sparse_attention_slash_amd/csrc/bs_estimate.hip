// Block-sparse estimate, gfx950 [MInference 1.0 article, §2.2 Block-Sparse
// Head: mean-pool Q and K over blocks, score the block pairs, keep the top-k
// key blocks per query block].
//
// pool_kernel: one work-group per (row, block): each thread sums 4 adjacent
//   dims over a strided subset of the block's rows (coalesced 8/16-byte loads),
//   the partial sums meet in LDS in a fixed order, and the mean is written in
//   fp32. HBM-bound: every input byte is read once.
// logits_kernel: L[a][c] = scale * Qp[a] . Kp[c] for the causal triangle
//   c <= a, in 64x64 tiles with fp32 MFMA (16x16x4): fp32 products keep the
//   logits within rounding of the exact dot, which the block ranking needs.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int POOL_THREADS = 256;

template <typename T, int D>
__global__ __launch_bounds__(POOL_THREADS) void pool_kernel(const T* __restrict__ x, int32_t n,
                                                            HeadMap hm, float* __restrict__ out) {
  constexpr int TPR = D / 4;                 // threads per row (4 dims each)
  constexpr int RG = POOL_THREADS / TPR;     // row groups
  __shared__ float part[RG][D];
  const int32_t a = blockIdx.x, row = blockIdx.y;
  const int32_t nb = (n + BLOCK - 1) / BLOCK;
  const int32_t tid = threadIdx.x, dq = tid % TPR, rg = tid / TPR;
  const T* src = x + hm.q_slab(row, n, D);
  const int32_t r0 = a * BLOCK, r1 = min(n, r0 + BLOCK);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int32_t r = r0 + rg; r < r1; r += RG) {
    if constexpr (sizeof(T) == 2) {
      u32x2 w = *reinterpret_cast<const u32x2*>(src + (size_t)r * D + 4 * dq);
      acc[0] += bf16_bits_to_f32(w[0] & 0xffffu);
      acc[1] += bf16_bits_to_f32(w[0] >> 16);
      acc[2] += bf16_bits_to_f32(w[1] & 0xffffu);
      acc[3] += bf16_bits_to_f32(w[1] >> 16);
    } else {
      f32x4 w = *reinterpret_cast<const f32x4*>(src + (size_t)r * D + 4 * dq);
      acc[0] += w[0]; acc[1] += w[1]; acc[2] += w[2]; acc[3] += w[3];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) part[rg][4 * dq + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) s += part[g][tid];
    out[((size_t)row * nb + a) * D + tid] = s / (float)(r1 - r0);
  }
}

template <int D>
__global__ __launch_bounds__(64) void logits_kernel(const float* __restrict__ qp, const float* __restrict__ kp,
                                                    int32_t row0, int32_t nb, float scale, int32_t kv_map,
                                                    HeadMap hm, float* __restrict__ logits) {
  constexpr int DK = D / 4;  // lane group g holds dims DK*g .. DK*g + DK - 1
  const int32_t t = blockIdx.x, lrow = blockIdx.y;
  // triangle tile index t -> (at, ct), ct <= at
  int32_t at = (int32_t)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((at + 1) * (at + 2) / 2 <= t) ++at;
  while (at * (at + 1) / 2 > t) --at;
  const int32_t ct = t - at * (at + 1) / 2;
  const int32_t lane = threadIdx.x, g = lane >> 4, l16 = lane & 15;
  const int32_t grow = row0 + lrow;
  const float* q = qp + (size_t)lrow * nb * D;
  const float* k = kv_map ? kp + ((size_t)hm.b(grow) * hm.kv_heads + hm.kv(grow)) * nb * D
                          : kp + (size_t)lrow * nb * D;
  f32x4 acc[4][4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* qa[4];
  const float* kc[4];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4) {
    qa[b4] = q + (size_t)min(at * 64 + 16 * b4 + l16, nb - 1) * D + DK * g;
    kc[b4] = k + (size_t)min(ct * 64 + 16 * b4 + l16, nb - 1) * D + DK * g;
  }
  for (int s4 = 0; s4 < DK; s4 += 4) {
    f32x4 av[4], bv[4];
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      av[b4] = *reinterpret_cast<const f32x4*>(qa[b4] + s4);
      bv[b4] = *reinterpret_cast<const f32x4*>(kc[b4] + s4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) acc[ib][jb] = mfma_f32(av[ib][e], bv[jb][e], acc[ib][jb]);
  }
  float* L = logits + (size_t)lrow * nb * nb;
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int32_t a = at * 64 + 16 * ib + 4 * g + i;
        const int32_t c = ct * 64 + 16 * jb + l16;
        if (a < nb && c <= a) L[(size_t)a * nb + c] = acc[ib][jb][i] * scale;
      }
}

}  // namespace

hipError_t launch_pool(const void* x, int32_t dtype, int32_t seq_len, int32_t head_dim,
                       int32_t rows, const HeadMap& hm, float* out, hipStream_t s) {
  if (rows == 0 || seq_len == 0) return hipSuccess;
  const int32_t nb = (seq_len + BLOCK - 1) / BLOCK;
  dim3 grid(nb, rows);
  if (dtype == BF16) {
    if (head_dim == 64) hipLaunchKernelGGL((pool_kernel<uint16_t, 64>), grid, dim3(POOL_THREADS), 0, s, static_cast<const uint16_t*>(x), seq_len, hm, out);
    else hipLaunchKernelGGL((pool_kernel<uint16_t, 128>), grid, dim3(POOL_THREADS), 0, s, static_cast<const uint16_t*>(x), seq_len, hm, out);
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((pool_kernel<float, 64>), grid, dim3(POOL_THREADS), 0, s, static_cast<const float*>(x), seq_len, hm, out);
    else hipLaunchKernelGGL((pool_kernel<float, 128>), grid, dim3(POOL_THREADS), 0, s, static_cast<const float*>(x), seq_len, hm, out);
  }
  return hipGetLastError();
}

hipError_t launch_block_logits(const float* qp, const float* kp, int32_t row0, int32_t rows,
                               int32_t nb, int32_t head_dim, float scale, bool kv_map,
                               const HeadMap& hm, float* logits, hipStream_t s) {
  if (rows == 0 || nb == 0) return hipSuccess;
  const int32_t nt = (nb + 63) / 64;
  dim3 grid(nt * (nt + 1) / 2, rows);
  if (head_dim == 64)
    hipLaunchKernelGGL(logits_kernel<64>, grid, dim3(64), 0, s, qp, kp, row0, nb, scale, (int32_t)kv_map, hm, logits);
  else
    hipLaunchKernelGGL(logits_kernel<128>, grid, dim3(64), 0, s, qp, kp, row0, nb, scale, (int32_t)kv_map, hm, logits);
  return hipGetLastError();
}

}  // namespace dsa
