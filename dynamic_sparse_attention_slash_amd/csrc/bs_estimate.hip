// Block-sparse estimate, gfx950 [MInference 1.0 article, §2.2 Block-Sparse
// Head: mean-pool Q and K over blocks, score the block pairs, keep the top-k
// key blocks per query block].
//
// pool_kernel: one work-group per (row, block): each thread sums the 8 (bf16)
//   or 4 (fp32) adjacent dims of one 16-byte load over a strided subset of the
//   block's rows, all its loads of a whole block in flight at once,
//   the partial sums meet in LDS in a fixed order, and the mean is written in
//   fp32. HBM-bound: every input byte is read once.
// logits_kernel: L[a][c] = scale * Qp[a] . Kp[c] for the causal triangle
//   c <= a, in 64x64 tiles. The fp32 dot products run on the bf16 MFMA as
//   three products of hi/lo bf16 splits with fp32 accumulation, which keeps
//   them within about 2^-16 relative of the exact dot at five times the rate
//   of the fp32 MFMA; split_kernel forms the splits once per pooled row
//   beforehand.
#include "kernels.hpp"

namespace dsa {
namespace {

constexpr int POOL_THREADS = 256;

template <typename T, int D>
__global__ __launch_bounds__(POOL_THREADS) void pool_kernel(const T* __restrict__ x, int32_t n,
                                                            HeadMap hm, float* __restrict__ out) {
  constexpr int EPT = 16 / sizeof(T);         // dims per thread: one 16-byte load per row
  constexpr int TPR = D / EPT;                // threads per row
  constexpr int RG = POOL_THREADS / TPR;      // row groups
  constexpr int RPT = BLOCK / RG;             // rows per thread in a whole block
  __shared__ float part[RG][D];
  const int32_t a = blockIdx.x, row = blockIdx.y;
  const int32_t nb = (n + BLOCK - 1) / BLOCK;
  const int32_t tid = threadIdx.x, dq = tid % TPR, rg = tid / TPR;
  const T* src = x + hm.q_slab(row, n, D);
  const int32_t r0 = a * BLOCK, r1 = min(n, r0 + BLOCK);
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
  auto add_row = [&](const u32x4& w) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_bits_to_f32(w[e] & 0xffffu);
        acc[2 * e + 1] += bf16_bits_to_f32(w[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(w[e]);
    }
  };
  const u32x4* base = reinterpret_cast<const u32x4*>(src + (size_t)r0 * D + EPT * dq);
  if (r1 - r0 == BLOCK) {
    // a whole block: all of this thread's rows loaded before they are added
    u32x4 w[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) w[k] = base[(size_t)(rg + RG * k) * (D / EPT)];
#pragma unroll
    for (int k = 0; k < RPT; ++k) add_row(w[k]);
  } else {
    for (int32_t r = rg; r < r1 - r0; r += RG) add_row(base[(size_t)r * (D / EPT)]);
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) part[rg][EPT * dq + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) s += part[g][tid];
    out[((size_t)row * nb + a) * D + tid] = s / (float)(r1 - r0);
  }
}

// Eight fp32 values as bf16 pairs: hi = bf16(x) (nearest even) and
// lo = bf16(x - hi), so x - hi - lo is below 2^-17 |x|.
__device__ __forceinline__ void split8(const float* p, u32x4& hi, u32x4& lo) {
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
  const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t h = pack_bf16x2(x[2 * e], x[2 * e + 1]);
    hi[e] = h;
    lo[e] = pack_bf16x2(x[2 * e] - __uint_as_float(h << 16), x[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
  }
}

// Pooled rows [row0, row0 + rows) of a call as bf16 hi / lo arrays
// [rows][nb][dim], eight values per thread. kv_map: row r reads pooled-K row
// b * kv_heads + kv head of call row row0 + r; else row r of src.
__global__ __launch_bounds__(256) void split_kernel(const float* __restrict__ src, int32_t row0, int32_t nb,
                                                    int32_t dim, int32_t kv_map, HeadMap hm,
                                                    uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  const size_t per_row = (size_t)nb * dim;  // a multiple of 8
  const int32_t r = blockIdx.y;
  const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (e >= per_row) return;
  const int32_t grow = row0 + r;
  const float* x = kv_map ? src + ((size_t)hm.b(grow) * hm.kv_heads + hm.kv(grow)) * per_row
                          : src + (size_t)r * per_row;
  u32x4 h, l;
  split8(x + e, h, l);
  *reinterpret_cast<u32x4*>(hi + (size_t)r * per_row + e) = h;
  *reinterpret_cast<u32x4*>(lo + (size_t)r * per_row + e) = l;
}

// One wave per 64x64 tile of the causal triangle, on the hi / lo splits of
// the pooled rows: each fp32 product qp . kp is taken as hi.hi + hi.lo +
// lo.hi on the bf16 MFMA (16x16x32), accumulated in fp32; the dropped lo.lo
// term and the split residuals stay below about 2^-16 of |qp| |kp| per
// product. The tile goes out through LDS, 16 rows at a time, as 256-byte row
// segments.
template <int D>
__global__ __launch_bounds__(64) void logits_kernel(const uint16_t* __restrict__ qh, const uint16_t* __restrict__ ql,
                                                    const uint16_t* __restrict__ kh, const uint16_t* __restrict__ kl,
                                                    int32_t nb, float scale, float* __restrict__ logits) {
  constexpr int KS = D / 32;  // k-steps; lane group g holds dims 32s + 8g .. + 7
  constexpr int PS = 68;      // padded LDS row (floats)
  __shared__ __align__(16) float buf[16 * PS];
  const int32_t t = blockIdx.x, lrow = blockIdx.y;
  // triangle tile index t -> (at, ct), ct <= at
  int32_t at = (int32_t)((sqrtf(8.f * (float)t + 1.f) - 1.f) * 0.5f);
  while ((at + 1) * (at + 2) / 2 <= t) ++at;
  while (at * (at + 1) / 2 > t) --at;
  const int32_t ct = t - at * (at + 1) / 2;
  const int32_t lane = threadIdx.x, g = lane >> 4, l16 = lane & 15;
  const size_t rbase = (size_t)lrow * nb * D;
  f32x4 acc[4][4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
  size_t qo[4], ko[4];
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4) {
    qo[b4] = rbase + (size_t)min(at * 64 + 16 * b4 + l16, nb - 1) * D + 8 * g;
    ko[b4] = rbase + (size_t)min(ct * 64 + 16 * b4 + l16, nb - 1) * D + 8 * g;
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int b4 = 0; b4 < 4; ++b4) {
      ah[b4] = *reinterpret_cast<const u32x4*>(qh + qo[b4] + 32 * s);
      al[b4] = *reinterpret_cast<const u32x4*>(ql + qo[b4] + 32 * s);
      bh[b4] = *reinterpret_cast<const u32x4*>(kh + ko[b4] + 32 * s);
      bl[b4] = *reinterpret_cast<const u32x4*>(kl + ko[b4] + 32 * s);
    }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        acc[ib][jb] = mfma_bf16(ah[ib], bh[jb], acc[ib][jb]);
        acc[ib][jb] = mfma_bf16(ah[ib], bl[jb], acc[ib][jb]);
        acc[ib][jb] = mfma_bf16(al[ib], bh[jb], acc[ib][jb]);
      }
  }
  float* L = logits + (size_t)lrow * nb * nb;
  // a tile wholly inside the triangle and the arrays, and rows whose 16-byte
  // segments stay aligned, go out as float4 rows; others element by element
  const bool whole = ct < at && at * 64 + 64 <= nb && (nb & 3) == 0;
  const int32_t rr0 = lane >> 4, cc = 4 * (lane & 15);
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
#pragma unroll
      for (int i = 0; i < 4; ++i) buf[(4 * g + i) * PS + 16 * jb + l16] = acc[ib][jb][i] * scale;
    __syncthreads();
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int32_t rr = 4 * q4 + rr0;
      const f32x4 v = *reinterpret_cast<const f32x4*>(&buf[rr * PS + cc]);
      const int32_t a = at * 64 + 16 * ib + rr, c = ct * 64 + cc;
      if (whole) {
        *reinterpret_cast<f32x4*>(L + (size_t)a * nb + c) = v;
      } else if (a < nb) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e <= a && c + e < nb) L[(size_t)a * nb + c + e] = v[e];
      }
    }
    __syncthreads();
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
                               const HeadMap& hm, uint16_t* split, float* logits, hipStream_t s) {
  if (rows == 0 || nb == 0) return hipSuccess;
  const size_t per = (size_t)rows * nb * head_dim;
  uint16_t* qh = split;
  uint16_t* ql = qh + per;
  uint16_t* kh = ql + per;
  uint16_t* kl = kh + per;
  const dim3 sgrid((unsigned)(((size_t)nb * head_dim / 8 + 255) / 256), rows);
  hipLaunchKernelGGL(split_kernel, sgrid, dim3(256), 0, s, qp, row0, nb, head_dim, 0, hm, qh, ql);
  hipLaunchKernelGGL(split_kernel, sgrid, dim3(256), 0, s, kp, row0, nb, head_dim, (int32_t)kv_map, hm, kh, kl);
  const int32_t nt = (nb + 63) / 64;
  dim3 grid(nt * (nt + 1) / 2, rows);
  if (head_dim == 64)
    hipLaunchKernelGGL(logits_kernel<64>, grid, dim3(64), 0, s, qh, ql, kh, kl, nb, scale, logits);
  else
    hipLaunchKernelGGL(logits_kernel<128>, grid, dim3(64), 0, s, qh, ql, kh, kl, nb, scale, logits);
  return hipGetLastError();
}

}  // namespace dsa
