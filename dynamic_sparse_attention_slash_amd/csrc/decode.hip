// Sparse decode attention, gfx950: one new query row per head attends over a
// list of cached keys (for instance the keys kept after prefill by the
// retention scores), or over the whole cache.
//
//   o = sum over listed keys j of softmax_j(scale * q . k_j) * v_j
//
// [Novita blog, §2 Modificación de Atención: after prefill, decoding uses only
// the KV entries a head kept; MInference 1.0 article, §1 Problem Formulation:
// attention restricted to a key set, masked entries excluded exactly.] The
// decode row comes after every cached key, so no causal cut applies.
//
// Work: the list of a row (batch x listed head) is cut into splits of
// split_keys entries; a 256-thread work-group takes one (rows, split). Decoding
// is bound by HBM: every listed key costs its K and V rows once and little
// arithmetic, so the kernel is plain VALU with coalesced 16-byte lane loads.
// A key row is read by LPK = D * sizeof(T) / 16 lanes (16 for bf16, D = 128),
// so a wave covers 64 / LPK keys per step; each lane group keeps its own
// running (max, sum, output) and the groups of a work-group merge through
// registers and LDS at the end. UNROLL steps of K and V loads are issued
// before any of them is used. The splits of a row meet in a second kernel, in
// split order (bit-reproducible).
//
// Whole-cache decode takes the heads of a kv group in bundles of up to four
// rows per work-group, so every K and V row is read once for all of them.
#include <mutex>

#include "../../include/dsa.h"
#include "kernels.hpp"

namespace dsa {
namespace {

// Split partials of the allocation-free decode entry point: a fixed device
// array (each GPU the library runs on holds its own copy for the life of the
// process). Host code never passes this name to a kernel: it is a host-side
// stand-in, not a device address; decode_static_scratch() looks the address
// up once per device.
static __device__ __align__(256) float scratch[DSA_DECODE_NOALLOC_MAX_BYTES / sizeof(float)];
constexpr int MAX_DEVICES = 64;

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int DEC_UNROLL = 4;
constexpr int DEC_HB = 4;  // heads per work-group for the whole cache

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {  // 8 bf16
  static constexpr int E = 8;
  __device__ static void load(const uint16_t* p, float (&x)[8]) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};
template <>
struct Vec16<float> {  // 4 fp32
  static constexpr int E = 4;
  __device__ static void load(const float* p, float (&x)[4]) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = u[i];
  }
};

// Sum over each group of G consecutive lanes (G = 2 .. 32), every lane of the
// group receiving it: DPP quad permutes, then a half-row mirror (G = 8) or row
// rotations by 4 and 8 (G >= 16, which sum the four quads of a 16-lane row),
// then one cross-row swap for G = 32.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 2) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
  if constexpr (G >= 4) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
  if constexpr (G == 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
  if constexpr (G >= 16) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  }
  if constexpr (G == 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// (m, l, acc) of two partial softmax sums over disjoint key sets -> one; m in
// log2 units, NEG_BIG for an empty set
template <int E>
__device__ __forceinline__ void merge_partial(float& m, float& l, float (&acc)[E], float m2, float l2,
                                              const float (&acc2)[E]) {
  const float mn = fmaxf(m, m2);
  const float a1 = fast_exp2(m - mn), a2 = fast_exp2(m2 - mn);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = acc[e] * a1 + acc2[e] * a2;
  m = mn;
}

// Rows of one work-group: a key list is per row (bundles of one row); the
// whole cache is shared by the heads of a kv group, so those go in bundles of
// up to HB rows of one (batch, kv group), each K and V row then read once for
// all of them. Bundle u of a batch walks the kv groups of the work order.
template <int HB>
__device__ __forceinline__ int32_t bundle_rows(const DecodeArgs& a, int32_t u, int32_t (&rows)[HB]) {
  if (HB == 1) {
    rows[0] = u;
    return 1;
  }
  const int32_t b = u / a.bundles_per_batch;
  int32_t r = u - b * a.bundles_per_batch, gi = 0;
  for (;; ++gi) {
    const int32_t size = a.wo.gstart[gi + 1] - a.wo.gstart[gi];
    const int32_t ch = (size + HB - 1) / HB;
    if (r < ch || gi + 1 >= a.wo.n_groups) break;
    r -= ch;
  }
  const int32_t first = a.wo.gstart[gi] + HB * r;
  const int32_t nh = min(HB, a.wo.gstart[gi + 1] - first);
#pragma unroll
  for (int t = 0; t < HB; ++t) rows[t] = b * a.hm.n + a.wo.order[first + min(t, nh - 1)];
  return nh;
}

template <typename T, int D, int HB>
__global__ __launch_bounds__(DEC_THREADS) void decode_split_kernel(DecodeArgs a) {
  constexpr int E = Vec16<T>::E;        // elements per 16-byte lane load
  constexpr int LPK = D / E;            // lanes per key row
  constexpr int KPW = 64 / LPK;         // keys per wave per step
  constexpr int STEP = DEC_WAVES * KPW; // keys per work-group per step
  __shared__ float red[DEC_WAVES][HB][2 + D];

  const int32_t split = blockIdx.x % a.splits;
  int32_t rows[HB];
  const int32_t nh = bundle_rows<HB>(a, blockIdx.x / a.splits, rows);
  const int32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t ks = lane / LPK, pt = lane % LPK;
  // an empty cache has no key to clamp a listed entry into
  const int32_t nk = a.n == 0 ? 0 : a.keys ? min(max(a.n_keys[rows[0]], 0), a.max_keys) : a.n;
  const int32_t s0 = split * a.split_keys, s1 = min(nk, s0 + a.split_keys);
  const int32_t* list = a.keys ? a.keys + (size_t)rows[0] * a.max_keys : nullptr;

  // every row of a bundle reads the same kv head
  const T* ks_ = static_cast<const T*>(a.k) + a.hm.kv_slab(rows[0], a.n, D) + pt * E;
  const T* vs_ = static_cast<const T*>(a.v) + a.hm.kv_slab(rows[0], a.n, D) + pt * E;
  float qv[HB][E], m[HB], l[HB], acc[HB][E];
#pragma unroll
  for (int h = 0; h < HB; ++h) {
    Vec16<T>::load(static_cast<const T*>(a.q) + a.hm.q_slab(rows[h], 1, D) + pt * E, qv[h]);
    m[h] = NEG_BIG;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }

  // The loop runs while the group's first key is in the split; keys past
  // the split end (slots u > 0 of the last step) read the split's last key
  // and get p = 0. One max and one rescale per head and step of DEC_UNROLL
  // keys.
  for (int32_t base = s0 + wave * KPW + ks; base < s1; base += STEP * DEC_UNROLL) {
    float kr[DEC_UNROLL][E], vr[DEC_UNROLL][E];
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      const int32_t pos = min(base + u * STEP, s1 - 1);
      // listed keys are clamped into the cache, so no index reads outside k, v
      const int32_t j = list ? min(max(list[pos], 0), a.n - 1) : pos;
      Vec16<T>::load(ks_ + (size_t)j * D, kr[u]);
      Vec16<T>::load(vs_ + (size_t)j * D, vr[u]);
    }
#pragma unroll
    for (int h = 0; h < HB; ++h) {
      if (h >= nh) break;  // uniform over the work-group
      float sc[DEC_UNROLL];
      float mn = m[h];
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; ++u) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) x = fmaf(qv[h][e], kr[u][e], x);
        x = group_sum<LPK>(x) * a.scale_log2;
        sc[u] = base + u * STEP < s1 ? x : -INFINITY;
        mn = fmaxf(mn, sc[u]);
      }
      const float alpha = fast_exp2(m[h] - mn);
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < DEC_UNROLL; ++u) {
        const float p = fast_exp2(sc[u] - mn);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, vr[u][e], acc[h][e]);
      }
      m[h] = mn;
    }
  }
  // key slots of a wave (lanes with equal pt), then the waves through LDS
#pragma unroll
  for (int h = 0; h < HB; ++h) {
#pragma unroll
    for (int msk = LPK; msk < 64; msk <<= 1) {
      float acc2[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc2[e] = __shfl_xor(acc[h][e], msk, 64);
      const float m2 = __shfl_xor(m[h], msk, 64), l2 = __shfl_xor(l[h], msk, 64);
      merge_partial<E>(m[h], l[h], acc[h], m2, l2, acc2);
    }
    if (ks == 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) red[wave][h][2 + pt * E + e] = acc[h][e];
      if (pt == 0) { red[wave][h][0] = m[h]; red[wave][h][1] = l[h]; }
    }
  }
  __syncthreads();
  for (int32_t t = threadIdx.x; t < nh * (D + 2); t += DEC_THREADS) {
    const int32_t h = t / (D + 2), d = t - h * (D + 2);
    float M = NEG_BIG;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, red[w][h][0]);
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) x += (d == 0 ? 0.f : red[w][h][d]) * fast_exp2(red[w][h][0] - M);
    a.part[((size_t)rows[h] * a.splits + split) * (2 + D) + d] = d == 0 ? M : x;
  }
}

// o = (sum_s 2^(m_s - M) o_s) / (sum_s 2^(m_s - M) l_s) over the splits of a
// row, in split order; a row with no key gives zeros
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int32_t row = blockIdx.x, d = threadIdx.x;
  const float* p = a.part + (size_t)row * a.splits * (2 + D);
  float M = NEG_BIG;
  for (int32_t s = 0; s < a.splits; ++s) M = fmaxf(M, p[(size_t)s * (2 + D)]);
  float L = 0.f, x = 0.f;
  for (int32_t s = 0; s < a.splits; ++s) {
    const float* ps = p + (size_t)s * (2 + D);
    const float w = fast_exp2(ps[0] - M);
    L += ps[1] * w;
    x += ps[2 + d] * w;
  }
  const float out = L > 0.f ? x / L : 0.f;
  T* o = static_cast<T*>(a.o) + a.hm.q_slab(row, 1, D);
  if constexpr (sizeof(T) == 2) o[d] = (T)f32_to_bf16_bits(out);
  else o[d] = out;
}

}  // namespace

int32_t decode_splits(int32_t rows, int32_t max_keys, int32_t& split_keys) {
  // about 4096 work-groups over all rows, at least 256 keys per split
  const int32_t target = rows > 0 ? (4096 + rows - 1) / rows : 1;
  int32_t sk = (max_keys + target - 1) / target;
  sk = ((sk + 255) / 256) * 256;
  split_keys = sk < 256 ? 256 : sk;
  const int32_t splits = (max_keys + split_keys - 1) / split_keys;
  return splits < 1 ? 1 : splits;
}

size_t decode_workspace_bytes(int32_t rows, int32_t max_keys, int32_t head_dim) {
  int32_t sk;
  const int32_t splits = decode_splits(rows, max_keys, sk);
  return (size_t)rows * splits * (2 + head_dim) * sizeof(float);
}

hipError_t decode_static_scratch(float** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // with `dev` current: this device's copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = static_cast<float*>(addr[dev]);
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t launch_decode(DecodeArgs a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  a.splits = decode_splits(a.rows, a.keys ? a.max_keys : a.n, a.split_keys);
  int32_t bundles = a.rows;
  if (!a.keys) {
    a.bundles_per_batch = 0;
    for (int32_t g = 0; g < a.wo.n_groups; ++g)
      a.bundles_per_batch += (a.wo.gstart[g + 1] - a.wo.gstart[g] + DEC_HB - 1) / DEC_HB;
    bundles = (a.rows / a.hm.n) * a.bundles_per_batch;
  }
  const dim3 grid((unsigned)((long long)bundles * a.splits));
  auto sp = a.keys
      ? (a.dtype == BF16 ? (a.head_dim == 64 ? decode_split_kernel<uint16_t, 64, 1> : decode_split_kernel<uint16_t, 128, 1>)
                         : (a.head_dim == 64 ? decode_split_kernel<float, 64, 1> : decode_split_kernel<float, 128, 1>))
      : (a.dtype == BF16 ? (a.head_dim == 64 ? decode_split_kernel<uint16_t, 64, DEC_HB> : decode_split_kernel<uint16_t, 128, DEC_HB>)
                         : (a.head_dim == 64 ? decode_split_kernel<float, 64, DEC_HB> : decode_split_kernel<float, 128, DEC_HB>));
  auto cb = a.dtype == BF16 ? (a.head_dim == 64 ? decode_combine_kernel<uint16_t, 64> : decode_combine_kernel<uint16_t, 128>)
                            : (a.head_dim == 64 ? decode_combine_kernel<float, 64> : decode_combine_kernel<float, 128>);
  hipLaunchKernelGGL(sp, grid, dim3(DEC_THREADS), 0, s, a);
  hipLaunchKernelGGL(cb, dim3(a.rows), dim3(a.head_dim), 0, s, a);
  return hipGetLastError();
}

}  // namespace dsa
