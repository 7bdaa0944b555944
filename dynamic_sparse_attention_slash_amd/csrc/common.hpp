// Shared device-side helpers for the gfx950 kernels: vector types, bf16
// conversion, MFMA wrappers, wave reductions and the head-row map.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int BLOCK = 64;        // query/key block rows
constexpr int MAX_HEADS = 256;   // heads one call may list

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Dtype : int32_t { BF16 = 0, F32 = 1 };

// Row r of a call's work = (batch b, listed head t): query head h[t], kv head
// h[t] / (q_heads / kv_heads). Passed by value as a kernel argument.
struct HeadMap {
  int32_t n;         // listed heads
  int32_t q_heads;   // heads of the tensor the rows index (q, or x for pooling)
  int32_t kv_heads;  // kv heads (k, v)
  int32_t h[MAX_HEADS];
  __device__ __forceinline__ int32_t b(int32_t row) const { return row / n; }
  __device__ __forceinline__ int32_t head(int32_t row) const { return h[row % n]; }
  __device__ __forceinline__ int32_t kv(int32_t row) const {
    return h[row % n] / (q_heads / kv_heads);
  }
  // element offsets of the [seq][dim] slabs this row reads / writes
  __device__ __forceinline__ size_t q_slab(int32_t row, int32_t seq, int32_t dim) const {
    return ((size_t)b(row) * q_heads + head(row)) * (size_t)seq * dim;
  }
  __device__ __forceinline__ size_t kv_slab(int32_t row, int32_t seq, int32_t dim) const {
    return ((size_t)b(row) * kv_heads + kv(row)) * (size_t)seq * dim;
  }
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (low half = lo), round to nearest even; one
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// sum of the two bf16 values of a packed pair, as floats
__device__ __forceinline__ float packed_pair_sum(uint32_t u) {
  return __uint_as_float(u << 16) + __uint_as_float(u & 0xffff0000u);
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m, 64)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m, 64); }

// XOR swizzle of the 16-byte chunks of LDS row r (an XOR-linear map of r's
// low four bits), under which 16 rows read at one logical chunk per 16 lanes
// (ds_read_b128) and 4 rows x 2 chunks per 16 lanes (ds_read_b64 and its
// transposing form) touch distinct banks in every pass of gfx950's LDS.
// Chunk c of row r lives at chunk c ^ lds_chunk_swz(r) (masked to the row's
// chunk count).
__device__ __forceinline__ int lds_chunk_swz(int r) {
  return (int)((0xae629d51bf738c40ull >> (4 * (r & 15))) & 15);
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_BIG = -1.0e30f;  // finite "minus infinity" for running maxima

}  // namespace dsa
