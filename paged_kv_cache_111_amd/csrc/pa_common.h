// Device helpers shared by the HIP kernels of the paged-KV attention step (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even (NaN stays NaN). Used for outputs.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// Two finite non-negative floats (softmax weights) -> packed bf16 pair, rounding half up: add half a bf16 ulp to
// the bit pattern and keep the upper halves (two integer adds and one byte permute). Differs from round to
// nearest even only on exact ties.
__device__ __forceinline__ uint32_t pack_weights_bf16x2(float lo, float hi) {
  const uint32_t a = __float_as_uint(lo) + 0x8000u;
  const uint32_t b = __float_as_uint(hi) + 0x8000u;
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // bytes 3,2 of b (high) and 3,2 of a (low)
}

// Sum of the two bf16 values of a packed pair, as floats. The softmax normaliser is summed from the rounded
// weights that enter the PV product, so that the weights the output is averaged with sum to one exactly: the
// rounding of a dominant weight then cancels against the normaliser instead of scaling the output.
__device__ __forceinline__ float sum_bf16x2(uint32_t w) {
  return __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Max / sum over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float xgroup16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float xgroup16_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}
// Max / sum over the two 32-lane halves of a wave (lane l and lane l ^ 32).
__device__ __forceinline__ float xhalf_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }
__device__ __forceinline__ float xhalf_sum(float v) { return v + __shfl_xor(v, 32, 64); }

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Loads of data a call reads once (the KV rows a decode streams through): the non-temporal cache policy ("nt"
// on gfx950's buffer and global loads) lets the lines leave the caches first, which keeps the reused data (block
// tables, queries, partials) cached and measured 8-10% faster on the decode workloads than the default policy.
constexpr int kLoadStream = 2;  // cache-policy operand of __builtin_amdgcn_raw_buffer_load_*: nt
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// LDS transposed read of 4 x 16-bit: within each 16-lane group, lane i receives element (i % 4) of the 8 bytes
// addressed by lane 4*j + i/4 of its group, for j = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(const_cast<void*>(lds_ptr)));
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename V>
__device__ __forceinline__ bf16x8 as_bf16x8(V v) {
  return __builtin_bit_cast(bf16x8, v);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <typename V>
__device__ __forceinline__ f16x8 as_f16x8(V v) {
  return __builtin_bit_cast(f16x8, v);
}

__device__ __forceinline__ f32x16 mfma32x32x16_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two bf16 values (one 32-bit word) -> two fp16 values. Exact for magnitudes in [2^-14, 65504] (a bf16
// mantissa fits in an fp16 one); smaller magnitudes are truncated toward zero and larger ones clamp to 65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                 __uint_as_float(w & 0xffff0000u)));
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  return u32x4{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]), bf16x2_to_f16x2(v[3])};
}

// Two floats -> packed fp16 pair, round to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + both fp16 values of a packed pair (one v_dot2 against (1, 1)).
__device__ __forceinline__ float add_f16x2(uint32_t w, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, acc, false);
}

}  // namespace pa
