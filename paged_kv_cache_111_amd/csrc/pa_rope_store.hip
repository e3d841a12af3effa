// Pre-attention step of the new tokens, fused into one pass per token: k_norm (RMSNorm of each KV head's key
// with a learned weight), rotary position embedding by table lookup, and the store of the rotated key into the
// token's cache slot; V is stored as is; Q, when given, gets q_norm and the same rotation into its own output.
// In a layer these run back to back before attention (q_norm -> k_norm -> rope -> store_kvcache, "一个 prompt
// 的一生：nano-vllm 从起服务到吐出 token" §2.2.4; the rotation is a table lookup, same page §3.3.2); fusing them reads
// and writes each key once instead of three times.
//
// Formulas (the pages name the steps, not their arithmetic): y = x / sqrt(mean(x^2) + eps) * w over head_dim,
// then the pairs (y[i], y[i + D/2]) are rotated by the angle of frequency i at the token's position, whose cos
// and sin are row `position` of the table, cos in [0, D/2) and sin in [D/2, D). Arithmetic in fp32; bf16
// results are rounded to nearest even.
//
// Layout of the work: one wave per token. A head of D elements is handled by D/16 lanes; lane s of a head owns
// the 8 pairs 8s .. 8s+7, i.e. elements 8s.. of the first half and D/2 + 8s.. of the second (two 8-element
// vectors). The sum of squares is combined over the head's lanes with shuffles. 64 / (D/16) heads per pass.
#include "pa_launch.h"

namespace pa {

constexpr int kRopeThreads = 256;  // four tokens per workgroup

// Eight consecutive elements to and from fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
  const u32x4 v = ld16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(v[i] << 16);
    x[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&x)[8]) {
  const u32x4 v = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
  st16(p, v);
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void copy8(uint16_t* d, const uint16_t* s) { st16(d, ld16(s)); }
__device__ __forceinline__ void copy8(float* d, const float* s) {
  *reinterpret_cast<f32x4*>(d) = *reinterpret_cast<const f32x4*>(s);
  *reinterpret_cast<f32x4*>(d + 4) = *reinterpret_cast<const f32x4*>(s + 4);
}

// RMSNorm + rotation of the H heads of one token: src [H, D] -> dst [H, D].
template <typename T>
__device__ __forceinline__ void norm_rope_heads(const T* __restrict__ src, T* __restrict__ dst,
                                                const T* __restrict__ w, const float* __restrict__ cs_row, int H,
                                                int D, float eps, int lane) {
  const int lph = D >> 4;       // lanes per head (a power of two)
  const int hpp = 64 / lph;     // heads per pass
  const int p = 8 * (lane & (lph - 1));  // first pair owned by this lane
  const int half = D >> 1;
  float wa[8], wb[8], ca[8], sa[8];
  load8(w + p, wa);
  load8(w + half + p, wb);
  load8(cs_row + p, ca);
  load8(cs_row + half + p, sa);
  const float inv_d = 1.f / float(D);
  for (int h0 = 0; h0 < H; h0 += hpp) {
    const int h = h0 + lane / lph;
    const bool ok = h < H;
    float a[8], b[8];
    if (ok) {
      load8(src + int64_t(h) * D + p, a);
      load8(src + int64_t(h) * D + half + p, b);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = b[i] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += a[i] * a[i] + b[i] * b[i];
    for (int off = 1; off < lph; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const float r = 1.f / sqrtf(ss * inv_d + eps);
    float oa[8], ob[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x1 = a[i] * r * wa[i];
      const float x2 = b[i] * r * wb[i];
      oa[i] = x1 * ca[i] - x2 * sa[i];
      ob[i] = x2 * ca[i] + x1 * sa[i];
    }
    if (ok) {
      store8(dst + int64_t(h) * D + p, oa);
      store8(dst + int64_t(h) * D + half + p, ob);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void norm_rope_store_kernel(
    const T* __restrict__ k, int64_t k_stride, const T* __restrict__ v, int64_t v_stride,
    const T* __restrict__ k_w, const T* __restrict__ q, int64_t q_stride, const T* __restrict__ q_w,
    T* __restrict__ q_out, int32_t Hq, float eps, const int32_t* __restrict__ positions,
    const float* __restrict__ cos_sin, int32_t max_position, T* __restrict__ k_cache, T* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t Hkv, int32_t D) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kRopeThreads / 64) + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int pos = min(max(positions[t], 0), max_position - 1);  // a position outside the table reads its edge
  const float* row = cos_sin + int64_t(pos) * D;
  const int32_t slot = slot_mapping[t];
  if (slot >= 0) {
    const int64_t row_elems = int64_t(Hkv) * D;
    norm_rope_heads(k + int64_t(t) * k_stride, k_cache + int64_t(slot) * row_elems, k_w, row, Hkv, D, eps, lane);
    const T* vs = v + int64_t(t) * v_stride;
    T* vd = v_cache + int64_t(slot) * row_elems;
    for (int64_t i = 8 * lane; i < row_elems; i += 512) copy8(vd + i, vs + i);
  }
  if (q != nullptr)
    norm_rope_heads(q + int64_t(t) * q_stride, q_out + int64_t(t) * Hq * D, q_w, row, Hq, D, eps, lane);
}

void launch_norm_rope_store(const void* k, int64_t k_stride, const void* v, int64_t v_stride, const void* k_w,
                            const void* q, int64_t q_stride, const void* q_w, void* q_out, int32_t Hq, float eps,
                            const int32_t* positions, const float* cos_sin, int32_t max_position, void* k_cache,
                            void* v_cache, const int32_t* slot_mapping, int32_t num_tokens, int32_t Hkv,
                            int32_t D, bool bf16, hipStream_t stream) {
  const int grid = (num_tokens + kRopeThreads / 64 - 1) / (kRopeThreads / 64);
  if (bf16) {
    using T = uint16_t;
    hipLaunchKernelGGL(norm_rope_store_kernel<T>, dim3(grid), dim3(kRopeThreads), 0, stream,
                       static_cast<const T*>(k), k_stride, static_cast<const T*>(v), v_stride,
                       static_cast<const T*>(k_w), static_cast<const T*>(q), q_stride, static_cast<const T*>(q_w),
                       static_cast<T*>(q_out), Hq, eps, positions, cos_sin, max_position, static_cast<T*>(k_cache),
                       static_cast<T*>(v_cache), slot_mapping, num_tokens, Hkv, D);
  } else {
    using T = float;
    hipLaunchKernelGGL(norm_rope_store_kernel<T>, dim3(grid), dim3(kRopeThreads), 0, stream,
                       static_cast<const T*>(k), k_stride, static_cast<const T*>(v), v_stride,
                       static_cast<const T*>(k_w), static_cast<const T*>(q), q_stride, static_cast<const T*>(q_w),
                       static_cast<T*>(q_out), Hq, eps, positions, cos_sin, max_position, static_cast<T*>(k_cache),
                       static_cast<T*>(v_cache), slot_mapping, num_tokens, Hkv, D);
  }
}

}  // namespace pa
