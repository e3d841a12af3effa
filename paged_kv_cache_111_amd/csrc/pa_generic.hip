// Plain vector-ALU attention over the paged cache, for shapes the matrix-core kernels do not take
// (float32 data, head_dim other than 128, GQA groups above 16).
//
// One wave per (query row, query head). Keys are visited 64 at a time, one key per lane: the lane computes its
// score with a dot product, the wave keeps the running max and sum (online softmax), and the weighted values
// are accumulated with the value rows broadcast key by key. Only keys at or before the query's position are
// read, so cache rows past a sequence's length are never touched.
#include "pa_launch.h"

namespace pa {

template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(
    const T* __restrict__ q, int64_t q_stride, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t batch, int32_t Hq, int32_t Hkv, int32_t D,
    int32_t block_size, float scale_log2, void* __restrict__ out, int out_bf16) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  int s, q_len, k_len, r;
  if (cu_q != nullptr) {  // prefill: find the sequence of flattened row t
    int a = 0, b = batch;
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (cu_q[mid] <= t) a = mid; else b = mid;
    }
    s = a;
    q_len = cu_q[s + 1] - cu_q[s];
    k_len = cu_k[s + 1] - cu_k[s];
    r = t - cu_q[s];
  } else {  // decode: row t is sequence t
    s = t;
    q_len = 1;
    k_len = ctx_lens[s];
    r = 0;
  }
  const int pos = k_len - q_len + r;  // this query sees keys 0..pos
  const int G = Hq / Hkv;
  const int g = h / G;
  const int32_t* table = block_table + int64_t(s) * mbps;

  __shared__ float qs[256];
  for (int d = lane; d < D; d += 64) qs[d] = load_as_f32(q + int64_t(t) * q_stride + int64_t(h) * D + d);
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // d = lane + 64 * i
  for (int c0 = 0; c0 <= pos; c0 += 64) {
    const int c = c0 + lane;
    const bool valid = c <= pos;
    float sc = -INFINITY;
    if (valid) {
      const int32_t phys = table[c / block_size];
      const T* kp = k_cache + ((int64_t(phys) * block_size + c % block_size) * Hkv + g) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot += qs[d] * load_as_f32(kp + d);
      sc = dot * scale_log2;
    }
    const float mn = fmaxf(m, wave_max(sc));  // finite: lane 0 is always valid
    const float alpha = exp2f(m - mn);
    const float p = valid ? exp2f(sc - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= alpha;
    const int nvalid = min(64, pos - c0 + 1);
    for (int j = 0; j < nvalid; ++j) {
      const float pj = __shfl(p, j, 64);
      const int cj = c0 + j;
      const int32_t phys = table[cj / block_size];
      const T* vp = v_cache + ((int64_t(phys) * block_size + cj % block_size) * Hkv + g) * D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) acc[i] += pj * load_as_f32(vp + d);
      }
    }
    m = mn;
  }
  const float inv = 1.f / l;
  const int64_t ob = (int64_t(t) * Hq + h) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    if (d >= D) continue;
    if (out_bf16) static_cast<uint16_t*>(out)[ob + d] = f32_to_bf16(acc[i] * inv);
    else static_cast<float*>(out)[ob + d] = acc[i] * inv;
  }
}

void launch_attn_generic(bool bf16, const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                         const int32_t* cu_q, const int32_t* cu_k, const int32_t* ctx_lens,
                         const int32_t* block_table, int32_t mbps, int32_t batch, int32_t rows, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t block_size, float scale, void* out, bool out_bf16,
                         hipStream_t stream) {
  const dim3 grid(rows, Hq);
  const float sl2 = scale * kLog2e;
  if (bf16) {
    hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(64), 0, stream,
                       static_cast<const uint16_t*>(q), q_stride, static_cast<const uint16_t*>(k_cache),
                       static_cast<const uint16_t*>(v_cache), cu_q, cu_k, ctx_lens, block_table, mbps, batch, Hq,
                       Hkv, D, block_size, sl2, out, int(out_bf16));
  } else {
    hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(64), 0, stream, static_cast<const float*>(q),
                       q_stride, static_cast<const float*>(k_cache), static_cast<const float*>(v_cache), cu_q, cu_k,
                       ctx_lens, block_table, mbps, batch, Hq, Hkv, D, block_size, sl2, out, int(out_bf16));
  }
}

}  // namespace pa
