// Next-token sampling from each sequence's logits with temperature, softmax and Gumbel-max ("Nano-vLLM 架构详解"
// §2.4, the sampling stage; "一个 prompt 的一生" §4, logits -> Sampler (Gumbel-max) -> token ids).
//
// Gumbel-max draws from softmax(l / T) as argmax_i (log softmax(l / T)_i + g_i), g_i = -ln(-ln u_i); the
// log-sum-exp of the softmax is the same for every i, so the kernel maximises s_i = l_i * (1/T) + g_i and never
// forms the softmax. T = 0 is greedy (s_i = l_i). Ties go to the lower index.
//
// The uniforms come from a counter-based generator, Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011): one call per 4 consecutive logits, counter
// (i / 4, row, offset mod 2^32, offset div 2^32), key (seed mod 2^32, seed div 2^32); word i % 4 gives
// u = ((x >> 9) + 1/2) * 2^-23, exact in fp32 and strictly inside (0, 1). Same draws for the same (seed, offset,
// row, i) in any launch shape.
//
// Two passes: workgroups take chunks of a row (each thread 4 logits at a time) and leave the chunk's best
// (score, index); one wave per row then picks the best chunk. The work is the generator and two logarithms per
// logit; the logits are read once.
#include "pa_launch.h"

namespace pa {

constexpr int kSampleThreads = 256;

struct Philox4 {
  uint32_t x[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return Philox4{{c0, c1, c2, c3}};
}

// g = -ln(-ln u) through the hardware log2 (u >= 2^-24 and -ln u >= 2^-24: no denormal inputs).
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  constexpr float kLn2 = 0.69314718055994530942f;
  const float u = __fmaf_rn(float(x >> 9), 1.1920928955078125e-07f, 5.9604644775390625e-08f);  // exact
  const float e = -kLn2 * __builtin_amdgcn_logf(u);  // -ln u > 0
  return -kLn2 * __builtin_amdgcn_logf(e);
}

__device__ __forceinline__ void take_best(float s, int i, float& best, int& best_i) {
  if (s > best || (s == best && i < best_i)) {
    best = s;
    best_i = i;
  }
}

// Pass 1: grid (n_chunks, batch). part[b * n_chunks + c] = (best score, its index) over chunk c of row b.
__global__ __launch_bounds__(kSampleThreads) void sample_chunk_kernel(
    const float* __restrict__ logits, int64_t row_stride, const float* __restrict__ temperatures, int32_t vocab,
    int32_t chunk_groups, uint32_t k0, uint32_t k1, uint32_t off_lo, uint32_t off_hi, float2* __restrict__ part,
    int vec4) {
  const int b = blockIdx.y;
  const int c = blockIdx.x;
  const float* row = logits + int64_t(b) * row_stride;
  const float T = temperatures[b];
  const bool greedy = !(T > 0.f);
  const float inv_t = greedy ? 0.f : 1.f / T;
  const int groups = (vocab + 3) >> 2;
  const int g0 = c * chunk_groups;
  const int g1 = min(groups, g0 + chunk_groups);
  float best = -INFINITY;
  int best_i = INT32_MAX;
  for (int g = g0 + int(threadIdx.x); g < g1; g += kSampleThreads) {
    const int i0 = 4 * g;
    float l[4];
    if (vec4 && i0 + 3 < vocab) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(row + i0);
#pragma unroll
      for (int j = 0; j < 4; ++j) l[j] = v[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) l[j] = i0 + j < vocab ? row[i0 + j] : -INFINITY;
    }
    if (greedy) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i0 + j < vocab) take_best(l[j], i0 + j, best, best_i);
    } else {
      const Philox4 r = philox4x32_10(uint32_t(g), uint32_t(b), off_lo, off_hi, k0, k1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i0 + j < vocab) take_best(__fadd_rn(__fmul_rn(l[j], inv_t), gumbel_of(r.x[j])), i0 + j, best, best_i);
    }
  }
  // wave, then workgroup reduction of (score, index)
  for (int off = 32; off > 0; off >>= 1) {
    const float s = __shfl_xor(best, off, 64);
    const int i = __shfl_xor(best_i, off, 64);
    take_best(s, i, best, best_i);
  }
  __shared__ float ws[kSampleThreads / 64];
  __shared__ int wi[kSampleThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    ws[wave] = best;
    wi[wave] = best_i;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kSampleThreads / 64; ++w) take_best(ws[w], wi[w], best, best_i);
    part[int64_t(b) * gridDim.x + c] = make_float2(best, __int_as_float(best_i));
  }
}

// Pass 2: one wave per row picks the best chunk.
__global__ __launch_bounds__(64) void sample_pick_kernel(const float2* __restrict__ part, int32_t n_chunks,
                                                         int32_t vocab, int32_t* __restrict__ tokens) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  float best = -INFINITY;
  int best_i = INT32_MAX;
  for (int c = lane; c < n_chunks; c += 64) {
    const float2 p = part[int64_t(b) * n_chunks + c];
    take_best(p.x, __float_as_int(p.y), best, best_i);
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float s = __shfl_xor(best, off, 64);
    const int i = __shfl_xor(best_i, off, 64);
    take_best(s, i, best, best_i);
  }
  if (lane == 0) tokens[b] = best_i < vocab ? best_i : 0;  // a row of NaN logits has no maximum: token 0
}

int32_t sample_chunks(int32_t batch, int32_t vocab) {
  const int32_t groups = (vocab + 3) / 4;
  const int32_t want = (1024 + batch - 1) / batch;            // about 1024 workgroups in all
  const int32_t most = max(1, (groups + 511) / 512);          // at least 512 groups (2048 logits) per chunk
  return max(1, min(want, most));
}

void launch_sample(const float* logits, int64_t row_stride, const float* temperatures, int32_t batch,
                   int32_t vocab, uint64_t seed, uint64_t offset, int32_t* tokens, void* workspace,
                   hipStream_t stream) {
  const int32_t n_chunks = sample_chunks(batch, vocab);
  const int32_t groups = (vocab + 3) / 4;
  const int32_t chunk_groups = (groups + n_chunks - 1) / n_chunks;
  const int vec4 = (row_stride % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) ? 1 : 0;
  float2* part = static_cast<float2*>(workspace);
  hipLaunchKernelGGL(sample_chunk_kernel, dim3(n_chunks, batch), dim3(kSampleThreads), 0, stream, logits,
                     row_stride, temperatures, vocab, chunk_groups, uint32_t(seed), uint32_t(seed >> 32),
                     uint32_t(offset), uint32_t(offset >> 32), part, vec4);
  hipLaunchKernelGGL(sample_pick_kernel, dim3(batch), dim3(64), 0, stream, part, n_chunks, vocab, tokens);
}

}  // namespace pa
