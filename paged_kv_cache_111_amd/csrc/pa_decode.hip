// Paged decode on the matrix cores: one query token per sequence, bf16, head_dim 128, GQA group <= 16.
//
// Work item = (sequence s, KV head, split of split_tokens keys); one wave each. The G query heads of the KV
// head are the N = 16 columns of 16x16x32 bf16 MFMAs (unused columns are zero), so each key's K and V row is
// read from HBM exactly once per split:
//   S^T[key, g] = K[key, :] . Q[g, :]      A = K rows straight from HBM (16 B per lane), B = Q^T in registers
//   O^T[d, g]  += V^T[d, key] P^T[key, g]  A = V^T from a row-major LDS tile via the transpose read, B = P^T
//                                           kept in the registers the score MFMA left it in
// The key -> MFMA k-slot assignment of the second product is chosen so that P^T needs no data movement: lane
// group lg (lanes 16lg..16lg+15) holds keys 4lg..4lg+3 of each 16-key score tile, and those become its k-slots.
// Online softmax runs per column g in the log2 domain. Each split writes an unnormalised partial (m, l, O);
// sequences that fit in one split write the final output directly.
//
// Keys past the sequence's length are never loaded: their scores are -inf and their V rows are zero in LDS, so
// whatever the cache holds there (NaN included) cannot reach the output. The split/merge scheme is the
// standard log-sum-exp combination; the pages do not describe the decode kernel's internals (they only name
// the FlashAttention KV-cache call, "Nano-vLLM 架构详解" §3.2).
#include "pa_launch.h"

namespace pa {

constexpr int kDecKeys = 32;       // keys per inner iteration (two 16-key score tiles)
constexpr int kVRow = 128 + 8;     // LDS row stride of the V tile, in bf16 elements (272 bytes)

template <bool kPow2>
__device__ __forceinline__ int64_t slot_of_key(const int32_t* table, int key, int bs, int bs_shift) {
  if (kPow2) return int64_t(table[key >> bs_shift]) * bs + (key & (bs - 1));
  const int blk = key / bs;
  return int64_t(table[blk]) * bs + (key - blk * bs);
}

template <bool kPow2>
__global__ __launch_bounds__(64) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t Hq, int32_t Hkv, int32_t bs, int32_t bs_shift,
    float scale_log2, void* __restrict__ out, int out_bf16, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int32_t split_tokens, int32_t max_splits) {
  const int h = blockIdx.x;
  const int split = blockIdx.y;
  const int s = blockIdx.z;
  const int L = ctx_lens[s];
  const int nsplit = (L + split_tokens - 1) / split_tokens;
  if (split >= nsplit) return;
  const int t0 = split * split_tokens;
  const int t1 = min(L, t0 + split_tokens);
  const int G = Hq / Hkv;
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int li = lane & 15;
  const int32_t* table = block_table + int64_t(s) * mbps;
  const int64_t row_stride = int64_t(Hkv) * 128;  // elements between consecutive slots
  const uint16_t* kbase = k_cache + h * 128;
  const uint16_t* vbase = v_cache + h * 128;

  // B operand of the score MFMA: lane holds Q[g = li][d = 8lg + 32ks .. +7]
  bf16x8 qb[4];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp = q + int64_t(s) * q_stride + int64_t(h * G + li) * 128 + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = as_bf16x8(li < G ? ld16(qp + 32 * ks) : z);
  }

  __shared__ __attribute__((aligned(16))) uint16_t vt[kDecKeys * kVRow];

  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  for (int base = t0; base < t1; base += kDecKeys) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    // K rows for the two 16-key score tiles: lane holds K[base + 16tt + li][8lg + 32ks .. +7]
    u32x4 kr[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int key = base + 16 * tt + li;
      if (key < t1) {
        const uint16_t* kp = kbase + slot_of_key<kPow2>(table, key, bs, bs_shift) * row_stride + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kr[tt][ks] = ld16(kp + 32 * ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kr[tt][ks] = z;
      }
    }
    // V tile: 32 keys x 128 d as 512 pieces of 16 bytes; piece c -> key c / 16, d 8 * (c % 16)
    u32x4 vr[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = it * 64 + lane;
      const int key = base + (c >> 4);
      vr[it] = key < t1 ? ld16(vbase + slot_of_key<kPow2>(table, key, bs, bs_shift) * row_stride + 8 * (c & 15))
                        : z;
    }

    // scores: sc[tt][i] is key base + 16tt + 4lg + i, query column g = li
    f32x4 sc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[tt] = mfma16x16x32(as_bf16x8(kr[tt][ks]), qb[ks], sc[tt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = base + 16 * tt + 4 * lg + i;
        const float v = key < t1 ? sc[tt][i] * scale_log2 : -INFINITY;
        sc[tt][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = xgroup16_max(mx);
    const float mn = fmaxf(m, mx);  // finite: every tile holds at least one key
    const float alpha = exp2f(m - mn);
    m = mn;
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = exp2f(sc[j >> 2][j & 3] - mn);
      psum += pv[j];
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
    const u32x4 pw = {pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                      pack_bf16x2(pv[6], pv[7])};
    const bf16x8 pb = as_bf16x8(pw);

    __syncthreads();  // the previous tile's transposed reads are done
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = it * 64 + lane;
      st16(&vt[(c >> 4) * kVRow + 8 * (c & 15)], vr[it]);
    }
    __syncthreads();
    // A operand of O^T: lane (li, lg) needs V[key][d = 16mt + li] for keys 4lg..4lg+3 and 16+4lg..16+4lg+3
    const uint16_t* r0 = &vt[(4 * lg + (li >> 2)) * kVRow + 4 * (li & 3)];
    const uint16_t* r1 = r0 + 16 * kVRow;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const i16x4 a0 = lds_read_tr16(r0 + 16 * mt);
      const i16x4 a1 = lds_read_tr16(r1 + 16 * mt);
      const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[mt] = mfma16x16x32(av, pb, o[mt]);
    }
  }

  lsum = xgroup16_sum(lsum);
  if (li >= G) return;
  // o[mt][i] is O^T[d = 16mt + 4lg + i][g = li]
  const int hq = h * G + li;
  if (nsplit == 1) {
    const float inv = 1.f / lsum;
    const int64_t ob = (int64_t(s) * Hq + hq) * 128 + 4 * lg;
    if (out_bf16) {
      uint16_t* op = static_cast<uint16_t*>(out) + ob;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const u32x2 w = {pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv), pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv)};
        *reinterpret_cast<u32x2*>(op + 16 * mt) = w;
      }
    } else {
      float* op = static_cast<float*>(out) + ob;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(op + 16 * mt) = o[mt] * inv;
    }
  } else {
    const int64_t pi = (int64_t(s) * Hq + hq) * max_splits + split;
    float* pp = part_o + pi * 128 + 4 * lg;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(pp + 16 * mt) = o[mt];
    if (lg == 0) part_ml[pi] = make_float2(m, lsum);
  }
}

// Merge of the split partials of one (sequence, query head): M = max m_i, L = sum l_i 2^(m_i - M),
// O = sum O_i 2^(m_i - M) / L. Sequences that fit in one split were finished by the first pass.
__global__ __launch_bounds__(64) void decode_reduce_kernel(const int32_t* __restrict__ ctx_lens,
                                                           const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml, int32_t Hq,
                                                           int32_t split_tokens, int32_t max_splits,
                                                           void* __restrict__ out, int out_bf16) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = ctx_lens[s];
  const int nsplit = (L + split_tokens - 1) / split_tokens;
  if (nsplit <= 1) return;
  const int64_t pi0 = (int64_t(s) * Hq + hq) * max_splits;
  float M = -INFINITY;
  for (int j = lane; j < nsplit; j += 64) M = fmaxf(M, part_ml[pi0 + j].x);
  M = wave_max(M);
  float Ls = 0.f;
  for (int j = lane; j < nsplit; j += 64) {
    const float2 ml = part_ml[pi0 + j];
    Ls += ml.y * exp2f(ml.x - M);
  }
  Ls = wave_sum(Ls);
  float a0 = 0.f, a1 = 0.f;
  for (int j = 0; j < nsplit; ++j) {
    const float w = exp2f(part_ml[pi0 + j].x - M);
    const float2 v = *reinterpret_cast<const float2*>(part_o + (pi0 + j) * 128 + 2 * lane);
    a0 += w * v.x;
    a1 += w * v.y;
  }
  const float inv = 1.f / Ls;
  const int64_t ob = (int64_t(s) * Hq + hq) * 128 + 2 * lane;
  if (out_bf16) {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + ob) = pack_bf16x2(a0 * inv, a1 * inv);
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(out) + ob) = make_float2(a0 * inv, a1 * inv);
  }
}

void launch_decode_mfma(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                        const int32_t* ctx_lens, const int32_t* block_table, int32_t mbps, int32_t batch,
                        int32_t Hq, int32_t Hkv, int32_t block_size, float scale, void* out, bool out_bf16,
                        int32_t split_tokens, int32_t max_splits, void* workspace, hipStream_t stream) {
  float* part_o = static_cast<float*>(workspace);
  float2* part_ml = reinterpret_cast<float2*>(part_o + int64_t(batch) * Hq * max_splits * 128);
  const dim3 grid(Hkv, max_splits, batch);
  const float sl2 = scale * kLog2e;
  const bool pow2 = (block_size & (block_size - 1)) == 0;
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kc = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(v_cache);
  if (pow2) {
    hipLaunchKernelGGL(decode_mfma_kernel<true>, grid, dim3(64), 0, stream, qp, q_stride, kc, vc, ctx_lens,
                       block_table, mbps, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), part_o, part_ml,
                       split_tokens, max_splits);
  } else {
    hipLaunchKernelGGL(decode_mfma_kernel<false>, grid, dim3(64), 0, stream, qp, q_stride, kc, vc, ctx_lens,
                       block_table, mbps, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), part_o, part_ml,
                       split_tokens, max_splits);
  }
  if (max_splits > 1) {
    hipLaunchKernelGGL(decode_reduce_kernel, dim3(Hq, batch), dim3(64), 0, stream, ctx_lens, part_o, part_ml, Hq,
                       split_tokens, max_splits, out, int(out_bf16));
  }
}

}  // namespace pa
