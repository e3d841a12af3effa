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
#include "pa_decode_tile.h"

namespace pa {

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 2
#endif

template <bool kAligned, bool kPow2, int kHeadsPerWG>
__global__ __launch_bounds__(64 * kHeadsPerWG) __attribute__((amdgpu_waves_per_eu(PA_DECODE_WAVES, PA_DECODE_WAVES))) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t Hq, int32_t Hkv, int32_t bs, int32_t bs_shift,
    float scale_log2, void* __restrict__ out, int out_bf16, float* __restrict__ part_o,
    float2* __restrict__ part_ml, int32_t split_tokens, int32_t max_splits, int32_t n_seq) {
  // Flat grid, KV head fastest: workgroup i takes head group i % (Hkv / heads per workgroup) of work item
  // (sequence, split) i / (Hkv / heads per workgroup). The heads of one work item are dispatched back to back
  // and the hardware's round-robin over the 8 XCDs gives every XCD the same share of every work item.
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));  // wave-uniform
  const int n_hg = Hkv / kHeadsPerWG;
  const int h = int(blockIdx.x % n_hg) * kHeadsPerWG + wave;
  const int work = int(blockIdx.x / n_hg);
  const int split = work % max_splits;
  const int s = work / max_splits;
  if (s >= n_seq) return;
  const int L = ctx_lens[s];
  const int nsplit = (L + split_tokens - 1) / split_tokens;
  if (split >= nsplit) return;
  const int t0 = split * split_tokens;
  const int t1 = min(L, t0 + split_tokens);
  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int li = lane & 15;
  const int32_t* table = block_table + int64_t(s) * mbps;
  const int64_t row_bytes = int64_t(Hkv) * 256;  // bytes between consecutive slots
  const char* kbase = reinterpret_cast<const char*>(k_cache + h * 128);
  const char* vbase = reinterpret_cast<const char*>(v_cache + h * 128);
  const LaneOffsets lo = {uint32_t(li * row_bytes + 16 * lg), uint32_t(lg * row_bytes + 16 * li)};

  bf16x8 qb[4];
  load_q(qb, q + int64_t(s) * q_stride + int64_t(h * G) * 128, G, lane);

  // then start the first tiles' loads (Q is loaded first so that waiting for a tile also covers Q)
  KVTile buf[kNBuf];
#pragma unroll
  for (int b = 0; b < kNBuf; ++b)
    load_tile<kAligned, kPow2>(buf[b], kbase, vbase, table, t0 + b * kDecKeys, t0, t1, bs, bs_shift, row_bytes,
                               lo, lane);

  // one V tile per wave; each wave only touches its own tile, and LDS accesses of one wave complete in order
  __shared__ __attribute__((aligned(16))) uint16_t vt_all[kHeadsPerWG][kDecKeys * kVRow];
  const VTileLane vl = v_tile_lane(vt_all[wave], lane);

  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  for (int g0 = t0; g0 < t1; g0 += kNBuf * kDecKeys) {
#pragma unroll
    for (int b = 0; b < kNBuf; ++b) {
      // Every step runs, also for a tile past the end (only possible in the last group, and only on the
      // aligned path): its loads return zeros without touching memory, its scores are -inf and it leaves
      // m, l and O unchanged. Unconditional steps keep the count of loads in flight the same on every path.
      const int base = g0 + b * kDecKeys;
      f32x4 sc[2];
      tile_scores(buf[b], qb, vl, sc);
      // the registers of this tile are free: start loading the tile kNBuf tiles ahead into them
      load_tile<kAligned, kPow2>(buf[b], kbase, vbase, table, base + kNBuf * kDecKeys, t0, t1, bs, bs_shift,
                                 row_bytes, lo, lane);
      tile_softmax_pv(sc, base, t1, scale_log2, lane, vl, o, m, lsum);
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
// O = sum O_i 2^(m_i - M) / L. Sequences that fit in one split were finished by the first pass. Lane j first
// holds split j's weight; the partial rows are then read four splits at a time so their loads overlap.
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
  const float* po = part_o + pi0 * 128 + 2 * lane;
  float a0 = 0.f, a1 = 0.f;
  for (int j0 = 0; j0 < nsplit; j0 += 64) {
    const float wl = j0 + lane < nsplit ? exp2f(part_ml[pi0 + j0 + lane].x - M) : 0.f;
    const int n = min(64, nsplit - j0);
    int j = 0;
    for (; j + 4 <= n; j += 4) {
      float2 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const float2*>(po + int64_t(j0 + j + u) * 128);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = __shfl(wl, j + u, 64);
        a0 += w * v[u].x;
        a1 += w * v[u].y;
      }
    }
    for (; j < n; ++j) {
      const float2 v = *reinterpret_cast<const float2*>(po + int64_t(j0 + j) * 128);
      const float w = __shfl(wl, j, 64);
      a0 += w * v.x;
      a1 += w * v.y;
    }
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
  const float sl2 = scale * kLog2e;
  // the KV heads of one (sequence, split) run as the waves of one workgroup, so each token row of the cache is
  // read whole (all heads) by one CU at about the same time
#ifndef PA_DECODE_HPW
#define PA_DECODE_HPW 1
#endif
  const int hpw = (Hkv % PA_DECODE_HPW == 0) ? PA_DECODE_HPW : (Hkv % 4 == 0 ? 4 : 1);
  const bool pow2 = (block_size & (block_size - 1)) == 0;
  const bool aligned = block_size % kDecKeys == 0;  // split_tokens is a multiple of 32 too
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kc = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(v_cache);
  const int n_hg = Hkv / hpw;
  const int64_t n_work = int64_t(batch) * max_splits;
  const dim3 grid(unsigned(n_hg * n_work));
#define PA_LAUNCH_DEC(A, P)                                                                                     \
  if (hpw == 8)                                                                                                 \
    hipLaunchKernelGGL((decode_mfma_kernel<A, P, 8>), grid, dim3(512), 0, stream, qp, q_stride, kc, vc,          \
                       ctx_lens, block_table, mbps, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), part_o,  \
                       part_ml, split_tokens, max_splits, batch);                                                \
  else if (hpw == 4)                                                                                            \
    hipLaunchKernelGGL((decode_mfma_kernel<A, P, 4>), grid, dim3(256), 0, stream, qp, q_stride, kc, vc,          \
                       ctx_lens, block_table, mbps, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), part_o,  \
                       part_ml, split_tokens, max_splits, batch);                                                \
  else                                                                                                          \
    hipLaunchKernelGGL((decode_mfma_kernel<A, P, 1>), grid, dim3(64), 0, stream, qp, q_stride, kc, vc, ctx_lens, \
                       block_table, mbps, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), part_o, part_ml,   \
                       split_tokens, max_splits, batch)
  if (aligned && pow2) PA_LAUNCH_DEC(true, true);
  else if (aligned) PA_LAUNCH_DEC(true, false);
  else if (pow2) PA_LAUNCH_DEC(false, true);
  else PA_LAUNCH_DEC(false, false);
#undef PA_LAUNCH_DEC
  if (max_splits > 1) {
    hipLaunchKernelGGL(decode_reduce_kernel, dim3(Hq, batch), dim3(64), 0, stream, ctx_lens, part_o, part_ml, Hq,
                       split_tokens, max_splits, out, int(out_bf16));
  }
}

}  // namespace pa
