// Paged decode, balanced: a fixed grid of workers, each taking an equal slice of all (KV head, key) work.
//
// The work of a decode call is, per KV head, every key of every sequence. Keys of each sequence are padded to
// a multiple of 32 (padding keys are masked, and past the end the loads return zeros without touching memory),
// and the (KV head, sequence, key) triples are laid end to end: u = h * T' + cum[s] + t, with T' the padded
// total and cum the padded prefix sums. Worker w takes u in [w * chunk, (w + 1) * chunk), chunk a multiple of
// 32, so every worker reads the same number of K/V bytes whatever the mix of sequence lengths, and tiles stay
// 32-aligned inside their block. A worker walks its slice across sequence boundaries: a (sequence, KV head)
// pair wholly inside the slice is finished in place (normalised output written directly); a pair cut by the
// slice's ends leaves an unnormalised partial (m, l, O) in one of the worker's two slots, and the merge pass
// combines the partials of each cut pair with the log-sum-exp rule.
//
// Against a split of fixed size per sequence, this removes both the finishing imbalance of long splits on mixed
// lengths and the per-wave fixed costs of short ones. The per-tile work (32-key tiles of K and V through buffer
// descriptors, 16x16x32 bf16 MFMAs for scores and PV, online softmax) is the split kernel's.
#include "pa_decode_tile.h"

namespace pa {

constexpr int kStreamWaves = 4;                       // workers per workgroup (they share the prefix sums)
constexpr int kSlotFloats = 16 + 16 + 16 * 128;       // one partial: m[16], l[16], O[16][128] (G <= 16)

#ifndef PA_STREAM_NBUF
#define PA_STREAM_NBUF 2
#endif
constexpr int kStreamNBuf = PA_STREAM_NBUF;

// cum[s] = sum over i < s of the lengths rounded up to 32, lens[s] = the length (LDS; batch <= 4096). Each
// thread sums a run of sequences, the runs are scanned within each wave with shuffles and across the four waves
// through LDS.
__device__ __forceinline__ void stream_prefix(const int32_t* __restrict__ ctx_lens, int batch, int32_t* cum,
                                              int32_t* lens) {
  __shared__ int32_t wave_tot[kStreamWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int per = (batch + 64 * kStreamWaves - 1) / (64 * kStreamWaves);
  const int lo = min(batch, tid * per), hi = min(batch, lo + per);
  int32_t sum = 0;
  for (int s = lo; s < hi; ++s) {
    const int32_t L = ctx_lens[s];
    lens[s] = L;
    sum += (L + 31) & ~31;
  }
  int32_t inc = sum;  // inclusive scan over the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t v = __shfl_up(inc, off, 64);
    if (lane >= off) inc += v;
  }
  if (lane == 63) wave_tot[wv] = inc;
  __syncthreads();
  int32_t run = inc - sum;
  for (int w = 0; w < wv; ++w) run += wave_tot[w];
  if (tid == 0) cum[0] = 0;
  for (int s = lo; s < hi; ++s) {
    run += (lens[s] + 31) & ~31;
    cum[s + 1] = run;
  }
  __syncthreads();
}

template <bool kPow2>
__global__ __launch_bounds__(64 * kStreamWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_stream_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t batch, int32_t Hq, int32_t Hkv, int32_t bs,
    int32_t bs_shift, float scale_log2, void* __restrict__ out, int out_bf16, float* __restrict__ part,
    int32_t n_workers) {
  extern __shared__ int32_t smem[];
  int32_t* cum = smem;               // [batch + 1]
  int32_t* lens = smem + batch + 1;  // [batch]
  __shared__ __attribute__((aligned(16))) uint16_t vt_all[kStreamWaves][kDecKeys * kVRow];
  stream_prefix(ctx_lens, batch, cum, lens);

  const int64_t Tp = __builtin_amdgcn_readfirstlane(cum[batch]);
  const int64_t total = Tp * Hkv;
  const int64_t chunk = ((total + n_workers - 1) / n_workers + 31) & ~int64_t(31);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wid = int(blockIdx.x) * kStreamWaves + wave;
  int64_t u = int64_t(wid) * chunk;
  const int64_t u_end = min(total, u + chunk);

  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int li = lane & 15;
  const int64_t row_bytes = int64_t(Hkv) * 256;
  const LaneOffsets lo = {uint32_t(li * row_bytes + 16 * lg), uint32_t(lg * row_bytes + 16 * li)};
  const VTileLane vl = v_tile_lane(vt_all[wave], lane);
  int slot = 0;  // 0 for the slice's first pair, 1 for its last

  while (u < u_end) {
    const int h = int(u / Tp);
    const int r = int(u - int64_t(h) * Tp);
    int a = 0, b = batch;  // the pair's sequence: cum[a] <= r < cum[b]
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (cum[mid] <= r) a = mid; else b = mid;
    }
    // (LDS values are the same in every lane; readfirstlane tells the compiler they are wave-uniform)
    const int s = __builtin_amdgcn_readfirstlane(a);
    const int t0 = __builtin_amdgcn_readfirstlane(r - cum[s]);  // first key of this piece of the pair
    const int Lp = __builtin_amdgcn_readfirstlane(cum[s + 1] - cum[s]);
    const int L = __builtin_amdgcn_readfirstlane(lens[s]);
    const int seg = int(min(int64_t(Lp - t0), u_end - u));
    const int t1 = min(L, t0 + seg);                  // real keys of the piece end here
    const bool whole = t0 == 0 && seg == Lp;

    f32x4 o[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float lsum = 0.f;
    if (t0 < L) {  // the piece holds at least one real key (else it only covers padding)
      const int32_t* table = block_table + int64_t(s) * mbps;
      const char* kbase = reinterpret_cast<const char*>(k_cache + h * 128);
      const char* vbase = reinterpret_cast<const char*>(v_cache + h * 128);
      bf16x8 qb[4];
      load_q(qb, q + int64_t(s) * q_stride + int64_t(h * G) * 128, G, lane);
      KVTile buf[kStreamNBuf];
#pragma unroll
      for (int bb = 0; bb < kStreamNBuf; ++bb)
        load_tile<true, kPow2>(buf[bb], kbase, vbase, table, t0 + bb * kDecKeys, t0, t1, bs, bs_shift, row_bytes,
                               lo, lane);
      for (int g0 = t0; g0 < t1; g0 += kStreamNBuf * kDecKeys) {
#pragma unroll
        for (int bb = 0; bb < kStreamNBuf; ++bb) {
          const int base = g0 + bb * kDecKeys;
          f32x4 sc[2];
          tile_scores(buf[bb], qb, vl, sc);
          load_tile<true, kPow2>(buf[bb], kbase, vbase, table, base + kStreamNBuf * kDecKeys, t0, t1, bs,
                                 bs_shift, row_bytes, lo, lane);
          tile_softmax_pv(sc, base, t1, scale_log2, lane, vl, o, m, lsum);
        }
      }
    }
    lsum = xgroup16_sum(lsum);
    if (li < G) {
      // o[mt][i] is O^T[d = 16mt + 4lg + i][g = li]
      if (whole) {
        const float inv = 1.f / lsum;
        const int64_t ob = (int64_t(s) * Hq + h * G + li) * 128 + 4 * lg;
        if (out_bf16) {
          uint16_t* op = static_cast<uint16_t*>(out) + ob;
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const u32x2 w = {pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv),
                             pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv)};
            *reinterpret_cast<u32x2*>(op + 16 * mt) = w;
          }
        } else {
          float* op = static_cast<float*>(out) + ob;
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(op + 16 * mt) = o[mt] * inv;
        }
      } else {
        float* pp = part + (int64_t(wid) * 2 + slot) * kSlotFloats;
        if (lg == 0) {
          pp[li] = m;
          pp[16 + li] = lsum;
        }
        float* po = pp + 32 + li * 128 + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(po + 16 * mt) = o[mt];
      }
    }
    slot = 1;
    u += seg;
  }
}

// Merge of a (sequence, KV head) pair cut by worker slices: the workers w0..w1 whose slices meet the pair each
// left a partial (slot 0 if the pair is the first piece of the worker's slice, else slot 1). For each query
// head: M = max m_i, L = sum l_i 2^(m_i - M), O = sum O_i 2^(m_i - M) / L. One wave per (sequence, query head);
// pairs inside one slice return. The rows of the first eight partials are loaded together with every partial's
// (m, l) (lane j holds partial j's, 64 at a time), so most pairs take one round of dependent loads.
constexpr int kMergeEager = 8;

__global__ __launch_bounds__(64) void decode_stream_merge_kernel(const int32_t* __restrict__ ctx_lens, int32_t batch,
                                                                 int32_t Hq, int32_t Hkv,
                                                                 const float* __restrict__ part, int32_t n_workers,
                                                                 void* __restrict__ out, int out_bf16) {
  const int G = Hq / Hkv;
  const int h = int(blockIdx.x) / G;
  const int g = int(blockIdx.x) - h * G;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  int64_t before = 0, all = 0;
  for (int i = lane; i < batch; i += 64) {
    const int32_t Lp = (ctx_lens[i] + 31) & ~31;
    all += Lp;
    if (i < s) before += Lp;
  }
  for (int off = 32; off > 0; off >>= 1) {
    before += __shfl_xor(before, off, 64);
    all += __shfl_xor(all, off, 64);
  }
  const int64_t total = all * Hkv;
  const int64_t chunk = ((total + n_workers - 1) / n_workers + 31) & ~int64_t(31);
  const int64_t a = int64_t(h) * all + before;
  const int64_t b = a + ((ctx_lens[s] + 31) & ~31);
  const int w0 = int(a / chunk);
  const int w1 = int((b - 1) / chunk);
  if (w0 == w1) return;
  const int n = w1 - w0 + 1;  // partials of this pair (more than 64 when slices are short)
  const int first_slot = int64_t(w0) * chunk < a ? 1 : 0;
  auto part_of = [&](int j) {
    return part + (int64_t(w0 + j) * 2 + (j == 0 ? first_slot : 0)) * kSlotFloats;
  };
  float2 v[kMergeEager];
#pragma unroll
  for (int e = 0; e < kMergeEager; ++e)
    v[e] = e < n ? *reinterpret_cast<const float2*>(part_of(e) + 32 + g * 128 + 2 * lane) : make_float2(0.f, 0.f);
  float mj = lane < n ? part_of(lane)[g] : -INFINITY;
  float lj = lane < n ? part_of(lane)[16 + g] : 0.f;
  float M = mj;
  for (int j = lane + 64; j < n; j += 64) M = fmaxf(M, part_of(j)[g]);
  M = wave_max(M);
  float wj = lane < n ? exp2f(mj - M) : 0.f;
  float Ls = wave_sum(wj * lj);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int e = 0; e < kMergeEager; ++e) {
    const float w = __shfl(wj, e, 64);  // zero past n
    a0 += w * v[e].x;
    a1 += w * v[e].y;
  }
  for (int jb = 0; jb < n; jb += 64) {  // the remaining partials, 64 weights at a time
    const int nb = min(64, n - jb);
    if (jb > 0) {
      mj = lane < nb ? part_of(jb + lane)[g] : -INFINITY;
      lj = lane < nb ? part_of(jb + lane)[16 + g] : 0.f;
      wj = lane < nb ? exp2f(mj - M) : 0.f;
      Ls += wave_sum(wj * lj);
    }
    int k = jb == 0 ? kMergeEager : 0;
    for (; k + 4 <= nb; k += 4) {
      float2 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = *reinterpret_cast<const float2*>(part_of(jb + k + e) + 32 + g * 128 + 2 * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = __shfl(wj, k + e, 64);
        a0 += w * r[e].x;
        a1 += w * r[e].y;
      }
    }
    for (; k < nb; ++k) {
      const float2 r = *reinterpret_cast<const float2*>(part_of(jb + k) + 32 + g * 128 + 2 * lane);
      const float w = __shfl(wj, k, 64);
      a0 += w * r.x;
      a1 += w * r.y;
    }
  }
  const float inv = 1.f / Ls;
  const int64_t ob = (int64_t(s) * Hq + h * G + g) * 128 + 2 * lane;
  if (out_bf16) {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + ob) = pack_bf16x2(a0 * inv, a1 * inv);
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(out) + ob) = make_float2(a0 * inv, a1 * inv);
  }
}

size_t decode_stream_workspace_bytes(int32_t n_workers) {
  return size_t(n_workers) * 2 * kSlotFloats * sizeof(float);
}

void launch_decode_stream(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                          const int32_t* ctx_lens, const int32_t* block_table, int32_t mbps, int32_t batch,
                          int32_t Hq, int32_t Hkv, int32_t block_size, float scale, void* out, bool out_bf16,
                          int32_t n_workers, void* workspace, hipStream_t stream) {
  float* part = static_cast<float*>(workspace);
  const float sl2 = scale * kLog2e;
  const bool pow2 = (block_size & (block_size - 1)) == 0;
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const size_t lds = size_t(2 * batch + 1) * sizeof(int32_t);
  const dim3 grid(unsigned((n_workers + kStreamWaves - 1) / kStreamWaves));
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kc = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(v_cache);
  if (pow2) {
    hipLaunchKernelGGL(decode_stream_kernel<true>, grid, dim3(64 * kStreamWaves), lds, stream, qp, q_stride, kc, vc,
                       ctx_lens, block_table, mbps, batch, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), part,
                       n_workers);
  } else {
    hipLaunchKernelGGL(decode_stream_kernel<false>, grid, dim3(64 * kStreamWaves), lds, stream, qp, q_stride, kc,
                       vc, ctx_lens, block_table, mbps, batch, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16),
                       part, n_workers);
  }
  hipLaunchKernelGGL(decode_stream_merge_kernel, dim3(Hq, batch), dim3(64), 0, stream, ctx_lens, batch, Hq, Hkv,
                     part, n_workers, out, int(out_bf16));
}

}  // namespace pa
