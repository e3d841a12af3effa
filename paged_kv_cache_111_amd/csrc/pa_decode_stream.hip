// Paged decode, balanced: a fixed grid of workers, each taking an equal slice of all (KV head, key) work.
//
// The work of a decode call is, per KV head, every key of every sequence. Keys of each sequence are padded to
// a multiple of 32 (padding keys are masked, and past the end the loads return zeros without touching memory),
// and the (sequence, key) pairs are laid end to end: u = cum[s] + t, with cum the padded prefix sums. Workers
// come in groups of Hkv: worker w = g * Hkv + h takes KV head h of u in [g * chunk, (g + 1) * chunk), chunk a
// multiple of 32, so every worker reads the same number of K/V bytes whatever the mix of sequence lengths, tiles
// stay 32-aligned inside their block, and the Hkv head pieces of a token's cache row are read by the workers of
// one group, started together, at about the same time (whole rows in a short window: measured 2% faster than
// laying the heads end to end, where a row's heads are read by workers far apart). A worker walks its slice
// across sequence boundaries: a (sequence, KV head) pair wholly inside the slice is finished in place
// (normalised output written directly); a pair cut by the slice's ends leaves an unnormalised partial (m, l, O)
// in one of the worker's two slots, and the merge pass combines the partials of each cut pair with the
// log-sum-exp rule.
//
// Appending (the new token's K and V given with the cached lengths): each pair's length is its cached length plus
// one, and its new key is the last one. The worker whose slice holds that key, and no other, reads the key's
// tile, so before its first load it writes that head's piece of the new K and V rows to the key's slot (found in
// the block table) and then reads it back with the tile: the store and the attention of a decode step take the
// same two launches as the attention alone.
//
// Against a split of fixed size per sequence, this removes both the finishing imbalance of long splits on mixed
// lengths and the per-wave fixed costs of short ones. The per-tile work (32-key tiles of K and V through buffer
// descriptors, 16x16x32 bf16 MFMAs for scores and PV, online softmax) is the split kernel's.
#include "pa_decode_tile.h"
#include "pa_dpp.h"

namespace pa {

constexpr int kStreamWaves = 4;                       // workers per workgroup (they share the prefix sums)
constexpr int kSlotFloats = kStreamSlotFloats;       // one partial: m[16], l[16], O[16][128] (G <= 16)
#ifndef PA_STREAM_MIN_CHUNK
#define PA_STREAM_MIN_CHUNK 128
#endif
constexpr int64_t kMinChunk = PA_STREAM_MIN_CHUNK;    // keys per slice at least (a multiple of 32): on small calls
                                                      // fewer workers, and fewer partials per cut pair

// Keys per worker slice: an equal share of the padded total, rounded up to 32, at least kMinChunk. The decode
// pass and the merge compute it the same way.
__device__ __forceinline__ int64_t stream_chunk(int64_t total, int32_t n_workers) {
  return max(((total + n_workers - 1) / n_workers + 31) & ~int64_t(31), kMinChunk);
}

// Tiles whose loads are in flight per worker. With the non-temporal policy on the K/V loads one tile ahead
// measured 1% faster than two on the 0.6B mix (the same on long contexts), in 173 registers instead of 247.
#ifndef PA_STREAM_NBUF
#define PA_STREAM_NBUF 1
#endif
constexpr int kStreamNBuf = PA_STREAM_NBUF;

// cum[s] = sum over i < s of the lengths rounded up to 32, lens[s] = the length (LDS; batch <= 4096). Each
// thread sums a run of sequences, the runs are scanned within each wave by DPP and across the four waves
// through LDS.
__device__ __forceinline__ void stream_prefix(const int32_t* __restrict__ ctx_lens, int32_t len_add, int batch,
                                              int32_t* cum, int32_t* lens) {
  __shared__ int32_t wave_tot[kStreamWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int per = (batch + 64 * kStreamWaves - 1) / (64 * kStreamWaves);
  const int lo = min(batch, tid * per), hi = min(batch, lo + per);
  int32_t sum = 0;
  for (int s = lo; s < hi; ++s) {
    const int32_t L = ctx_lens[s] + len_add;
    lens[s] = L;
    sum += (L + 31) & ~31;
  }
  const int32_t inc = dpp_incl_scan_i(sum);  // inclusive scan over the wave
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

// Position of a 32-key tile of a worker's walk: its KV head h (fixed for the worker), sequence s, first key t of
// the tile, the sequence's length L and its length padded to 32 (all wave-uniform).
struct StreamCursor {
  int h, s, t, L, Lp;
};

// Steps to the next tile: the next 32 keys of the sequence, or key 0 of the next sequence with keys. Callers step
// only while another tile of the slice follows, so a sequence with keys lies ahead; the scan over zero-length
// sequences is bounded by the batch all the same.
__device__ __forceinline__ void cursor_next(StreamCursor& c, const int32_t* lens, int batch) {
  c.t += kDecKeys;
  if (c.t >= c.Lp) {
    c.t = 0;
    for (int k = 0; k < batch; ++k) {
      if (++c.s == batch) c.s = 0;  // not reached: a slice ends inside the batch
      c.L = __builtin_amdgcn_readfirstlane(lens[c.s]);
      c.Lp = (c.L + 31) & ~31;
      if (c.Lp > 0) break;
    }
  }
}

// Q^T of a (sequence, KV head) pair as the score MFMA's B operand (lane: Q[g = li][d = 8lg + 32ks .. +7]),
// read through a buffer descriptor sized to the G rows so lanes li >= G get zeros with no branch.
__device__ __forceinline__ void load_q_rsrc(bf16x8 (&qb)[4], const uint16_t* qrow0, int G, int lane) {
  const int lg = lane >> 4;
  const int li = lane & 15;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(qrow0), 0, G * 256, 0x00020000);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qb[ks] = as_bf16x8(__builtin_amdgcn_raw_buffer_load_b128(r, li * 256 + 16 * lg + 64 * ks, 0, 0));
}

// A worker's slice is a run of whole 32-key tiles (slice ends and padded lengths are multiples of 32), walked as
// one stream: the loads of tile i + NBUF (and the Q of tile i + 1's pair) are issued while tile i is computed,
// whether or not the tiles belong to the same (sequence, KV head) pair, so the loads stay in flight across pair
// boundaries. When the tile ends a piece (the end of its pair, or of the slice) the piece is finished: a pair
// held whole is normalised into the output; a cut pair leaves (m, l, O) in partial slot 0 (the slice's first
// piece) or 1 (its last).
template <bool kPow2>
__global__ __launch_bounds__(64 * kStreamWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_stream_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, uint16_t* __restrict__ k_cache,
    uint16_t* __restrict__ v_cache, const int32_t* __restrict__ ctx_lens,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t batch, int32_t Hq, int32_t Hkv, int32_t bs,
    int32_t bs_shift, float scale_log2, void* __restrict__ out, int out_bf16, float* __restrict__ part,
    int32_t n_workers, const uint16_t* __restrict__ k_new, int64_t k_new_stride, const uint16_t* __restrict__ v_new,
    int64_t v_new_stride) {
  extern __shared__ int32_t smem[];
  int32_t* cum = smem;               // [batch + 1]
  int32_t* lens = smem + batch + 1;  // [batch]
  __shared__ __attribute__((aligned(16))) uint16_t vt_all[kStreamWaves][kDecKeys * kVRow];
  const int32_t len_add = k_new ? 1 : 0;  // appending: ctx_lens holds the cached lengths, the new key comes after
  stream_prefix(ctx_lens, len_add, batch, cum, lens);

  const int64_t Tp = __builtin_amdgcn_readfirstlane(cum[batch]);
  const int n_groups = n_workers / Hkv;
  const int64_t chunk = stream_chunk(Tp, n_groups);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wid = int(blockIdx.x) * kStreamWaves + wave;
  const int grp = wid / Hkv;  // the Hkv workers of a group share a key range, one KV head each
  if (grp >= n_groups) return;
  const int64_t u0 = int64_t(grp) * chunk;
  const int64_t u1 = min(Tp, u0 + chunk);
  if (u0 >= u1) return;
  const int n_tiles = int((u1 - u0) / kDecKeys);

  const int G = Hq / Hkv;
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int li = lane & 15;
  const int64_t row_bytes = int64_t(Hkv) * 256;
  const LaneOffsets lo = {uint32_t(li * row_bytes + 16 * lg), uint32_t(lg * row_bytes + 16 * li)};
  const VTileLane vl = v_tile_lane(vt_all[wave], lane);

  StreamCursor cc;  // the tile being computed
  {
    const int h = wid - grp * Hkv;
    const int r = int(u0);
    int a = 0, b = batch;  // cum[a] <= r < cum[a + 1]
    while (b - a > 1) {
      const int mid = (a + b) >> 1;
      if (cum[mid] <= r) a = mid; else b = mid;
    }
    cc.h = h;
    cc.s = __builtin_amdgcn_readfirstlane(a);
    cc.t = __builtin_amdgcn_readfirstlane(r - cum[cc.s]);
    cc.L = __builtin_amdgcn_readfirstlane(lens[cc.s]);
    cc.Lp = (cc.L + 31) & ~31;
  }
  StreamCursor lc = cc;  // the next tile to load

  if (k_new) {
    // Appending: the new token of a pair is its last key, and only the worker whose slice holds that key reads
    // its row, so that worker writes the pair's head of the new K and V rows to their slot before its first
    // tile loads (lanes 0-15: 16 bytes of K each, lanes 16-31: of V). Pairs overlapping the slice are walked
    // from its first one.
    StreamCursor pc = cc;
    int64_t pu = u0 - pc.t;  // where the current pair starts
    for (int it = 0; it <= batch; ++it) {
      const int64_t last = pu + pc.L - 1;
      if (last >= u0 && last < u1 && lane < 32) {
        const int pos = pc.L - 1;
        const int blk = kPow2 ? (pos >> bs_shift) : (pos / bs);
        const int64_t slot = int64_t(block_table[int64_t(pc.s) * mbps + blk]) * bs + (pos - blk * bs);
        if (slot >= 0) {
          const bool is_v = lane >= 16;
          const int64_t e = int64_t(pc.h) * 128 + 8 * (lane & 15);
          const u32x4 x = *reinterpret_cast<const u32x4*>(
              is_v ? v_new + int64_t(pc.s) * v_new_stride + e : k_new + int64_t(pc.s) * k_new_stride + e);
          *reinterpret_cast<u32x4*>((is_v ? v_cache : k_cache) + slot * (int64_t(Hkv) * 128) + e) = x;
        }
      }
      pu += pc.Lp;
      if (pu >= u1) break;
      for (int k = 0; k < batch; ++k) {  // the next pair with keys
        if (++pc.s == batch) pc.s = 0;
        pc.L = __builtin_amdgcn_readfirstlane(lens[pc.s]);
        pc.Lp = (pc.L + 31) & ~31;
        if (pc.Lp > 0) break;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");  // the rows are written before this wave reads them
  }

  auto qrow = [&](const StreamCursor& c) { return q + int64_t(c.s) * q_stride + int64_t(c.h * G) * 128; };
  // Loads the tile at lc; a tile index past the slice gets a zero-sized descriptor at lc's (real) tile.
  auto issue = [&](KVTile& t, bool real) {
    load_tile<true, kPow2>(t, reinterpret_cast<const char*>(k_cache + lc.h * 128),
                           reinterpret_cast<const char*>(v_cache + lc.h * 128), block_table + int64_t(lc.s) * mbps,
                           lc.t, lc.t, real ? lc.L : lc.t, bs, bs_shift, row_bytes, lo, lane);
  };

  bf16x8 qb[4];
  load_q_rsrc(qb, qrow(cc), G, lane);
  KVTile buf[kStreamNBuf];
#pragma unroll
  for (int bb = 0; bb < kStreamNBuf; ++bb) {
    issue(buf[bb], bb < n_tiles);
    if (bb + 1 < n_tiles) cursor_next(lc, lens, batch);
  }

  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;
  int slot = 0;
  bool from_start = cc.t == 0;  // the current piece starts at its pair's first key

  // Every pass of the body issues the same loads in the same order (past the slice they are zero-sized), and
  // only the compute is skipped there, so the wait counts before each tile are the same on every path.
  for (int i0 = 0; i0 < n_tiles; i0 += kStreamNBuf) {
#pragma unroll
    for (int bb = 0; bb < kStreamNBuf; ++bb) {
      const int i = i0 + bb;
      const bool active = i < n_tiles;
      const bool pair_end = cc.t + kDecKeys >= cc.Lp;
      const bool piece_end = active && (pair_end || i + 1 == n_tiles);
      StreamCursor nc = cc;
      if (i + 1 < n_tiles) cursor_next(nc, lens, batch);

      f32x4 sc[2];
      if (active) tile_scores(buf[bb], qb, vl, sc);
      bf16x8 qn[4];
      load_q_rsrc(qn, qrow(nc), G, lane);
      const int j = i + kStreamNBuf;
      issue(buf[bb], j < n_tiles);
      if (j + 1 < n_tiles) cursor_next(lc, lens, batch);
      if (active) tile_softmax_pv(sc, cc.t, cc.L, scale_log2, lane, vl, o, m, lsum);

      if (piece_end) {
        const float ls = xgroup16_sum(lsum);
        if (li < G) {
          // o[mt][i] is O^T[d = 16mt + 4lg + i][g = li]
          if (from_start && pair_end) {
            const float inv = 1.f / ls;
            const int64_t ob = (int64_t(cc.s) * Hq + cc.h * G + li) * 128 + 4 * lg;
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
              pp[16 + li] = ls;
            }
            float* po = pp + 32 + li * 128 + 4 * lg;
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(po + 16 * mt) = o[mt];
          }
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        m = -INFINITY;
        lsum = 0.f;
        slot = 1;
        from_start = true;
      }
      cc = nc;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[ks] = qn[ks];
    }
  }
}

// Merge of a (sequence, KV head) pair cut by worker slices: the workers w0..w1 whose slices meet the pair each
// left a partial (slot 0 if the pair is the first piece of the worker's slice, else slot 1). For each query
// head: M = max m_i, L = sum l_i 2^(m_i - M), O = sum O_i 2^(m_i - M) / L. One wave per (sequence, query head);
// pairs inside one slice return. The rows of the first eight partials are loaded together with every partial's
// (m, l) (lane j holds partial j's, 64 at a time), so most pairs take one round of dependent loads; further
// rows are read eight at a time.
constexpr int kMergeEager = 8;


__global__ __launch_bounds__(64) void decode_stream_merge_kernel(const int32_t* __restrict__ ctx_lens,
                                                                 int32_t len_add, int32_t batch, int32_t Hq,
                                                                 int32_t Hkv, const float* __restrict__ part,
                                                                 int32_t n_workers, void* __restrict__ out,
                                                                 int out_bf16) {
  const int G = Hq / Hkv;
  const int h = int(blockIdx.x) / G;
  const int g = int(blockIdx.x) - h * G;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  // padded lengths sum below 2^31 (a condition of the balanced decode)
  int before32 = 0, all32 = 0;
  for (int i = lane; i < batch; i += 64) {
    const int32_t Lp = (ctx_lens[i] + len_add + 31) & ~31;
    all32 += Lp;
    if (i < s) before32 += Lp;
  }
  const int64_t before = dpp_sum_i(before32), all = dpp_sum_i(all32);
  const int64_t chunk = stream_chunk(all, n_workers / Hkv);
  const int64_t a = before;
  const int64_t b = a + ((ctx_lens[s] + len_add + 31) & ~31);
  if (b == a) return;  // no keys (lengths are documented >= 1)
  const int w0 = int(a / chunk);  // groups whose key ranges meet the sequence; worker w * Hkv + h holds head h
  const int w1 = int((b - 1) / chunk);
  if (w0 == w1) return;
  const int n = w1 - w0 + 1;  // partials of this pair (more than 64 when slices are short)
  const int first_slot = int64_t(w0) * chunk < a ? 1 : 0;
  auto part_of = [&](int j) {
    return part + ((int64_t(w0 + j) * Hkv + h) * 2 + (j == 0 ? first_slot : 0)) * kSlotFloats;
  };
  float2 v[kMergeEager];
#pragma unroll
  for (int e = 0; e < kMergeEager; ++e)
    v[e] = e < n ? *reinterpret_cast<const float2*>(part_of(e) + 32 + g * 128 + 2 * lane) : make_float2(0.f, 0.f);
  float mj = lane < n ? part_of(lane)[g] : -INFINITY;
  float lj = lane < n ? part_of(lane)[16 + g] : 0.f;
  float M = mj;
  for (int j = lane + 64; j < n; j += 64) M = fmaxf(M, part_of(j)[g]);
  M = dpp_max_f(M);
  float wj = lane < n ? exp2f(mj - M) : 0.f;
  float Ls = dpp_sum_f(wj * lj);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int e = 0; e < kMergeEager; ++e) {
    const float w = lane_of(wj, e);  // zero past n
    a0 += w * v[e].x;
    a1 += w * v[e].y;
  }
  for (int jb = 0; jb < n; jb += 64) {  // the remaining partials, 64 weights at a time
    const int nb = min(64, n - jb);
    if (jb > 0) {
      mj = lane < nb ? part_of(jb + lane)[g] : -INFINITY;
      lj = lane < nb ? part_of(jb + lane)[16 + g] : 0.f;
      wj = lane < nb ? exp2f(mj - M) : 0.f;
      Ls += dpp_sum_f(wj * lj);
    }
    int k = jb == 0 ? kMergeEager : 0;
    for (; k + 8 <= nb; k += 8) {
      float2 r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = *reinterpret_cast<const float2*>(part_of(jb + k + e) + 32 + g * 128 + 2 * lane);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = lane_of(wj, k + e);
        a0 += w * r[e].x;
        a1 += w * r[e].y;
      }
    }
    for (; k < nb; ++k) {
      const float2 r = *reinterpret_cast<const float2*>(part_of(jb + k) + 32 + g * 128 + 2 * lane);
      const float w = lane_of(wj, k);
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

void launch_decode_stream(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                          const int32_t* ctx_lens, const int32_t* block_table, int32_t mbps, int32_t batch,
                          int32_t Hq, int32_t Hkv, int32_t block_size, float scale, void* out, bool out_bf16,
                          int32_t n_workers, void* workspace, hipStream_t stream, const void* k_new,
                          int64_t k_new_stride, const void* v_new, int64_t v_new_stride) {
  float* part = static_cast<float*>(workspace);
  const float sl2 = scale * kLog2e;
  const bool pow2 = (block_size & (block_size - 1)) == 0;
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const size_t lds = size_t(2 * batch + 1) * sizeof(int32_t);
  // whole groups of Hkv workers (the caller guarantees Hkv <= n_workers); the kernel and the merge derive the
  // group count from this number the same way
  n_workers = (n_workers / Hkv) * Hkv;
  const dim3 grid(unsigned((n_workers + kStreamWaves - 1) / kStreamWaves));
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  // the caches are written only when appending (k_new given); pa_decode passes them as read-only
  uint16_t* kc = static_cast<uint16_t*>(const_cast<void*>(k_cache));
  uint16_t* vc = static_cast<uint16_t*>(const_cast<void*>(v_cache));
  const uint16_t* kn = static_cast<const uint16_t*>(k_new);
  const uint16_t* vn = static_cast<const uint16_t*>(v_new);
  if (pow2) {
    hipLaunchKernelGGL(decode_stream_kernel<true>, grid, dim3(64 * kStreamWaves), lds, stream, qp, q_stride, kc, vc,
                       ctx_lens, block_table, mbps, batch, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), part,
                       n_workers, kn, k_new_stride, vn, v_new_stride);
  } else {
    hipLaunchKernelGGL(decode_stream_kernel<false>, grid, dim3(64 * kStreamWaves), lds, stream, qp, q_stride, kc,
                       vc, ctx_lens, block_table, mbps, batch, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16),
                       part, n_workers, kn, k_new_stride, vn, v_new_stride);
  }
  hipLaunchKernelGGL(decode_stream_merge_kernel, dim3(Hq, batch), dim3(64), 0, stream, ctx_lens,
                     int32_t(k_new ? 1 : 0), batch, Hq, Hkv, part, n_workers, out, int(out_bf16));
}

}  // namespace pa
