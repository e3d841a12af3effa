// Paged varlen causal prefill on the matrix cores: bf16, head_dim 128.
//
// Workgroup = (sequence s, query head h, tile of 128 query rows); four waves of 32 rows each. Keys are walked in
// tiles of 32 gathered through the block table into LDS (row-major, both K and V), shared by the four waves:
//   S^T[key, q] = K[key, :] . Q[q, :]      32x32x16 MFMA, A = K rows from LDS, B = Q^T kept in registers
//   O^T[d, q]  += V^T[d, key] P^T[key, q]  32x32x16 MFMA, A = V^T via the LDS transpose read, B = P^T kept in
//                                           the registers the score MFMA left it in
// With scores transposed, each lane owns one query column, so the row max and sum need one exchange between
// the two wave halves per tile. The key -> k-slot assignment of the second product follows the score layout
// (lane half hh holds keys 8j + 4hh .. +3), so P^T needs no data movement.
//
// Causality follows absolute positions: the q_len new rows of a sequence with k_len keys sit at positions
// k_len - q_len .. k_len - 1 (a chunk continues after the cached prefix, "Nano-vLLM 源码逐行解析 第2篇",
// sequence.py), and a row at position p sees keys 0..p. Keys past k_len are never loaded (zero in LDS, -inf
// scores), so cache contents there cannot reach the output.
//
// Workgroup order: the flat grid is renumbered so that the workgroups the hardware sends to one XCD (every
// eighth) get consecutive logical ids, and the logical order is (KV head, sequence, query tile from the last,
// query head in the group). The G query heads that share a KV head, and the query tiles of that head, then run
// on one XCD and read the same K/V through its L2; the heaviest (last) tiles of each sequence start first.
#include "pa_launch.h"

namespace pa {

constexpr int kPreRows = 128;     // query rows per workgroup
constexpr int kPreKeys = 32;      // keys per tile
constexpr int kPreThreads = 256;  // four waves
constexpr int kKRow = 128 + 8;    // LDS row stride in bf16 elements (272 bytes)

template <bool kPow2>
__device__ __forceinline__ int64_t pf_slot(const int32_t* table, int key, int bs, int bs_shift) {
  if (kPow2) return int64_t(table[key >> bs_shift]) * bs + (key & (bs - 1));
  const int blk = key / bs;
  return int64_t(table[blk]) * bs + (key - blk * bs);
}

template <bool kPow2>
__global__ __launch_bounds__(kPreThreads) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t batch, int32_t Hq, int32_t Hkv, int32_t bs,
    int32_t bs_shift, float scale_log2, void* __restrict__ out, int out_bf16, int32_t n_qtiles, int32_t n_work) {
  // ---- which (KV head, sequence, query tile, query head) this workgroup computes
  const int per_xcd = (int(gridDim.x) + 7) >> 3;
  const int logical = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (logical >= n_work) return;
  const int G = Hq / Hkv;
  const int gi = logical % G;
  int rest = logical / G;
  const int qtile = n_qtiles - 1 - rest % n_qtiles;
  rest /= n_qtiles;
  const int s = rest % batch;
  const int kvh = rest / batch;
  const int h = kvh * G + gi;

  const int q0 = cu_q[s];
  const int q_len = cu_q[s + 1] - q0;
  const int row0 = qtile * kPreRows;
  if (row0 >= q_len) return;
  const int k_len = cu_k[s + 1] - cu_k[s];
  const int past = k_len - q_len;  // position of row 0
  const int row_end = min(q_len, row0 + kPreRows);
  const int n_keys = past + row_end;  // keys needed by the last row of the tile

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 31;   // query column owned by this lane
  const int hh = lane >> 5;   // wave half
  const int my_row = row0 + 32 * w + lr;
  const int wave_last_row = min(q_len - 1, row0 + 32 * w + 31);
  const int wave_keys = row0 + 32 * w < q_len ? past + wave_last_row + 1 : 0;
  const int32_t* table = block_table + int64_t(s) * mbps;
  const int64_t row_stride = int64_t(Hkv) * 128;

  // B operand of the score MFMA: lane holds Q[my_row][8hh + 16ks .. +7], ks = 0..7
  bf16x8 qb[8];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp = q + int64_t(q0 + my_row) * q_stride + int64_t(h) * 128 + 8 * hh;
    const bool ok = my_row < q_len;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = as_bf16x8(ok ? ld16(qp + 16 * ks) : z);
  }

  __shared__ __attribute__((aligned(16))) uint16_t kt[kPreKeys * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kPreKeys * kKRow];

  f32x16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
  float m = -INFINITY;
  float lsum = 0.f;
  const int my_pos = past + my_row;

  const uint16_t* kbase = k_cache + kvh * 128;
  const uint16_t* vbase = v_cache + kvh * 128;

  for (int kb = 0; kb < n_keys; kb += kPreKeys) {
    // ---- cooperative gather of the K and V tiles: 2 x 512 pieces of 16 bytes; piece c -> key c/16, d 8(c%16)
    {
      const u32x4 z = {0u, 0u, 0u, 0u};
      u32x4 kv[2], vv[2];
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int c = it * kPreThreads + tid;
        const int key = kb + (c >> 4);
        if (key < k_len) {
          const int64_t off = pf_slot<kPow2>(table, key, bs, bs_shift) * row_stride + 8 * (c & 15);
          kv[it] = ld16(kbase + off);
          vv[it] = ld16(vbase + off);
        } else {
          kv[it] = z;
          vv[it] = z;
        }
      }
      __syncthreads();  // previous tile fully consumed
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int c = it * kPreThreads + tid;
        st16(&kt[(c >> 4) * kKRow + 8 * (c & 15)], kv[it]);
        st16(&vt[(c >> 4) * kKRow + 8 * (c & 15)], vv[it]);
      }
      __syncthreads();
    }
    if (kb >= wave_keys) continue;  // every row of this wave is before this tile

    // ---- S^T = K Q^T: sc[i] is key kb + 8(i/4) + 4hh + (i%4), query column lr
    f32x16 sc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = 0.f;
    const uint16_t* ka = &kt[lr * kKRow + 8 * hh];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sc = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(ka + 16 * ks)), qb[ks], sc);

    float mx = -INFINITY;
    const bool need_mask = kb + kPreKeys - 1 > past + row0 + 32 * w;  // some key of the tile is after some row
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb + 8 * (i >> 2) + 4 * hh + (i & 3);
      float v = sc[i] * scale_log2;
      if (need_mask && key > my_pos) v = -INFINITY;
      sc[i] = v;
      mx = fmaxf(mx, v);
    }
    mx = xhalf_max(mx);
    const float mn = fmaxf(m, mx);  // finite: key 0 is visible to every row
    const float alpha = exp2f(m - mn);
    m = mn;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = exp2f(sc[i] - mn);
      psum += sc[i];
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 pw = {pack_bf16x2(sc[8 * kk + 0], sc[8 * kk + 1]), pack_bf16x2(sc[8 * kk + 2], sc[8 * kk + 3]),
                        pack_bf16x2(sc[8 * kk + 4], sc[8 * kk + 5]), pack_bf16x2(sc[8 * kk + 6], sc[8 * kk + 7])};
      pb[kk] = as_bf16x8(pw);
    }

    // ---- O^T += V^T P^T. Lane group g4 = lane/16: half hh = g4/2, d offset 16(g4%2). For k-step kk the lane's
    // slots 0..3 are keys 16kk + 4hh + 0..3 and slots 4..7 keys 16kk + 8 + 4hh + 0..3.
    const int li = lane & 15;
    const int g4 = lane >> 4;
    const uint16_t* vr = &vt[(4 * (g4 >> 1) + (li >> 2)) * kKRow + 16 * (g4 & 1) + 4 * (li & 3)];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const i16x4 a0 = lds_read_tr16(vr + (16 * kk) * kKRow + 32 * mt);
        const i16x4 a1 = lds_read_tr16(vr + (16 * kk + 8) * kKRow + 32 * mt);
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = mfma32x32x16(av, pb[kk], o[mt]);
      }
    }
  }

  if (my_row >= q_len) return;
  lsum = xhalf_sum(lsum);
  const float inv = 1.f / lsum;
  // o[mt][i] is O^T[d = 32mt + 8(i/4) + 4hh + (i%4)][query column lr]
  const int64_t ob = (int64_t(q0 + my_row) * Hq + h) * 128 + 4 * hh;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * mt + 8 * j;
      if (out_bf16) {
        const u32x2 wv = {pack_bf16x2(o[mt][4 * j] * inv, o[mt][4 * j + 1] * inv),
                          pack_bf16x2(o[mt][4 * j + 2] * inv, o[mt][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + ob + d) = wv;
      } else {
        const f32x4 fv = {o[mt][4 * j] * inv, o[mt][4 * j + 1] * inv, o[mt][4 * j + 2] * inv,
                          o[mt][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + ob + d) = fv;
      }
    }
  }
}

void launch_prefill_mfma(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                         const int32_t* cu_q, const int32_t* cu_k, const int32_t* block_table, int32_t mbps,
                         int32_t batch, int32_t max_seqlen_q, int32_t Hq, int32_t Hkv, int32_t block_size,
                         float scale, void* out, bool out_bf16, hipStream_t stream) {
  const int n_qtiles = (max_seqlen_q + kPreRows - 1) / kPreRows;
  const int n_work = batch * n_qtiles * Hq;
  const int grid = ((n_work + 7) / 8) * 8;
  const float sl2 = scale * kLog2e;
  const bool pow2 = (block_size & (block_size - 1)) == 0;
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kc = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(v_cache);
  if (pow2) {
    hipLaunchKernelGGL(prefill_mfma_kernel<true>, dim3(grid), dim3(kPreThreads), 0, stream, qp, q_stride, kc, vc,
                       cu_q, cu_k, block_table, mbps, batch, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16),
                       n_qtiles, n_work);
  } else {
    hipLaunchKernelGGL(prefill_mfma_kernel<false>, dim3(grid), dim3(kPreThreads), 0, stream, qp, q_stride, kc, vc,
                       cu_q, cu_k, block_table, mbps, batch, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16),
                       n_qtiles, n_work);
  }
}

}  // namespace pa
