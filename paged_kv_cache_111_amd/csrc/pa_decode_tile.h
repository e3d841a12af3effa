// Tile machinery of the paged decode kernels (one query token per sequence, bf16, head_dim 128, GQA group
// <= 16): loading a 32-key tile of K and V rows through the block table, and one online-softmax step over it.
//
// Per KV head, the G query heads are the N = 16 columns of 16x16x32 bf16 MFMAs (unused columns are zero):
//   S^T[key, g] = K[key, :] . Q[g, :]      A = K rows straight from HBM (16 B per lane), B = Q^T in registers
//   O^T[d, g]  += V^T[d, key] P^T[key, g]  A = V^T from a row-major LDS tile via the transpose read, B = P^T
//                                           kept in the registers the score MFMA left it in
// The key -> MFMA k-slot assignment of the second product is chosen so that P^T needs no data movement: lane
// group lg (lanes 16lg..16lg+15) holds keys 4lg..4lg+3 of each 16-key score tile, and those become its k-slots.
// Online softmax runs per column g in the log2 domain.
#pragma once

#include "pa_launch.h"

namespace pa {

constexpr int kDecKeys = 32;       // keys per tile (two 16-key score tiles)
constexpr int kVRow = 128 + 8;     // LDS row stride of the V tile, in bf16 elements (272 bytes)
#ifndef PA_DECODE_NBUF
#define PA_DECODE_NBUF 2
#endif
constexpr int kNBuf = PA_DECODE_NBUF;  // tiles whose loads are in flight per wave (software pipeline depth)

template <bool kPow2>
__device__ __forceinline__ int64_t slot_of_key(const int32_t* table, int key, int bs, int bs_shift) {
  if (kPow2) return int64_t(table[key >> bs_shift]) * bs + (key & (bs - 1));
  const int blk = key / bs;
  return int64_t(table[blk]) * bs + (key - blk * bs);
}

// One tile of K and V rows in registers. k[tt][ks]: key base + 16tt + li, d 8lg + 32ks .. +7 (the A operand of the
// score MFMA); v[it]: key base + 4it + lg, d 8li .. +7 (staged to LDS before use).
struct KVTile {
  u32x4 k[2][4];
  u32x4 v[8];
};

// Byte offsets of this lane's pieces inside a tile, the same for every tile.
struct LaneOffsets {
  uint32_t k;  // li * row_bytes + 16 lg
  uint32_t v;  // lg * row_bytes + 16 li
};

__device__ __forceinline__ u32x4 ld16_off(const char* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// Loads the tile of keys base .. base+31 (keys >= t1 read as zero).
//
// kAligned (block size a multiple of 32): the tile lies in one block, so its block id is read once as a
// wave-uniform scalar and the tile is read through a raw buffer descriptor based at the tile's first row and
// sized to its valid rows. Rows past the end fall outside the descriptor and the hardware returns zeros for
// them without touching memory, so there is no branch per load and the number of loads in flight is the same
// on every path. A tile wholly past the end gets a zero-sized descriptor (based at the first tile's block, so
// the table entry read is always a real one).
template <bool kAligned, bool kPow2>
__device__ __forceinline__ void load_tile(KVTile& t, const char* __restrict__ kbase, const char* __restrict__ vbase,
                                          const int32_t* __restrict__ table, int base, int t0, int t1, int bs,
                                          int bs_shift, int64_t row_bytes, LaneOffsets lo, int lane) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int lg = lane >> 4;
  const int li = lane & 15;
  if (kAligned) {
    const int n = max(0, min(kDecKeys, t1 - base));  // valid rows of this tile
    const int key0 = n > 0 ? base : t0;
    const int blk = kPow2 ? (key0 >> bs_shift) : (key0 / bs);
    const int phys = __builtin_amdgcn_readfirstlane(table[blk]);
    const int64_t tile_off = (int64_t(phys) * bs + (key0 - blk * bs)) * row_bytes;
    const int nbytes = __builtin_amdgcn_readfirstlane(int(n * row_bytes));
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kbase + tile_off), 0, nbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vbase + tile_off), 0, nbytes, 0x00020000);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int off = int(lo.k) + int(16 * tt * row_bytes);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        t.k[tt][ks] = __builtin_amdgcn_raw_buffer_load_b128(kr, off + 64 * ks, 0, kLoadStream);
    }
#pragma unroll
    for (int it = 0; it < 8; ++it)
      t.v[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, int(lo.v) + int(4 * it * row_bytes), 0, kLoadStream);
  } else {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int key = base + 16 * tt + li;
      if (key < t1) {
        const char* kp = kbase + slot_of_key<kPow2>(table, key, bs, bs_shift) * row_bytes + 16 * lg;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) t.k[tt][ks] = ld16_stream(kp + 64 * ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) t.k[tt][ks] = z;
      }
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int key = base + 4 * it + lg;
      t.v[it] = key < t1 ? ld16_stream(vbase + slot_of_key<kPow2>(table, key, bs, bs_shift) * row_bytes + 16 * li) : z;
    }
  }
}


// Per-lane LDS addresses of a wave's V tile.
struct VTileLane {
  uint16_t* w;        // this lane's V piece it goes to row 4it + lg, d 8li
  const uint16_t* r0; // transposed reads of keys 4lg..4lg+3 at d = 16mt + li
  const uint16_t* r1; // and of keys 16+4lg..16+4lg+3
};

__device__ __forceinline__ VTileLane v_tile_lane(uint16_t* vt, int lane) {
  const int lg = lane >> 4;
  const int li = lane & 15;
  VTileLane v;
  v.w = vt + lg * kVRow + 8 * li;
  v.r0 = vt + (4 * lg + (li >> 2)) * kVRow + 4 * (li & 3);
  v.r1 = v.r0 + 16 * kVRow;
  return v;
}

// The first half of a step over the tile of keys base .. base+31 held in t: V rows to LDS and the scores.
// sc[tt][i] is key base + 16tt + 4lg + i, query column g = li. After this the registers of t are free.
__device__ __forceinline__ void tile_scores(const KVTile& t, const bf16x8 (&qb)[4], const VTileLane& vl,
                                            f32x4 (&sc)[2]) {
#pragma unroll
  for (int it = 0; it < 8; ++it) st16(vl.w + 4 * it * kVRow, t.v[it]);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sc[tt] = mfma16x16x32(as_bf16x8(t.k[tt][ks]), qb[ks], sc[tt]);
  }
}

// The second half: mask keys >= t1, online softmax (running max m, this lane's part of the sum lsum) and
// O^T += V^T P^T. The running max must be finite after the step (the first tile of a run holds a valid key).
// The normaliser is summed from the bf16-rounded weights that enter the PV product.
__device__ __forceinline__ void tile_softmax_pv(f32x4 (&sc)[2], int base, int t1, float scale_log2, int lane,
                                                const VTileLane& vl, f32x4 (&o)[8], float& m, float& lsum) {
  const int lg = lane >> 4;
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
  const float mn = fmaxf(m, mx);
  const float alpha = exp2f(m - mn);
  m = mn;
  float pv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pv[j] = exp2f(sc[j >> 2][j & 3] - mn);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] *= alpha;
  const u32x4 pw = {pack_weights_bf16x2(pv[0], pv[1]), pack_weights_bf16x2(pv[2], pv[3]),
                    pack_weights_bf16x2(pv[4], pv[5]), pack_weights_bf16x2(pv[6], pv[7])};
  lsum = lsum * alpha + ((sum_bf16x2(pw[0]) + sum_bf16x2(pw[1])) + (sum_bf16x2(pw[2]) + sum_bf16x2(pw[3])));
  const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const i16x4 a0 = lds_read_tr16(vl.r0 + 16 * mt);
    const i16x4 a1 = lds_read_tr16(vl.r1 + 16 * mt);
    const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    o[mt] = mfma16x16x32(av, pb, o[mt]);
  }
}

// Q^T as the B operand of the score MFMA: lane holds Q[g = li][d = 8lg + 32ks .. +7] (zero for li >= G).
__device__ __forceinline__ void load_q(bf16x8 (&qb)[4], const uint16_t* qrow0, int G, int lane) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int lg = lane >> 4;
  const int li = lane & 15;
  const uint16_t* qp = qrow0 + int64_t(li) * 128 + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qb[ks] = as_bf16x8(li < G ? ld16(qp + 32 * ks) : z);
}

}  // namespace pa
