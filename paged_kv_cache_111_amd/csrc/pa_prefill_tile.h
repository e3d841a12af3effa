// Tile machinery of the paged prefill kernels (bf16 K/V, head_dim 128): 64-key K/V tiles gathered through the
// block table into LDS, scores and weights of a wave's 32 query rows, and the PV product on the matrix cores.
//
//   S^T[key, q] = K[key, :] . Q[q, :]      32x32x16 MFMA, A = K rows from LDS, B = Q^T kept in registers
//   O^T[d, q]  += V^T[d, key] P^T[key, q]  32x32x16 fp16 MFMA, A = V^T via the LDS transpose read (V is
//                                           converted to fp16 when staged), B = P^T (fp16) formed
//                                           lane by lane from the scores the score MFMA left
// With scores transposed, each lane owns one query column; its keys are split over the two wave halves, which
// exchange the row max only when a tile moves the running reference max, and the row sum once at the end.
// The key -> k-slot assignment of the second product follows the score layout (lane half hh holds keys
// 8j + 4hh .. +3), so P^T needs no data movement.
#pragma once

#include "pa_launch.h"

namespace pa {

constexpr int kPreThreads = 256;  // threads that stage one tile (four waves)
constexpr int kKRow = 128 + 8;    // LDS row stride of the K tile, in elements (272 bytes: the 16-byte reads of
                                  // 16 consecutive rows fall on distinct banks)
constexpr int kVRow = 128 + 32;   // LDS row stride of the V tile (320 bytes: the transposed 8-byte reads of 32
                                  // lanes span 4 rows x 64 bytes, which this stride spreads over all 64 banks;
                                  // 288-byte rows left a quarter of the LDS-active cycles in bank conflicts)
#ifndef PA_PREFILL_KEYS
#define PA_PREFILL_KEYS 64
#endif
constexpr int kPreKeys = PA_PREFILL_KEYS;  // keys per tile (a multiple of 32)
constexpr int kSub = kPreKeys / 32;        // 32-key score sub-tiles per tile
constexpr int kPieces = kPreKeys * 16 / kPreThreads;  // 16-byte pieces of K (and of V) per thread per tile
constexpr float kRescaleSlack = 8.f;       // the running max is only moved when it would grow by more than this

template <bool kPow2>
__device__ __forceinline__ int64_t pf_slot(const int32_t* table, int key, int bs, int bs_shift) {
  if (kPow2) return int64_t(table[key >> bs_shift]) * bs + (key & (bs - 1));
  const int blk = key / bs;
  return int64_t(table[blk]) * bs + (key - blk * bs);
}

// Buffer descriptor over the valid rows of the tile of keys kb .. kb + kPreKeys - 1 (kAligned case).
template <bool kPow2>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pf_tile_rsrc(const char* base, const int32_t* table, int kb,
                                                              int k_len, int bs, int bs_shift, int64_t row_bytes) {
  const int n = max(0, min(kPreKeys, k_len - kb));
  const int key0 = n > 0 ? kb : 0;
  const int blk = kPow2 ? (key0 >> bs_shift) : (key0 / bs);
  const int phys = __builtin_amdgcn_readfirstlane(table[blk]);
  const int64_t off = (int64_t(phys) * bs + (key0 - blk * bs)) * row_bytes;
  const int nbytes = __builtin_amdgcn_readfirstlane(int(n * row_bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), 0, nbytes, 0x00020000);
}

// Global loads of one tile (K or V) into staging registers: piece c = it * 256 + tid is key c / 16,
// d 8 (c % 16) .. +7. Keys >= k_len (and tiles wholly past the end) read as zero.
template <bool kAligned, bool kPow2>
__device__ __forceinline__ void pf_gload1(u32x4* dst, const char* base, const int32_t* table, int kb, int k_len,
                                          int bs, int bs_shift, int64_t row_bytes, int tid) {
  if (kAligned) {
    const __amdgpu_buffer_rsrc_t r = pf_tile_rsrc<kPow2>(base, table, kb, k_len, bs, bs_shift, row_bytes);
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int c = it * kPreThreads + tid;
      dst[it] = __builtin_amdgcn_raw_buffer_load_b128(r, int((c >> 4) * row_bytes) + 16 * (c & 15), 0, 0);
    }
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int it = 0; it < kPieces; ++it) {
      const int c = it * kPreThreads + tid;
      const int key = kb + (c >> 4);
      dst[it] = key < k_len ? ld16(base + pf_slot<kPow2>(table, key, bs, bs_shift) * row_bytes + 16 * (c & 15)) : z;
    }
  }
}

__device__ __forceinline__ void pf_lstore_k(const u32x4* src, uint16_t* kt, int tid) {
#pragma unroll
  for (int it = 0; it < kPieces; ++it) {
    const int c = it * kPreThreads + tid;
    st16(kt + (c >> 4) * kKRow + 8 * (c & 15), src[it]);
  }
}

// V is converted to fp16 on the way to LDS (exact in fp16's normal range): the PV product runs in fp16.
__device__ __forceinline__ void pf_lstore_v(const u32x4* src, uint16_t* vt, int tid) {
#pragma unroll
  for (int it = 0; it < kPieces; ++it) {
    const int c = it * kPreThreads + tid;
    st16(vt + (c >> 4) * kVRow + 8 * (c & 15), bf16x8_to_f16x8(src[it]));
  }
}

// S^T for the 64 keys of a K tile in LDS: sc[sub][i] is key 32 sub + 8 (i / 4) + 4 hh + (i % 4) of the tile,
// query column lr of the wave. With kBatch, a sub-tile's eight K operands are read before its MFMAs (eight LDS
// reads in flight instead of two; the per-key gathers of unaligned block sizes leave no registers for it).
template <bool kBatch>
__device__ __forceinline__ void pf_scores(f32x16 (&sc)[kSub], const uint16_t* kt, int ka_off, const bf16x8 (&qb)[8]) {
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[sub][i] = 0.f;
    const uint16_t* ka = kt + ka_off + 32 * sub * kKRow;
    if (kBatch) {
      u32x4 kr[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kr[ks] = *reinterpret_cast<const u32x4*>(ka + 16 * ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sc[sub] = mfma32x32x16(as_bf16x8(kr[ks]), qb[ks], sc[sub]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sc[sub] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(ka + 16 * ks)), qb[ks], sc[sub]);
    }
  }
}

// Causal mask of one tile's scores (only called where some key of the tile is after some row of the wave).
// Key kb + c + 4hh is masked (-inf) when it is after the row's position, i.e. c > lim = position - kb - 4hh;
// c is a constant per register, so the test compares constants with one per-lane limit.
__device__ __forceinline__ void pf_mask(f32x16 (&sc)[kSub], int lim) {
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int c = 32 * sub + 8 * (i >> 2) + (i & 3);
      if (c > lim) sc[sub][i] = -INFINITY;
    }
}

// The max over this lane's half of its row (-inf if all masked), unscaled.
__device__ __forceinline__ float pf_halfmax(const f32x16 (&sc)[kSub]) {
  float mx = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[sub][i]);
  return mx;
}

// Weights of one tile (fp16, round to nearest; the row sum is taken over the rounded weights that enter the PV
// product, so the weights the output averages with sum to one), as the B operand of the PV MFMA.
// Lane group g4 = lane / 16 (half hh = g4 / 2, d offset 16 (g4 % 2)); for k-step kk the lane's slots 0..3 are
// keys 16 kk + 4 hh + 0..3 and slots 4..7 keys 16 kk + 8 + 4 hh + 0..3.
__device__ __forceinline__ void pf_weights(const f32x16 (&sc)[kSub], f16x8 (&pb)[kSub][2], float m, float& lsum,
                                           float scale_log2) {
  float psum[2] = {0.f, 0.f};  // two independent chains
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[sub][8 * kk + i], scale_log2, -m));
      const u32x4 pw = {pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]), pack_f16x2(p[4], p[5]),
                        pack_f16x2(p[6], p[7])};
      psum[kk] = add_f16x2(pw[3], add_f16x2(pw[2], add_f16x2(pw[1], add_f16x2(pw[0], psum[kk]))));
      pb[sub][kk] = as_f16x8(pw);
    }
  }
  lsum += psum[0] + psum[1];
}

// O^T += V^T P^T from the V tile in LDS: 16 MFMAs back to back.
__device__ __forceinline__ void pf_pv(const f16x8 (&pb)[kSub][2], f32x16 (&o)[4], const uint16_t* vt, int va_off) {
#pragma unroll
  for (int sub = 0; sub < kSub; ++sub) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint16_t* vr = vt + va_off + (32 * sub + 16 * kk) * kVRow;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const i16x4 a0 = lds_read_tr16(vr + 32 * mt);
        const i16x4 a1 = lds_read_tr16(vr + 8 * kVRow + 32 * mt);
        const f16x8 av = __builtin_bit_cast(f16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = mfma32x32x16_f16(av, pb[sub][kk], o[mt]);
      }
    }
  }
}

// The tile's weights, then its PV product. The compiler forms each k-step's weights while the previous k-step's
// MFMAs run, which measured faster than forming all weights first (the PV block then waits on its LDS reads);
// the score MFMAs stay one block, since weights placed between them delayed the wave's MFMAs more than the other
// wave on the SIMD lost.
__device__ __forceinline__ void pf_weights_pv(const f32x16 (&sc)[kSub], f32x16 (&o)[4], float m, float& lsum,
                                              const uint16_t* vt, int va_off, float scale_log2) {
  f16x8 pb[kSub][2];
  pf_weights(sc, pb, m, lsum, scale_log2);
  pf_pv(pb, o, vt, va_off);
}

}  // namespace pa
