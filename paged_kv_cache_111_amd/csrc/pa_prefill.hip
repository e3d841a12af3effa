// Paged varlen causal prefill on the matrix cores: bf16, head_dim 128.
//
// Workgroup = (sequence s, KV head, a block of query rows, a group of HW query heads of that KV head); four waves
// of 32 rows x one query head each. HW is 4 when the GQA group size G is a multiple of 4 (one 32-row block,
// four heads: every wave has the same rows, so all four meet the causal diagonal at the same key tile), 2 when
// G is even (two 32-row blocks x two heads) and 1 otherwise (four 32-row blocks of one head). All waves of a
// workgroup read one KV head, so the K/V tiles a workgroup stages serve all of them. Keys are walked in tiles of
// 64 gathered through the block table into LDS (row-major, both K and V, double-buffered: the next tile's global
// loads are in flight in registers while the current tile is computed):
//   S^T[key, q] = K[key, :] . Q[q, :]      32x32x16 MFMA, A = K rows from LDS, B = Q^T kept in registers
//   O^T[d, q]  += V^T[d, key] P^T[key, q]  32x32x16 fp16 MFMA, A = V^T via the LDS transpose read (V is
//                                           converted to fp16 when staged), B = P^T (fp16) formed
//                                           lane by lane from the scores the score MFMA left
// With scores transposed, each lane owns one query column; its keys are split over the two wave halves, which
// exchange the row max only when a tile moves the running reference max, and the row sum once at the end.
// The key -> k-slot assignment of the second product follows the score layout (lane half hh holds keys
// 8j + 4hh .. +3), so P^T needs no data movement.
//
// Causality follows absolute positions: the q_len new rows of a sequence with k_len keys sit at positions
// k_len - q_len .. k_len - 1 (a chunk continues after the cached prefix, "Nano-vLLM 源码逐行解析 第2篇",
// sequence.py), and a row at position p sees keys 0..p. Keys past k_len are never loaded (zero in LDS, -inf
// scores), so cache contents there cannot reach the output.
//
// Workgroup order: the flat grid is renumbered so that the workgroups the hardware sends to one XCD (every
// eighth) get consecutive logical ids, and the logical order is (KV head, group of hw row blocks = 128 rows from
// the last, sequence, row block in the group, head group). The row blocks of one KV head run on one XCD and read
// the same K/V through its L2, and the blocks of a 128-row group start together and walk the same keys (with
// four heads per workgroup, ordering the blocks one by one across sequences instead ran the varlen workload 25%
// slower); the last (heaviest, under the causal mask) groups of all sequences start first, so the short tail of
// light blocks balances the finish. A grid sized from max_seqlen_q holds many row blocks past a shorter
// sequence's end; for batches of up to 64 sequences the grid is sized from total_q instead and each workgroup
// finds the c-th existing block of that order (the same items in the same order, without the empty workgroups).
#include <algorithm>
#include <type_traits>

#include "pa_dpp.h"
#include "pa_prefill_tile.h"

namespace pa {

constexpr int kPreRows = 128;  // query rows x heads per workgroup (4 waves x 32 rows)
constexpr int kPartRow = 132;  // floats per row of a split partial: m, l, two unused, O[128] (16-byte aligned)
constexpr int kCompactBatch = 64;  // batches up to this many sequences (and prompts up to 63 x 128 rows) number only
                                   // existing row blocks: one lane per sequence, one per 128-row group round

// Query heads per workgroup for a GQA group of G heads (see the header comment).
inline int prefill_heads_per_wg(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

template <bool kAligned, bool kPow2>
__global__ __launch_bounds__(kPreThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mfma_kernel(
    const uint16_t* __restrict__ q, int64_t q_stride, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t batch, int32_t Hq, int32_t Hkv, int32_t bs,
    int32_t bs_shift, float scale_log2, void* __restrict__ out, int out_bf16, int32_t hw, int32_t n_qtiles,
    int32_t n_work, int32_t n_splits, int32_t part_rows, float* __restrict__ part, int32_t per_kvh) {
  // ---- which (KV head, sequence, row block, key split, head group) this workgroup computes
  const int per_xcd = (int(gridDim.x) + 7) >> 3;
  const int logical = int(blockIdx.x & 7) * per_xcd + int(blockIdx.x >> 3);
  if (logical >= n_work) return;
  const int G = Hq / Hkv;
  const int n_hg = G / hw;
  const int rows = kPreRows / hw;  // query rows of the workgroup: 32 x (4 / hw)
  const int n_grp = n_qtiles / hw;
  // Row blocks in groups of hw (128 rows): the blocks of a group are consecutive ids, so they start together and
  // walk the same keys through the XCD's L2 (as the G one-head workgroups of a 128-row block would); groups go
  // from the last rows of the longest sequence down (heaviest under the causal mask first), and within a group
  // round by sequence, then by block from the group's last.
  int hg, sp, s, qtile, kvh, q0, q_len, k_len;
  if (per_kvh > 0) {
    // Compact numbering (batch <= 64, n_grp <= 63): the grid holds per_kvh >= the number of non-empty items of a
    // KV head, and item c is the c-th non-empty (row block, head group, split) in the order above. One lane per
    // sequence holds its row-block count; lane g counts the blocks of the first g group rounds, a ballot finds
    // the round of item c, and a walk over the sequences its row block (register reads only, no LDS).
    kvh = logical / per_kvh;
    int c = logical % per_kvh;
    hg = c % n_hg;
    c /= n_hg;
    sp = c % n_splits;
    c /= n_splits;
    const int lane = int(threadIdx.x) & 63;
    const bool has = lane < batch;  // this lane's sequence: its offsets and lengths in one round trip
    const int lq0 = has ? cu_q[lane] : 0, lq = has ? cu_q[lane + 1] - lq0 : 0, lk = has ? cu_k[lane + 1] - cu_k[lane] : 0;
    const int nq = (lq + rows - 1) / rows;
    int before = 0;  // lane g: blocks at or above block (n_grp - g) * hw, over all sequences
    for (int t = 0; t < batch; ++t) before += max(0, __builtin_amdgcn_readlane(nq, t) - (n_grp - lane) * hw);
    if (c >= __builtin_amdgcn_readlane(before, n_grp)) return;  // beyond the last non-empty item
    const int g = __builtin_amdgcn_readfirstlane(__popcll(__ballot(lane <= n_grp && before <= c))) - 1;
    const int base = (n_grp - 1 - g) * hw;  // lowest block of round g
    int r = c - __builtin_amdgcn_readlane(before, g);  // position within the round
    s = -1;
    qtile = 0;
    for (int t = 0; t < batch; ++t) {
      const int cnt = min(hw, max(0, __builtin_amdgcn_readlane(nq, t) - base));  // sequence t's blocks in the round
      if (r < cnt) {
        s = t;
        qtile = base + cnt - 1 - r;
        break;
      }
      r -= cnt;
    }
    if (s < 0) return;  // not reached: the round holds more than r blocks
    q0 = __builtin_amdgcn_readlane(lq0, s);
    q_len = __builtin_amdgcn_readlane(lq, s);
    k_len = __builtin_amdgcn_readlane(lk, s);
  } else {
    hg = logical % n_hg;
    int rest = logical / n_hg;
    sp = rest % n_splits;
    rest /= n_splits;
    const int qsub = rest % hw;
    rest /= hw;
    s = rest % batch;
    rest /= batch;
    qtile = (n_grp - 1 - rest % n_grp) * hw + (hw - 1 - qsub);
    kvh = rest / n_grp;
    q0 = cu_q[s];
    q_len = cu_q[s + 1] - q0;
    if (qtile * rows >= q_len) return;
    k_len = cu_k[s + 1] - cu_k[s];
  }
  const int row0 = qtile * rows;
  const int past = k_len - q_len;  // position of row 0
  const int row_end = min(q_len, row0 + rows);
  const int n_keys = past + row_end;  // keys needed by the last row of the block
  const int n_tiles_all = (n_keys + kPreKeys - 1) / kPreKeys;
  // Split sp of n_splits takes key tiles [t0, t1) of the workgroup's tiles (all of them when n_splits == 1); its
  // loads stop at key t1 * 64, and its rows leave unnormalised partials for the merge pass.
  const int per_split = (n_tiles_all + n_splits - 1) / n_splits;
  const int t0 = sp * per_split;
  const int t1 = min(n_tiles_all, t0 + per_split);
  const int n_tiles = t1 - t0;
  const int k_lim = min(k_len, t1 * kPreKeys);

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;   // query column owned by this lane
  const int hh = lane >> 5;   // wave half
  const int h = kvh * G + hg * hw + w % hw;  // this wave's query head
  const int wave_row0 = row0 + 32 * (w / hw);
  const int my_row = wave_row0 + lr;
  // partial row of (sequence, row, head, split): [batch][part_rows][Hq][n_splits][kPartRow] (split mode only)
  auto prow = [&]() { return ((int64_t(s) * part_rows + my_row) * Hq + h) * n_splits + sp; };
  if (n_tiles <= 0) {  // an empty split (only when n_splits > 1): its rows' partials say "no keys"
    if (hh == 0 && my_row < q_len) {
      part[prow() * kPartRow] = -INFINITY;
      part[prow() * kPartRow + 1] = 0.f;
    }
    return;
  }

  const int wave_keys = wave_row0 < q_len ? past + min(q_len - 1, wave_row0 + 31) + 1 : 0;
  const int wave_tiles = (wave_keys + kPreKeys - 1) / kPreKeys;  // the tiles this wave computes: 0 .. wave_tiles-1
  const int32_t* table = block_table + int64_t(s) * mbps;
  const int64_t row_bytes = int64_t(Hkv) * 256;
  const char* kbase = reinterpret_cast<const char*>(k_cache + kvh * 128);
  const char* vbase = reinterpret_cast<const char*>(v_cache + kvh * 128);
  const int my_pos = past + my_row;

  // B operand of the score MFMA: lane holds Q[my_row][8hh + 16ks .. +7], ks = 0..7
  bf16x8 qb[8];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const uint16_t* qp = q + int64_t(q0 + my_row) * q_stride + int64_t(h) * 128 + 8 * hh;
    const bool ok = my_row < q_len;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = as_bf16x8(ok ? ld16(qp + 16 * ks) : z);
  }

  // K tiles run one tile ahead of V tiles: step j computes tile j+1's scores as well as tile j's softmax and PV
  // (so a wave's matrix work comes in two blocks per step), while K tile j+2 and V tile j+1 are loading.
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][kPreKeys * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vt[2][kPreKeys * kVRow];

  f32x16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mt][i] = 0.f;
  float m = -INFINITY;  // running reference max of this row, in scaled log2 units
  bool started = false;  // the wave has set its reference max (wave-uniform)
  float lsum = 0.f;     // this lane's part of the row sum (the two halves are added at the end)

  const int li = lane & 15;
  const int g4 = lane >> 4;
  const int ka_off = lr * kKRow + 8 * hh;  // K A operand: row lr, d 8hh + 16ks
  const int va_off = (4 * (g4 >> 1) + (li >> 2)) * kVRow + 16 * (g4 & 1) + 4 * (li & 3);

  u32x4 kst[kPieces], vst[kPieces];
#define PF_GLOAD(dst, b, kb) pf_gload1<kAligned, kPow2>(dst, b, table, kb, k_lim, bs, bs_shift, row_bytes, tid)
  // prologue: K tiles t0 and t0+1, V tile t0 in LDS (their loads issued together: one round trip); scores of
  // tile t0
  {
    u32x4 k1st[kPieces];
    const int kb0 = t0 * kPreKeys;
    PF_GLOAD(kst, kbase, kb0);
    PF_GLOAD(vst, vbase, kb0);
    PF_GLOAD(k1st, kbase, kb0 + kPreKeys);
    pf_lstore_k(kst, kt[0], tid);
    pf_lstore_v(vst, vt[0], tid);
    pf_lstore_k(k1st, kt[1], tid);
  }
  __syncthreads();
  f32x16 sa[kSub], sb[kSub];
  pf_scores<kAligned>(sa, kt[0], ka_off, qb);
  __syncthreads();  // K tile t0 has been read by every wave before the first step replaces it

  auto step = [&](int j, f32x16 (&cur)[kSub], f32x16 (&nxt)[kSub], auto par) {
    constexpr int P = decltype(par)::value;  // (j - t0) % 2
    const int kb = j * kPreKeys;
    // K tile j+2 and V tile j+1 start loading (past the split's end they read as zero and touch no memory)
    PF_GLOAD(kst, kbase, kb + 2 * kPreKeys);
    PF_GLOAD(vst, vbase, kb + kPreKeys);
    if (j < wave_tiles) {
      if (kb + kPreKeys - 1 > past + wave_row0) pf_mask(cur, my_pos - kb - 4 * hh);
      const float mh = pf_halfmax(cur) * scale_log2;
      pf_scores<kAligned>(nxt, kt[1 - P], ka_off, qb);  // tile j+1's scores (K tile j+1 has been in LDS since the last step)
      // The reference max only moves when the row max would exceed it by more than the slack; until then the
      // weights exp2(s - m) stay below 2^8 and O, l need no rescaling. The result O / l does not depend on m.
      // The row's keys are split over the two wave halves: the vote runs on each half's own max (no half above
      // m + slack means no row above it), and only a tile that moves the reference max exchanges the halves.
      if (__any(mh > m + kRescaleSlack)) {
        const float mn = fmaxf(m, xhalf_max(mh));
        if (started) {  // on the wave's first tile O and l are still zero
          const float alpha = __builtin_amdgcn_exp2f(m - mn);
          lsum *= alpha;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) o[mt] *= alpha;
        }
        m = mn;
        started = true;
      }
      // a row that has seen no key yet (possible in a split that starts after its position) keeps m = -inf and
      // all its scores are -inf: its weights are formed against 0, so they are 0 and not NaN
      pf_weights_pv(cur, o, m == -INFINITY ? 0.f : m, lsum, vt[P], va_off, scale_log2);
      pf_lstore_k(kst, kt[P], tid);      // K tile j+2 replaces K tile j (scored in the previous step)
      pf_lstore_v(vst, vt[1 - P], tid);  // V tile j+1 replaces V tile j-1 (read by the previous step's PV)
    } else {
      pf_lstore_k(kst, kt[P], tid);
      pf_lstore_v(vst, vt[1 - P], tid);
    }
    __syncthreads();
  };
  for (int jr = 0; jr < n_tiles; jr += 2) {
    step(t0 + jr, sa, sb, std::integral_constant<int, 0>());
    if (jr + 1 < n_tiles) step(t0 + jr + 1, sb, sa, std::integral_constant<int, 1>());
  }

  if (my_row >= q_len) return;
  lsum = xhalf_sum(lsum);
  if (n_splits > 1) {  // unnormalised partial: m (scaled log2 units), l, O; the merge pass finishes the row
    float* pr = part + prow() * kPartRow;
    if (hh == 0) {
      pr[0] = m;
      pr[1] = lsum;
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(pr + 4 + 32 * mt + 8 * j + 4 * hh) =
            f32x4{o[mt][4 * j], o[mt][4 * j + 1], o[mt][4 * j + 2], o[mt][4 * j + 3]};
    return;
  }
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

// Key splits of a call (host sizes only): when the grid holds fewer workgroups than the chip runs at once (two per
// CU on the 256 CUs), each workgroup's key tiles are split so that about that many run, each split at least
// kMinSplitKeys keys, at most kMaxSplits splits. One split leaves the output to the attention kernel itself. The
// count is taken on 128-row units of work (row blocks x heads / 128), which is the same for every GQA packing.
constexpr int64_t kPrefillSlots = 512;
constexpr int64_t kMinSplitKeys = 1024;
constexpr int64_t kMaxSplits = 32;

int32_t prefill_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq) {
  const int64_t n_qtiles = (int64_t(max_seqlen_q) + kPreRows - 1) / kPreRows;
  const int64_t n_work = int64_t(batch) * n_qtiles * Hq;
  if (n_work <= 0 || n_work >= kPrefillSlots) return 1;
  int64_t sp = (kPrefillSlots + n_work - 1) / n_work;
  sp = std::min(sp, int64_t(max_seqlen_k) / kMinSplitKeys);
  sp = std::min(sp, kMaxSplits);
  return int32_t(std::max<int64_t>(sp, 1));
}

// Rows of one sequence in the partial layout: max_seqlen_q rounded up to 128 (a multiple of every packing's block).
static int64_t prefill_part_rows(int32_t max_seqlen_q) { return (int64_t(max_seqlen_q) + kPreRows - 1) / kPreRows * kPreRows; }

size_t prefill_mfma_workspace_bytes(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq) {
  const int32_t sp = prefill_splits(batch, max_seqlen_q, max_seqlen_k, Hq);
  if (sp <= 1) return 0;
  return size_t(int64_t(batch) * prefill_part_rows(max_seqlen_q) * Hq * sp * kPartRow) * sizeof(float);
}

// Merge of a row's split partials: M = max m_i, L = sum l_i 2^(m_i - M), O = sum O_i 2^(m_i - M) / L (splits with
// no key for the row have m = -inf and weight 0). One wave per (token, query head), two of the 128 d per lane.
__global__ __launch_bounds__(64) void prefill_merge_kernel(const int32_t* __restrict__ cu_q, int32_t batch, int32_t Hq,
                                                           int32_t part_rows, int32_t n_splits,
                                                           const float* __restrict__ part, void* __restrict__ out,
                                                           int out_bf16) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  int a = 0, b = batch;  // the sequence of token t: cu_q[a] <= t < cu_q[a + 1]
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    if (cu_q[mid] <= t) a = mid; else b = mid;
  }
  const int r = t - cu_q[a];
  const float* p = part + ((int64_t(a) * part_rows + r) * Hq + h) * n_splits * kPartRow;
  const float mj = lane < n_splits ? p[lane * kPartRow] : -INFINITY;
  const float lj = lane < n_splits ? p[lane * kPartRow + 1] : 0.f;
  const float M = dpp_max_f(mj);  // split 0 holds key 0, which every row sees: M is finite
  const float wj = mj == -INFINITY ? 0.f : exp2f(mj - M);
  const float L = dpp_sum_f(wj * lj);
  float a0 = 0.f, a1 = 0.f;
  for (int j = 0; j < n_splits; ++j) {
    const float w = lane_of(wj, j);
    if (w != 0.f) {  // wave-uniform; a split without keys for the row left no O
      const float2 v = *reinterpret_cast<const float2*>(p + j * kPartRow + 4 + 2 * lane);
      a0 += w * v.x;
      a1 += w * v.y;
    }
  }
  const float inv = 1.f / L;
  const int64_t ob = (int64_t(t) * Hq + h) * 128 + 2 * lane;
  if (out_bf16) {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + ob) = pack_bf16x2(a0 * inv, a1 * inv);
  } else {
    *reinterpret_cast<float2*>(static_cast<float*>(out) + ob) = make_float2(a0 * inv, a1 * inv);
  }
}

void launch_prefill_mfma(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                         const int32_t* cu_q, const int32_t* cu_k, const int32_t* block_table, int32_t mbps,
                         int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                         int32_t Hkv, int32_t block_size, float scale, void* out, bool out_bf16, void* workspace,
                         hipStream_t stream) {
  const int hw = prefill_heads_per_wg(Hq / Hkv);
  const int rows = kPreRows / hw;
  const int n_qtiles = (max_seqlen_q + kPreRows - 1) / kPreRows * hw;  // a multiple of hw: 128-row groups
  const int n_splits = prefill_splits(batch, max_seqlen_q, max_seqlen_k, Hq);
  // Up to 64 sequences the grid counts only row blocks that exist: at most (total_q + batch (rows - 1)) / rows of
  // them per KV head and head group, against batch x n_qtiles in the plain numbering.
  const int n_hg = (Hq / Hkv) / hw;
  const int64_t n_blocks = std::min<int64_t>(int64_t(batch) * n_qtiles, (int64_t(total_q) + int64_t(batch) * (rows - 1)) / rows);
  const int per_kvh = batch <= kCompactBatch && n_qtiles / hw <= 63 ? int(n_blocks) * n_hg * n_splits : 0;
  const int n_work = per_kvh > 0 ? per_kvh * Hkv : batch * n_qtiles * (Hq / hw) * n_splits;
  const int grid = ((n_work + 7) / 8) * 8;
  const int part_rows = int(prefill_part_rows(max_seqlen_q));
  const float sl2 = scale * kLog2e;
  const bool pow2 = (block_size & (block_size - 1)) == 0;
  const bool aligned = block_size % kPreKeys == 0;
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kc = static_cast<const uint16_t*>(k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(v_cache);
  float* part = static_cast<float*>(workspace);
#define PA_LAUNCH_PF(A, P)                                                                                      \
  hipLaunchKernelGGL((prefill_mfma_kernel<A, P>), dim3(grid), dim3(kPreThreads), 0, stream, qp, q_stride, kc, vc, \
                     cu_q, cu_k, block_table, mbps, batch, Hq, Hkv, block_size, shift, sl2, out, int(out_bf16), hw, \
                     n_qtiles, n_work, n_splits, part_rows, part, per_kvh)
  if (aligned && pow2) PA_LAUNCH_PF(true, true);
  else if (aligned) PA_LAUNCH_PF(true, false);
  else if (pow2) PA_LAUNCH_PF(false, true);
  else PA_LAUNCH_PF(false, false);
#undef PA_LAUNCH_PF
  if (n_splits > 1)
    hipLaunchKernelGGL(prefill_merge_kernel, dim3(unsigned(total_q), unsigned(Hq)), dim3(64), 0, stream, cu_q, batch,
                       Hq, part_rows, n_splits, part, out, int(out_bf16));
}

}  // namespace pa
