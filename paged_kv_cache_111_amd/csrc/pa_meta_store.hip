// Metadata build and store_kvcache kernels.
//
// Metadata: the flattening of a step's sequences into per-token positions and slots, and the prefix sums that
// delimit sequences ("一个 prompt 的一生" §3.3.2, prepare_prefill example; slot formula of "Nano-vLLM 架构详解"
// §1, Step2). Store: a bit copy of each new token's K/V row to its slot ("Nano-vLLM 架构详解" §3.2, KV cache
// 写入函数).
#include "pa_dpp.h"
#include "pa_launch.h"

namespace pa {

// ------------------------------------------------------------------------------------------------- metadata
//
// Every workgroup rebuilds the two prefix sums over the batch in LDS (each thread sums a run of sequences, the
// runs are scanned with wave shuffles and across the four waves), then handles 256 tokens: a binary search for
// the token's sequence, its absolute position and its slot. Workgroup 0 also writes cu_seqlens_q/k and
// context_lens.
constexpr int kMetaThreads = 256;

// Fills cu_q[0..batch] and cu_k[0..batch] (LDS) with the prefix sums of num_new and of num_cached + num_new;
// workgroup 0 also writes them, and context_lens, to global memory. Called by all kMetaThreads threads.
__device__ __forceinline__ void meta_prefix_sums(const int32_t* __restrict__ num_cached,
                                                 const int32_t* __restrict__ num_new, int32_t batch,
                                                 int32_t* cu_q, int32_t* cu_k, int32_t* wave_q, int32_t* wave_k,
                                                 int32_t* __restrict__ cu_q_out, int32_t* __restrict__ cu_k_out,
                                                 int32_t* __restrict__ ctx_out) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = (batch + kMetaThreads - 1) / kMetaThreads;
  const int lo = min(batch, tid * chunk), hi = min(batch, lo + chunk);
  int32_t sq = 0, sk = 0;
  for (int s = lo; s < hi; ++s) {
    const int32_t n = num_new[s];
    sq += n;
    sk += num_cached[s] + n;
  }
  // exclusive prefix of the per-thread sums: inclusive scan within each wave (DPP), then across the waves
  const int32_t iq = dpp_incl_scan_i(sq), ik = dpp_incl_scan_i(sk);
  if (lane == 63) {
    wave_q[wave] = iq;
    wave_k[wave] = ik;
  }
  if (tid == 0) {
    cu_q[0] = 0;
    cu_k[0] = 0;
  }
  __syncthreads();
  sq = iq - sq;
  sk = ik - sk;
  for (int w = 0; w < wave; ++w) {
    sq += wave_q[w];
    sk += wave_k[w];
  }
  for (int s = lo; s < hi; ++s) {
    const int32_t n = num_new[s];
    const int32_t kl = num_cached[s] + n;
    sq += n;
    sk += kl;
    cu_q[s + 1] = sq;
    cu_k[s + 1] = sk;
    if (blockIdx.x == 0) ctx_out[s] = kl;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int s = tid; s <= batch; s += kMetaThreads) {
      cu_q_out[s] = cu_q[s];
      cu_k_out[s] = cu_k[s];
    }
  }
}

// Sequence of new token t (the largest s with cu_q[s] <= t: sequences with no new tokens have
// cu_q[s] == cu_q[s + 1] and are skipped), its absolute position and its slot (-1 for a position outside the
// sequence's row of the block table).
__device__ __forceinline__ int32_t meta_token(int32_t t, const int32_t* cu_q, int32_t batch,
                                              const int32_t* __restrict__ num_cached,
                                              const int32_t* __restrict__ block_table, int32_t mbps,
                                              int32_t block_size, int32_t& pos) {
  int a = 0, b = batch;  // invariant: cu_q[a] <= t < cu_q[b]
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    if (cu_q[mid] <= t) a = mid; else b = mid;
  }
  pos = num_cached[a] + (t - cu_q[a]);
  const int32_t blk = pos / block_size;
  if (pos < 0 || blk >= mbps) return -1;  // outside the sequence's table row: no slot (and no read past the row)
  return block_table[int64_t(a) * mbps + blk] * block_size + (pos - blk * block_size);
}

__global__ __launch_bounds__(kMetaThreads) void build_metadata_kernel(
    const int32_t* __restrict__ num_cached, const int32_t* __restrict__ num_new,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t batch, int32_t total_q, int32_t block_size,
    int32_t* __restrict__ cu_q_out, int32_t* __restrict__ cu_k_out, int32_t* __restrict__ ctx_out,
    int32_t* __restrict__ pos_out, int32_t* __restrict__ slot_out) {
  extern __shared__ int32_t smem[];
  __shared__ int32_t wave_q[kMetaThreads / 64], wave_k[kMetaThreads / 64];
  int32_t* cu_q = smem;                  // [batch + 1]
  int32_t* cu_k = smem + (batch + 1);    // [batch + 1]
  meta_prefix_sums(num_cached, num_new, batch, cu_q, cu_k, wave_q, wave_k, cu_q_out, cu_k_out, ctx_out);
  const int t = blockIdx.x * kMetaThreads + threadIdx.x;
  if (t >= total_q) return;
  int32_t pos;
  const int32_t slot = meta_token(t, cu_q, batch, num_cached, block_table, mbps, block_size, pos);
  pos_out[t] = pos;
  slot_out[t] = slot;
}

// ------------------------------------------------------------------------------------------------- both
//
// Metadata and store in one launch: one wave per new token, four per workgroup (each workgroup rebuilds the
// prefix sums as above). The wave issues the loads of its token's K and V rows first, since they depend on the
// token index alone, so that they are in flight during the prefix sums; it then finds the token's slot, writes
// the position and the slot, and writes the rows to the slot (no write for a negative slot).
template <typename VecT>
__global__ __launch_bounds__(kMetaThreads) void metadata_store_kernel(
    const int32_t* __restrict__ num_cached, const int32_t* __restrict__ num_new,
    const int32_t* __restrict__ block_table, int32_t mbps, int32_t batch, int32_t total_q, int32_t block_size,
    int32_t* __restrict__ cu_q_out, int32_t* __restrict__ cu_k_out, int32_t* __restrict__ ctx_out,
    int32_t* __restrict__ pos_out, int32_t* __restrict__ slot_out, const char* __restrict__ k,
    int64_t k_stride_bytes, const char* __restrict__ v, int64_t v_stride_bytes, char* __restrict__ k_cache,
    char* __restrict__ v_cache, int32_t row_vecs) {
  extern __shared__ int32_t smem[];
  __shared__ int32_t wave_q[kMetaThreads / 64], wave_k[kMetaThreads / 64];
  int32_t* cu_q = smem;                  // [batch + 1]
  int32_t* cu_k = smem + (batch + 1);    // [batch + 1]
  constexpr int kRegVecs = 4;            // rows of up to 4 * 64 vectors are held in registers meanwhile

  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kMetaThreads / 64) + (threadIdx.x >> 6);
  const bool has_token = t < total_q;
  const bool in_regs = row_vecs <= kRegVecs * 64;
  const VecT* ks = reinterpret_cast<const VecT*>(k + int64_t(t) * k_stride_bytes);
  const VecT* vs = reinterpret_cast<const VecT*>(v + int64_t(t) * v_stride_bytes);
  VecT kr[kRegVecs] = {}, vr[kRegVecs] = {};
  if (has_token && in_regs) {
#pragma unroll
    for (int j = 0; j < kRegVecs; ++j) {
      const int i = lane + 64 * j;
      if (i < row_vecs) {
        kr[j] = ks[i];
        vr[j] = vs[i];
      }
    }
  }
  meta_prefix_sums(num_cached, num_new, batch, cu_q, cu_k, wave_q, wave_k, cu_q_out, cu_k_out, ctx_out);
  if (!has_token) return;
  int32_t pos;
  const int32_t slot = meta_token(t, cu_q, batch, num_cached, block_table, mbps, block_size, pos);
  if (lane == 0) {
    pos_out[t] = pos;
    slot_out[t] = slot;
  }
  if (slot < 0) return;
  const int64_t row_bytes = int64_t(row_vecs) * sizeof(VecT);
  VecT* kd = reinterpret_cast<VecT*>(k_cache + int64_t(slot) * row_bytes);
  VecT* vd = reinterpret_cast<VecT*>(v_cache + int64_t(slot) * row_bytes);
  if (in_regs) {
#pragma unroll
    for (int j = 0; j < kRegVecs; ++j) {
      const int i = lane + 64 * j;
      if (i < row_vecs) {
        kd[i] = kr[j];
        vd[i] = vr[j];
      }
    }
  } else {
    for (int i = lane; i < row_vecs; i += 64) {
      const VecT a = ks[i];
      const VecT b = vs[i];
      kd[i] = a;
      vd[i] = b;
    }
  }
}

void launch_metadata_store(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                           int32_t mbps, int32_t batch, int32_t total_q, int32_t block_size, int32_t* cu_q,
                           int32_t* cu_k, int32_t* ctx, int32_t* pos, int32_t* slot, const void* k,
                           int64_t k_stride_bytes, const void* v, int64_t v_stride_bytes, void* k_cache,
                           void* v_cache, int64_t row_bytes, int vec_bytes, hipStream_t stream) {
  const int grid = total_q > 0 ? (total_q + kMetaThreads / 64 - 1) / (kMetaThreads / 64) : 1;
  const size_t lds = size_t(2) * (batch + 1) * sizeof(int32_t);
  const char* kp = static_cast<const char*>(k);
  const char* vp = static_cast<const char*>(v);
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
#define PA_LAUNCH_MS(VT)                                                                                        \
  hipLaunchKernelGGL(metadata_store_kernel<VT>, dim3(grid), dim3(kMetaThreads), lds, stream, num_cached, num_new, \
                     block_table, mbps, batch, total_q, block_size, cu_q, cu_k, ctx, pos, slot, kp,              \
                     k_stride_bytes, vp, v_stride_bytes, kc, vc, int32_t(row_bytes / sizeof(VT)))
  switch (vec_bytes) {
    case 16: PA_LAUNCH_MS(u32x4); break;
    case 8: PA_LAUNCH_MS(u32x2); break;
    case 4: PA_LAUNCH_MS(uint32_t); break;
    default: PA_LAUNCH_MS(uint16_t); break;
  }
#undef PA_LAUNCH_MS
}

void launch_build_metadata(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                           int32_t mbps, int32_t batch, int32_t total_q, int32_t block_size, int32_t* cu_q,
                           int32_t* cu_k, int32_t* ctx, int32_t* pos, int32_t* slot, hipStream_t stream) {
  const int grid = total_q > 0 ? (total_q + kMetaThreads - 1) / kMetaThreads : 1;
  const size_t lds = size_t(2) * (batch + 1) * sizeof(int32_t);
  hipLaunchKernelGGL(build_metadata_kernel, dim3(grid), dim3(kMetaThreads), lds, stream, num_cached, num_new,
                     block_table, mbps, batch, total_q, block_size, cu_q, cu_k, ctx, pos, slot);
}

// ------------------------------------------------------------------------------------------------- store
//
// One wave per token, four tokens per workgroup. A wave copies the token's K row then its V row
// (num_kv_heads * head_dim elements each) with VEC-byte accesses; lanes cover consecutive VEC-byte pieces, so
// each row is read and written as whole contiguous runs.
constexpr int kStoreThreads = 256;

template <typename VecT>
__global__ __launch_bounds__(kStoreThreads) void store_kvcache_kernel(
    const char* __restrict__ k, int64_t k_stride_bytes, const char* __restrict__ v, int64_t v_stride_bytes,
    char* __restrict__ k_cache, char* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping,
    int32_t num_tokens, int32_t row_vecs) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kStoreThreads / 64) + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;
  const int64_t row_bytes = int64_t(row_vecs) * sizeof(VecT);
  const VecT* ks = reinterpret_cast<const VecT*>(k + t * k_stride_bytes);
  const VecT* vs = reinterpret_cast<const VecT*>(v + t * v_stride_bytes);
  VecT* kd = reinterpret_cast<VecT*>(k_cache + int64_t(slot) * row_bytes);
  VecT* vd = reinterpret_cast<VecT*>(v_cache + int64_t(slot) * row_bytes);
  for (int i = lane; i < row_vecs; i += 64) {
    const VecT a = ks[i];
    const VecT b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

void launch_store_kvcache(const void* k, int64_t k_stride_bytes, const void* v, int64_t v_stride_bytes,
                          void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                          int64_t row_bytes, int vec_bytes, hipStream_t stream) {
  const int grid = (num_tokens + kStoreThreads / 64 - 1) / (kStoreThreads / 64);
  const char* kp = static_cast<const char*>(k);
  const char* vp = static_cast<const char*>(v);
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  switch (vec_bytes) {
    case 16:
      hipLaunchKernelGGL(store_kvcache_kernel<u32x4>, dim3(grid), dim3(kStoreThreads), 0, stream, kp,
                         k_stride_bytes, vp, v_stride_bytes, kc, vc, slot_mapping, num_tokens,
                         int32_t(row_bytes / 16));
      break;
    case 8:
      hipLaunchKernelGGL(store_kvcache_kernel<u32x2>, dim3(grid), dim3(kStoreThreads), 0, stream, kp,
                         k_stride_bytes, vp, v_stride_bytes, kc, vc, slot_mapping, num_tokens,
                         int32_t(row_bytes / 8));
      break;
    case 4:
      hipLaunchKernelGGL(store_kvcache_kernel<uint32_t>, dim3(grid), dim3(kStoreThreads), 0, stream, kp,
                         k_stride_bytes, vp, v_stride_bytes, kc, vc, slot_mapping, num_tokens,
                         int32_t(row_bytes / 4));
      break;
    default:
      hipLaunchKernelGGL(store_kvcache_kernel<uint16_t>, dim3(grid), dim3(kStoreThreads), 0, stream, kp,
                         k_stride_bytes, vp, v_stride_bytes, kc, vc, slot_mapping, num_tokens,
                         int32_t(row_bytes / 2));
      break;
  }
}

}  // namespace pa
