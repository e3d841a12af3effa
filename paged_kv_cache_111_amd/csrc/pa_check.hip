// Validation of the index arrays a call will use: slots, the used block-table entries, context lengths and
// cumulative sequence lengths against the sizes of the pool and the table. The path itself trusts these
// indices (an out-of-range one is undefined behaviour there); this pass reads the index arrays only, never the
// caches, so it can run on arrays that are wrong and say how.
//
// report[k] counts the errors of kind k, report[kPaCheckKinds + k] holds the smallest offending index (token,
// sequence, or sequence * max_blocks_per_seq + block). Kinds, in the order of pa_check_kind in pa.h:
//   0 slot >= num_blocks * block_size                       (negative slots are "skip" and valid)
//   1 a used block-table entry outside [0, num_blocks)      (entries 0 .. ceil(k_len / block_size) - 1)
//   2 k_len < 0 or k_len > max_blocks_per_seq * block_size  (context_lens, or cu_seqlens_k differences)
//   3 cu_seqlens_q or cu_seqlens_k not starting at 0 or decreasing, or cu_seqlens_q[batch] != num_tokens
//   4 q_len > k_len                                         (prefill: new rows beyond the keys)
#include "pa_launch.h"

namespace pa {

constexpr int kPaCheckKinds = 5;
constexpr int kCheckThreads = 256;

__global__ void check_clear_kernel(uint32_t* __restrict__ report) {
  if (threadIdx.x < 2 * kPaCheckKinds) report[threadIdx.x] = threadIdx.x < kPaCheckKinds ? 0u : 0xffffffffu;
}

__device__ __forceinline__ void check_flag(uint32_t* report, int kind, uint32_t index) {
  atomicAdd(report + kind, 1u);
  atomicMin(report + kPaCheckKinds + kind, index);
}

// Grid-stride over tokens (slots), then over sequences (lengths, their used table entries, cu_seqlens).
__global__ __launch_bounds__(kCheckThreads) void check_indices_kernel(
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, const int32_t* __restrict__ block_table,
    int32_t batch, int32_t mbps, const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int32_t num_blocks, int32_t block_size, uint32_t* __restrict__ report) {
  const int64_t n_slots = int64_t(num_blocks) * block_size;
  const int64_t cap = int64_t(mbps) * block_size;
  const int stride = int(gridDim.x) * kCheckThreads;
  const int gid = int(blockIdx.x) * kCheckThreads + int(threadIdx.x);
  if (slot_mapping) {
    for (int t = gid; t < num_tokens; t += stride)
      if (slot_mapping[t] >= n_slots) check_flag(report, 0, uint32_t(t));
  }
  if (cu_q || cu_k) {
    // prefix arrays: element i of each against element i - 1 (and 0 at i = 0, num_tokens at i = batch)
    for (int i = gid; i <= batch; i += stride) {
      bool bad = false;
      if (cu_q) {
        bad |= i == 0 ? cu_q[0] != 0 : cu_q[i] < cu_q[i - 1];
        if (i == batch) bad |= cu_q[batch] != num_tokens;
      }
      if (cu_k) bad |= i == 0 ? cu_k[0] != 0 : cu_k[i] < cu_k[i - 1];
      if (bad) check_flag(report, 3, uint32_t(i));
    }
  }
  if (context_lens || cu_k) {
    for (int s = gid; s < batch; s += stride) {
      const int64_t k_len = context_lens ? int64_t(context_lens[s]) : int64_t(cu_k[s + 1]) - cu_k[s];
      if (k_len < 0 || k_len > cap) {
        check_flag(report, 2, uint32_t(s));
        continue;  // its table entries are not looked at: the length that would choose them is wrong
      }
      if (cu_q && cu_k) {
        const int64_t q_len = int64_t(cu_q[s + 1]) - cu_q[s];
        if (q_len > k_len) check_flag(report, 4, uint32_t(s));
      }
      const int used = int((k_len + block_size - 1) / block_size);
      const int32_t* row = block_table + int64_t(s) * mbps;
      for (int b = 0; b < used; ++b) {
        const int32_t id = row[b];
        if (id < 0 || id >= num_blocks) check_flag(report, 1, uint32_t(int64_t(s) * mbps + b));
      }
    }
  }
}

void launch_check_indices(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* block_table,
                          int32_t batch, int32_t mbps, const int32_t* context_lens, const int32_t* cu_q,
                          const int32_t* cu_k, int32_t num_blocks, int32_t block_size, uint32_t* report,
                          hipStream_t stream) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(64), 0, stream, report);
  const int64_t work = num_tokens > batch + 1 ? int64_t(num_tokens) : int64_t(batch) + 1;
  const int64_t blocks = (work + kCheckThreads - 1) / kCheckThreads;
  const int grid = int(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(check_indices_kernel, dim3(grid), dim3(kCheckThreads), 0, stream, slot_mapping,
                     num_tokens, block_table, batch, mbps, context_lens, cu_q, cu_k, num_blocks, block_size,
                     report);
}

}  // namespace pa
