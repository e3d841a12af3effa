// The C ABI: argument checks on the host, kernel choice, launch. No allocation, no synchronisation, no reads of
// device memory; every error that the host can see is returned before anything is launched.
#include <mutex>

#include "../../include/pa.h"
#include "pa_launch.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int64_t kInt32Max = 2147483647;

bool aligned(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % uintptr_t(bytes)) == 0; }

bool valid_dtype(pa_dtype d) { return d == PA_F32 || d == PA_BF16; }

int elem_bytes(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }

bool valid_head_dim(int32_t d) { return d > 0 && d <= 256 && d % 8 == 0; }

pa_status launched() { return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// Widest access (16, 8, 4 or 2 bytes, at least the element size) that every row start and the row length allow
// for a K/V row copy; 0 when even the element size does not (misaligned element pointers).
int store_vec(const void* k, int64_t k_stride_bytes, const void* v, int64_t v_stride_bytes, const void* k_cache,
              const void* v_cache, int64_t row_bytes, int elem) {
  for (int vec = 16; vec >= elem; vec >>= 1)
    if (row_bytes % vec == 0 && k_stride_bytes % vec == 0 && v_stride_bytes % vec == 0 && aligned(k, vec) &&
        aligned(v, vec) && aligned(k_cache, vec) && aligned(v_cache, vec))
      return vec;
  return 0;
}

// Keys per decode split chosen from host sizes only: about 32k work items for contexts at half the table's
// capacity, clamped to [256, 4096] keys and rounded to a power of two (a multiple of 32).
int32_t auto_split(int32_t batch, int32_t num_kv_heads, int32_t mbps, int32_t block_size) {
  const int64_t max_len = int64_t(mbps) * block_size;
  const int64_t head_keys = int64_t(batch) * num_kv_heads * (max_len / 2 + 1);
  int64_t want = head_keys / 32768;
  int32_t split = 256;
  while (split < 4096 && split < want) split *= 2;
  return split;
}

int32_t max_splits_for(int32_t mbps, int32_t block_size, int32_t split) {
  const int64_t max_len = int64_t(mbps) * block_size;
  return int32_t((max_len + split - 1) / split);
}

bool decode_uses_mfma(pa_dtype dtype, int32_t Hq, int32_t Hkv, int32_t D) {
  return dtype == PA_BF16 && D == 128 && Hq / Hkv <= 16;
}

// Workers of the balanced decode (split_tokens == 0), one wave each: one and a half rounds of the 2048 that fit
// at once (two waves per SIMD of the 256 CUs). Measured fastest of 2048 to 8192 on both short mixed and long
// contexts: later workers fill the slots of early finishers, and slices stay long.
#ifndef PA_STREAM_WORKERS
#define PA_STREAM_WORKERS 3072
#endif
constexpr int32_t kStreamWorkers = PA_STREAM_WORKERS;

// The balanced decode takes split_tokens == 0 when its kernel fits the sizes: D = 128, at most 16 query heads per
// KV head (one partial slot holds 16 rows), at least one worker per KV head, 32-key tiles inside a block, a batch
// whose prefix sums fit in LDS (4096 sequences), and padded lengths whose sum over the batch fits the int32
// prefix sums.
bool decode_uses_stream(int32_t split_tokens, int32_t Hq, int32_t Hkv, int32_t D, int32_t mbps, int32_t block_size,
                        int32_t batch) {
  const int64_t padded_max = (int64_t(mbps) * block_size + 31) & ~int64_t(31);
  return split_tokens == 0 && D == 128 && Hq / Hkv <= 16 && Hkv <= kStreamWorkers && block_size % 32 == 0 &&
         batch <= 4096 && int64_t(batch) * padded_max < (int64_t(1) << 31);
}

// Argument checks of pa_decode_append and pa_decode_append_noalloc (everything but the workspace).
pa_status check_decode_append(const void* q, int64_t q_tok_stride, const void* k_new, int64_t k_tok_stride,
                              const void* v_new, int64_t v_tok_stride, const void* k_cache, const void* v_cache,
                              const int32_t* num_cached, const int32_t* block_table, int32_t max_blocks_per_seq,
                              int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t num_blocks, int32_t block_size, float softmax_scale, pa_dtype dtype,
                              const void* out, pa_dtype out_dtype) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype) || !valid_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || block_size <= 0 ||
      num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if (q_tok_stride < int64_t(num_heads) * head_dim || k_tok_stride < row || v_tok_stride < row) return PA_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !num_cached || !block_table || !out) return PA_ERR_NULL;
  if (!decode_uses_mfma(dtype, num_heads, num_kv_heads, head_dim) ||
      !decode_uses_stream(0, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size, batch))
    return PA_ERR_UNSUPPORTED;
  if (q_tok_stride % 8 || k_tok_stride % 8 || v_tok_stride % 8 || !aligned(q, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

// The scratch of pa_decode_append_noalloc, for callers that cannot allocate: the balanced decode's partial slots
// (kStreamWorkers workers x 2 slots x kStreamSlotFloats floats = 51.1 MB), one array per GPU the library runs on,
// held until the process ends. Its contents never need clearing (every partial the merge reads was written by the
// same call), and calls that overlap on one GPU share it and race.
constexpr size_t kScratchBytes = size_t(kStreamWorkers) * 2 * pa::kStreamSlotFloats * sizeof(float);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The array's device address per device, resolved once with that device current (host code never passes the
// array's name itself to a kernel: on the host it is only a stand-in for the symbol).
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

pa_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  if (stream) {  // the kernels run on the stream's device: it must be the current one, whose address is resolved
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return PA_ERR_LAUNCH;
    if (sdev != dev) return PA_ERR_SHAPE;
  }
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: dtype or head_dim not supported";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: kernel launch failed";
  }
  return "unknown pa_status";
}

int pa_version(void) { return kVersion; }

pa_status pa_build_metadata(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                            int32_t max_blocks_per_seq, int32_t batch, int32_t total_q, int32_t num_blocks,
                            int32_t block_size, int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                            int32_t* context_lens, int32_t* positions, int32_t* slot_mapping, void* stream) {
  if (batch < 0 || batch > 4096 || total_q < 0 || block_size <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  if (batch == 0) return total_q == 0 ? PA_OK : PA_ERR_SHAPE;
  if (max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (!num_cached || !num_new || !block_table || !cu_seqlens_q || !cu_seqlens_k || !context_lens)
    return PA_ERR_NULL;
  if (total_q > 0 && (!positions || !slot_mapping)) return PA_ERR_NULL;
  pa::launch_build_metadata(num_cached, num_new, block_table, max_blocks_per_seq, batch, total_q, block_size,
                            cu_seqlens_q, cu_seqlens_k, context_lens, positions, slot_mapping,
                            static_cast<hipStream_t>(stream));
  return launched();
}

pa_status pa_store_kvcache(const void* k, int64_t k_tok_stride, const void* v, int64_t v_tok_stride,
                           void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                           pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
    return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if (k_tok_stride < row || v_tok_stride < row) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  const int eb = elem_bytes(dtype);
  const int vec = store_vec(k, k_tok_stride * eb, v, v_tok_stride * eb, k_cache, v_cache, row * eb, eb);
  if (!vec) return PA_ERR_SHAPE;  // misaligned element pointers
  pa::launch_store_kvcache(k, k_tok_stride * eb, v, v_tok_stride * eb, k_cache, v_cache, slot_mapping, num_tokens,
                           row * eb, vec, static_cast<hipStream_t>(stream));
  return launched();
}

pa_status pa_build_metadata_store(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, int32_t batch, int32_t total_q, int32_t num_blocks,
                                  int32_t block_size, int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                                  int32_t* context_lens, int32_t* positions, int32_t* slot_mapping, const void* k,
                                  int64_t k_tok_stride, const void* v, int64_t v_tok_stride, void* k_cache,
                                  void* v_cache, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                  void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
  if (batch < 0 || batch > 4096 || total_q < 0 || block_size <= 0 || num_blocks <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0)
    return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if (k_tok_stride < row || v_tok_stride < row) return PA_ERR_SHAPE;
  if (batch == 0) return total_q == 0 ? PA_OK : PA_ERR_SHAPE;
  if (max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (!num_cached || !num_new || !block_table || !cu_seqlens_q || !cu_seqlens_k || !context_lens)
    return PA_ERR_NULL;
  if (total_q > 0 && (!positions || !slot_mapping || !k || !v || !k_cache || !v_cache)) return PA_ERR_NULL;
  const int eb = elem_bytes(dtype);
  int vec = eb;
  if (total_q > 0) {
    vec = store_vec(k, k_tok_stride * eb, v, v_tok_stride * eb, k_cache, v_cache, row * eb, eb);
    if (!vec) return PA_ERR_SHAPE;
  }
  pa::launch_metadata_store(num_cached, num_new, block_table, max_blocks_per_seq, batch, total_q, block_size,
                            cu_seqlens_q, cu_seqlens_k, context_lens, positions, slot_mapping, k, k_tok_stride * eb,
                            v, v_tok_stride * eb, k_cache, v_cache, row * eb, vec,
                            static_cast<hipStream_t>(stream));
  return launched();
}

pa_status pa_check_indices(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* block_table,
                           int32_t batch, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_blocks,
                           int32_t block_size, uint32_t* report, void* stream) {
  if (num_tokens < 0 || batch < 0 || num_blocks <= 0 || block_size <= 0) return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  if (context_lens && cu_seqlens_k) return PA_ERR_SHAPE;  // one source of key lengths
  if (!report || !aligned(report, 4)) return PA_ERR_NULL;
  if (num_tokens > 0 && !slot_mapping && !cu_seqlens_q) return PA_ERR_NULL;
  if (batch > 0 && (context_lens || cu_seqlens_k)) {
    if (!block_table) return PA_ERR_NULL;
    if (max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  }
  pa::launch_check_indices(num_tokens > 0 ? slot_mapping : nullptr, num_tokens, block_table, batch,
                           max_blocks_per_seq, context_lens, cu_seqlens_q, cu_seqlens_k, num_blocks, block_size,
                           report, static_cast<hipStream_t>(stream));
  return launched();
}

pa_status pa_norm_rope_store_kvcache(const void* k, int64_t k_tok_stride, const void* v, int64_t v_tok_stride,
                                     const void* k_norm_weight, const void* q, int64_t q_tok_stride,
                                     const void* q_norm_weight, void* q_out, int32_t num_heads, float rms_eps,
                                     const int32_t* positions, const float* cos_sin, int32_t max_position,
                                     void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                     int32_t block_size, pa_dtype dtype, void* stream) {
  if (!valid_dtype(dtype)) return PA_ERR_UNSUPPORTED;
  if (head_dim < 16 || head_dim > 512 || (head_dim & (head_dim - 1))) return PA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0 || max_position <= 0)
    return PA_ERR_SHAPE;
  if (!(rms_eps >= 0.f) || rms_eps > 3.0e38f) return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if (k_tok_stride < row || v_tok_stride < row) return PA_ERR_SHAPE;
  if (q && (num_heads <= 0 || q_tok_stride < int64_t(num_heads) * head_dim)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_norm_weight || !positions || !cos_sin || !k_cache || !v_cache || !slot_mapping)
    return PA_ERR_NULL;
  if (q && (!q_norm_weight || !q_out)) return PA_ERR_NULL;
  const int eb = elem_bytes(dtype);
  if ((k_tok_stride * eb) % 16 || (v_tok_stride * eb) % 16 || (q && (q_tok_stride * eb) % 16)) return PA_ERR_SHAPE;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_norm_weight, 16) || !aligned(cos_sin, 16) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return PA_ERR_SHAPE;
  if (q && (!aligned(q, 16) || !aligned(q_norm_weight, 16) || !aligned(q_out, 16))) return PA_ERR_SHAPE;
  pa::launch_norm_rope_store(k, k_tok_stride, v, v_tok_stride, k_norm_weight, q, q_tok_stride, q_norm_weight, q_out,
                             num_heads, rms_eps, positions, cos_sin, max_position, k_cache, v_cache, slot_mapping,
                             num_tokens, num_kv_heads, head_dim, dtype == PA_BF16,
                             static_cast<hipStream_t>(stream));
  return launched();
}

size_t pa_sample_workspace_bytes(int32_t batch, int32_t vocab) {
  if (batch <= 0 || vocab <= 0) return 0;
  return size_t(batch) * pa::sample_chunks(batch, vocab) * 2 * sizeof(float);
}

pa_status pa_sample(const float* logits, int64_t row_stride, const float* temperatures, int32_t batch,
                    int32_t vocab, uint64_t seed, uint64_t offset, int32_t* tokens, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (batch < 0 || batch > 65535 || vocab <= 0 || row_stride < vocab) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!logits || !temperatures || !tokens || !workspace) return PA_ERR_NULL;
  if (workspace_bytes < pa_sample_workspace_bytes(batch, vocab)) return PA_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return PA_ERR_SHAPE;
  pa::launch_sample(logits, row_stride, temperatures, batch, vocab, seed, offset, tokens, workspace,
                    static_cast<hipStream_t>(stream));
  return launched();
}

size_t pa_prefill_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, int32_t max_seqlen_q,
                                  int32_t max_seqlen_k) {
  // only the matrix-core kernel (head_dim 128) uses a workspace: the partials of its key splits
  if (batch <= 0 || num_heads <= 0 || head_dim != 128 || max_seqlen_q <= 0 || max_seqlen_k <= 0) return 0;
  return pa::prefill_mfma_workspace_bytes(batch, max_seqlen_q, max_seqlen_k, num_heads);
}

pa_status pa_prefill_varlen(const void* q, int64_t q_tok_stride, const void* k_cache, const void* v_cache,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* block_table,
                            int32_t max_blocks_per_seq, int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t num_blocks, int32_t block_size, float softmax_scale, pa_dtype dtype,
                            void* out, pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype) || !valid_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (batch < 0 || total_q < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      block_size <= 0 || num_blocks <= 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  if (q_tok_stride < int64_t(num_heads) * head_dim) return PA_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f) return PA_ERR_SHAPE;
  if (batch == 0 || total_q == 0) return PA_OK;
  if (max_seqlen_q <= 0 || max_blocks_per_seq <= 0 || int64_t(max_seqlen_k) > int64_t(max_blocks_per_seq) * block_size)
    return PA_ERR_SHAPE;
  // grids: heads are a y dimension (at most 65535) of the per-(row, head) kernels, and the matrix-core kernel's
  // flat grid of (sequence, query tile, head, key split) workgroups must fit an int
  if (num_heads > 65535 ||
      int64_t(batch) * ((int64_t(max_seqlen_q) + 127) / 128) * num_heads *
              pa::prefill_splits(batch, max_seqlen_q, max_seqlen_k, num_heads) > (int64_t(1) << 30))
    return PA_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !cu_seqlens_k || !block_table || !out) return PA_ERR_NULL;
  if (workspace_bytes < pa_prefill_workspace_bytes(batch, num_heads, head_dim, max_seqlen_q, max_seqlen_k))
    return PA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool out_bf16 = out_dtype == PA_BF16;
  const bool mfma = dtype == PA_BF16 && head_dim == 128 && q_tok_stride % 8 == 0 && aligned(q, 16) &&
                    aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(out, 16);
  if (mfma) {
    if (pa::prefill_splits(batch, max_seqlen_q, max_seqlen_k, num_heads) > 1 && (!workspace || !aligned(workspace, 16)))
      return PA_ERR_NULL;
    pa::launch_prefill_mfma(q, q_tok_stride, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_table,
                            max_blocks_per_seq, batch, total_q, max_seqlen_q, max_seqlen_k, num_heads, num_kv_heads,
                            block_size, softmax_scale, out, out_bf16, workspace, st);
  } else {
    pa::launch_attn_generic(dtype == PA_BF16, q, q_tok_stride, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k,
                            nullptr, block_table, max_blocks_per_seq, batch, total_q, num_heads, num_kv_heads,
                            head_dim, block_size, softmax_scale, out, out_bf16, st);
  }
  return launched();
}

int32_t pa_decode_split_tokens(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int32_t block_size) {
  (void)num_heads; (void)head_dim;
  if (batch <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 256;
  return auto_split(batch, num_kv_heads, max_blocks_per_seq, block_size);
}

size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t block_size, int32_t split_tokens) {
  if (batch <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0 || split_tokens < 0)
    return 0;
  if (decode_uses_stream(split_tokens, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size, batch))
    return pa::decode_stream_workspace_bytes(kStreamWorkers);
  const int32_t split = split_tokens > 0 ? split_tokens
                                         : auto_split(batch, num_kv_heads, max_blocks_per_seq, block_size);
  const int32_t ms = max_splits_for(max_blocks_per_seq, block_size, split);
  if (ms <= 1) return 0;
  return size_t(batch) * num_heads * ms * (size_t(head_dim) * sizeof(float) + 2 * sizeof(float));
}

pa_status pa_decode(const void* q, int64_t q_tok_stride, const void* k_cache, const void* v_cache,
                    const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks_per_seq,
                    int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                    int32_t block_size, float softmax_scale, pa_dtype dtype, void* out, pa_dtype out_dtype,
                    int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype) || !valid_head_dim(head_dim)) return PA_ERR_UNSUPPORTED;
  if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 || block_size <= 0 ||
      num_blocks <= 0 || split_tokens < 0 || split_tokens % 32 != 0)
    return PA_ERR_SHAPE;
  if (int64_t(num_blocks) * block_size > kInt32Max) return PA_ERR_SHAPE;
  if (q_tok_stride < int64_t(num_heads) * head_dim) return PA_ERR_SHAPE;
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (max_blocks_per_seq <= 0 || batch > 65535 || num_heads > 65535) return PA_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !context_lens || !block_table || !out) return PA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool out_bf16 = out_dtype == PA_BF16;
  const bool mfma = decode_uses_mfma(dtype, num_heads, num_kv_heads, head_dim) && q_tok_stride % 8 == 0 &&
                    aligned(q, 16) && aligned(k_cache, 16) && aligned(v_cache, 16) && aligned(out, 16);
  if (mfma && decode_uses_stream(split_tokens, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size, batch)) {
    const size_t need = pa::decode_stream_workspace_bytes(kStreamWorkers);
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!workspace || !aligned(workspace, 16)) return PA_ERR_NULL;
    pa::launch_decode_stream(q, q_tok_stride, k_cache, v_cache, context_lens, block_table, max_blocks_per_seq, batch,
                             num_heads, num_kv_heads, block_size, softmax_scale, out, out_bf16, kStreamWorkers,
                             workspace, st);
  } else if (mfma) {
    const int32_t split = split_tokens > 0 ? split_tokens
                                           : auto_split(batch, num_kv_heads, max_blocks_per_seq, block_size);
    const int32_t ms = max_splits_for(max_blocks_per_seq, block_size, split);
    if (ms > 65535 || int64_t(batch) * ms * num_kv_heads > (int64_t(1) << 30)) return PA_ERR_SHAPE;
    const size_t need = pa_decode_workspace_bytes(batch, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                                                  block_size, split);
    if (workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (need > 0 && (!workspace || !aligned(workspace, 16))) return PA_ERR_NULL;
    pa::launch_decode_mfma(q, q_tok_stride, k_cache, v_cache, context_lens, block_table, max_blocks_per_seq, batch,
                           num_heads, num_kv_heads, block_size, softmax_scale, out, out_bf16, split, ms, workspace,
                           st);
  } else {
    pa::launch_attn_generic(dtype == PA_BF16, q, q_tok_stride, k_cache, v_cache, nullptr, nullptr, context_lens,
                            block_table, max_blocks_per_seq, batch, batch, num_heads, num_kv_heads, head_dim,
                            block_size, softmax_scale, out, out_bf16, st);
  }
  return launched();
}

pa_status pa_decode_append(const void* q, int64_t q_tok_stride, const void* k_new, int64_t k_tok_stride,
                           const void* v_new, int64_t v_tok_stride, void* k_cache, void* v_cache,
                           const int32_t* num_cached, const int32_t* block_table, int32_t max_blocks_per_seq,
                           int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t num_blocks, int32_t block_size, float softmax_scale, pa_dtype dtype, void* out,
                           pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  const pa_status st = check_decode_append(q, q_tok_stride, k_new, k_tok_stride, v_new, v_tok_stride, k_cache,
                                           v_cache, num_cached, block_table, max_blocks_per_seq, batch, num_heads,
                                           num_kv_heads, head_dim, num_blocks, block_size, softmax_scale, dtype, out,
                                           out_dtype);
  if (st != PA_OK || batch == 0) return st;
  const size_t need = pa::decode_stream_workspace_bytes(kStreamWorkers);
  if (workspace_bytes < need) return PA_ERR_WORKSPACE;
  if (!workspace || !aligned(workspace, 16)) return PA_ERR_NULL;
  pa::launch_decode_stream(q, q_tok_stride, k_cache, v_cache, num_cached, block_table, max_blocks_per_seq, batch,
                           num_heads, num_kv_heads, block_size, softmax_scale, out, out_dtype == PA_BF16,
                           kStreamWorkers, workspace, static_cast<hipStream_t>(stream), k_new, k_tok_stride, v_new,
                           v_tok_stride);
  return launched();
}

pa_status pa_decode_append_noalloc(const void* q, int64_t q_tok_stride, const void* k_new, int64_t k_tok_stride,
                                   const void* v_new, int64_t v_tok_stride, void* k_cache, void* v_cache,
                                   const int32_t* num_cached, const int32_t* block_table, int32_t max_blocks_per_seq,
                                   int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t num_blocks, int32_t block_size, float softmax_scale, pa_dtype dtype,
                                   void* out, pa_dtype out_dtype, void* stream) {
  const pa_status st = check_decode_append(q, q_tok_stride, k_new, k_tok_stride, v_new, v_tok_stride, k_cache,
                                           v_cache, num_cached, block_table, max_blocks_per_seq, batch, num_heads,
                                           num_kv_heads, head_dim, num_blocks, block_size, softmax_scale, dtype, out,
                                           out_dtype);
  if (st != PA_OK || batch == 0) return st;
  static_assert(pa::decode_stream_workspace_bytes(kStreamWorkers) <= kScratchBytes, "scratch too small");
  if (pa::decode_stream_workspace_bytes(kStreamWorkers) > kScratchBytes) return PA_ERR_WORKSPACE;
  void* part = nullptr;
  const pa_status sc = scratch_for(static_cast<hipStream_t>(stream), &part);
  if (sc != PA_OK) return sc;
  pa::launch_decode_stream(q, q_tok_stride, k_cache, v_cache, num_cached, block_table, max_blocks_per_seq, batch,
                           num_heads, num_kv_heads, block_size, softmax_scale, out, out_dtype == PA_BF16,
                           kStreamWorkers, part, static_cast<hipStream_t>(stream), k_new, k_tok_stride, v_new,
                           v_tok_stride);
  return launched();
}

}  // extern "C"
