// Internal launchers behind the C ABI (pa_api.hip validates every argument before calling these).
#pragma once

#include "pa_common.h"

namespace pa {

void launch_build_metadata(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                           int32_t mbps, int32_t batch, int32_t total_q, int32_t block_size, int32_t* cu_q,
                           int32_t* cu_k, int32_t* ctx, int32_t* pos, int32_t* slot, hipStream_t stream);

void launch_metadata_store(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                           int32_t mbps, int32_t batch, int32_t total_q, int32_t block_size, int32_t* cu_q,
                           int32_t* cu_k, int32_t* ctx, int32_t* pos, int32_t* slot, const void* k,
                           int64_t k_stride_bytes, const void* v, int64_t v_stride_bytes, void* k_cache,
                           void* v_cache, int64_t row_bytes, int vec_bytes, hipStream_t stream);

void launch_check_indices(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* block_table,
                          int32_t batch, int32_t mbps, const int32_t* context_lens, const int32_t* cu_q,
                          const int32_t* cu_k, int32_t num_blocks, int32_t block_size, uint32_t* report,
                          hipStream_t stream);

void launch_store_kvcache(const void* k, int64_t k_stride_bytes, const void* v, int64_t v_stride_bytes,
                          void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                          int64_t row_bytes, int vec_bytes, hipStream_t stream);

void launch_norm_rope_store(const void* k, int64_t k_stride, const void* v, int64_t v_stride, const void* k_w,
                            const void* q, int64_t q_stride, const void* q_w, void* q_out, int32_t Hq, float eps,
                            const int32_t* positions, const float* cos_sin, int32_t max_position, void* k_cache,
                            void* v_cache, const int32_t* slot_mapping, int32_t num_tokens, int32_t Hkv,
                            int32_t D, bool bf16, hipStream_t stream);

int32_t sample_chunks(int32_t batch, int32_t vocab);
void launch_sample(const float* logits, int64_t row_stride, const float* temperatures, int32_t batch,
                   int32_t vocab, uint64_t seed, uint64_t offset, int32_t* tokens, void* workspace,
                   hipStream_t stream);

void launch_attn_generic(bool bf16, const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                         const int32_t* cu_q, const int32_t* cu_k, const int32_t* ctx_lens,
                         const int32_t* block_table, int32_t mbps, int32_t batch, int32_t rows, int32_t Hq,
                         int32_t Hkv, int32_t D, int32_t block_size, float scale, void* out, bool out_bf16,
                         hipStream_t stream);

void launch_decode_mfma(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                        const int32_t* ctx_lens, const int32_t* block_table, int32_t mbps, int32_t batch,
                        int32_t Hq, int32_t Hkv, int32_t block_size, float scale, void* out, bool out_bf16,
                        int32_t split_tokens, int32_t max_splits, void* workspace, hipStream_t stream);

// One partial slot of the balanced decode: m[16], l[16], O[16][128] floats (G <= 16); each worker owns two.
constexpr int kStreamSlotFloats = 16 + 16 + 16 * 128;
constexpr size_t decode_stream_workspace_bytes(int32_t n_workers) {
  return size_t(n_workers) * 2 * kStreamSlotFloats * sizeof(float);
}

void launch_decode_stream(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                          const int32_t* ctx_lens, const int32_t* block_table, int32_t mbps, int32_t batch,
                          int32_t Hq, int32_t Hkv, int32_t block_size, float scale, void* out, bool out_bf16,
                          int32_t n_workers, void* workspace, hipStream_t stream, const void* k_new = nullptr,
                          int64_t k_new_stride = 0, const void* v_new = nullptr, int64_t v_new_stride = 0);

void launch_prefill_mfma(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                         const int32_t* cu_q, const int32_t* cu_k, const int32_t* block_table, int32_t mbps,
                         int32_t batch, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq,
                         int32_t Hkv, int32_t block_size, float scale, void* out, bool out_bf16, void* workspace,
                         hipStream_t stream);
// Key splits the prefill kernel uses for these host sizes, and the workspace its partials need (0 for one split).
int32_t prefill_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq);
size_t prefill_mfma_workspace_bytes(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq);


}  // namespace pa
