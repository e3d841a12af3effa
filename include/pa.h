/*
 * pa.h -- C ABI of the paged-KV attention step for AMD MI355X (gfx950).
 *
 * The step is the attention layer's work per decoder layer in a paged-KV inference engine: write the new
 * tokens' K/V into a block-paged cache, then run attention over that cache through per-sequence block tables,
 * either as variable-length causal prefill or as one-query-per-sequence decode ("一个 prompt 的一生" §3.3.2 and
 * the summary of §4: store_kvcache, then flash_attn; "Nano-vLLM 架构详解" §2.4, Attention stage, and §3.2,
 * Attention 运算 for the argument formats).
 *
 * Conventions shared by every entry point
 *   - Pointers marked (device) are HIP device pointers; (host) are host pointers. The caller owns every buffer.
 *     The library allocates nothing, keeps no per-call state and may be called from several host threads.
 *   - Every call only enqueues work on `stream` (a hipStream_t, NULL = the default stream) and returns; it does
 *     not synchronise and reads no device memory on the host. Grids depend only on host scalars, so a captured
 *     graph can be replayed with new lengths and tables as long as those scalars stay the same.
 *   - Cache of one layer, for K and for V separately: [num_blocks, block_size, num_kv_heads, head_dim],
 *     contiguous ("一个 prompt 的一生" §2.2.3, the pool `torch.empty(2, num_layers, num_blocks, block_size,
 *     num_kv_heads, head_dim)` whose per-layer views are handed to the layer). Because it is contiguous in
 *     (block, offset), a slot s = block_id * block_size + offset addresses row s of a flat
 *     [num_blocks * block_size, num_kv_heads, head_dim] view ("Nano-vLLM 架构详解" §1, Step2).
 *   - Index arrays are int32. A block table is [batch, max_blocks_per_seq], row s listing sequence s's physical
 *     blocks in logical order, padded with -1 ("Nano-vLLM 架构详解" §3.2, block_tables format). Only the first
 *     ceil(k_len / block_size) entries of a row are read.
 *   - Query head h reads KV head h / (num_heads / num_kv_heads) (contiguous GQA groups).
 *   - A query token at absolute position p sees keys 0..p. In prefill, the q_len new tokens of a sequence with
 *     k_len keys are at positions k_len - q_len .. k_len - 1 (a chunk continues at the number of cached tokens,
 *     "Nano-vLLM 源码逐行解析 第2篇", sequence.py counter example).
 *   - Attention inputs are read from the cache only: call pa_store_kvcache for the new tokens first.
 *   - Device-side indices are trusted: out-of-range block ids or slots, duplicate slots within one store and
 *     k_len < q_len are undefined behaviour. Cache contents outside each sequence's first k_len positions are
 *     never read, so they may hold any bits (NaN included).
 *   - Return value: PA_OK, or an error code for a problem the host can see before launching (nothing is
 *     launched then); PA_ERR_LAUNCH if a launch failed. batch == 0 or no tokens is a no-op returning PA_OK.
 *
 * softmax_scale must be positive and finite (PA_ERR_SHAPE otherwise).
 * Supported: dtype PA_BF16 or PA_F32 for Q/K/V and cache (same for all); out_dtype PA_F32 or PA_BF16
 * (round to nearest even); head_dim a multiple of 8 and at most 256 (bf16, head_dim 128 and a GQA group of at
 * most 16 take the matrix-core kernels; other shapes take a plain vector kernel, one wave per query row and
 * head, that is a correctness path: on MI355X it runs a bf16 head_dim-64 prefill at about 2.3 TFLOP/s and a
 * head_dim-64 decode at about 0.01 of the HBM rate (83 GB/s), against 650-970 TFLOP/s and 0.7-0.8 of HBM for
 * the matrix-core kernels).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* inconsistent sizes (e.g. num_heads % num_kv_heads != 0, negative sizes) */
  PA_ERR_UNSUPPORTED = 3, /* dtype / head_dim combination not built */
  PA_ERR_WORKSPACE = 4,   /* workspace smaller than the *_workspace_bytes query asks for */
  PA_ERR_LAUNCH = 5       /* the HIP runtime reported an error when launching */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Human-readable name of a status code (static string). */
const char* pa_status_str(pa_status s);

/* Library version: major * 10000 + minor * 100 + patch. */
int pa_version(void);

/*
 * pa_build_metadata -- per-step metadata of the paged cache, computed on the device.
 *
 * Sequence s computes num_new[s] tokens at absolute positions num_cached[s] .. num_cached[s] + num_new[s] - 1,
 * after which it has k_len = num_cached[s] + num_new[s] keys. Outputs (device, int32):
 *   cu_seqlens_q [batch+1]  prefix sums of num_new (cu_seqlens_q[0] = 0)
 *   cu_seqlens_k [batch+1]  prefix sums of k_len
 *   context_lens [batch]    k_len
 *   positions    [total_q]  absolute position of each flattened new token
 *   slot_mapping [total_q]  block_table[s][pos / block_size] * block_size + pos % block_size, or -1 when pos
 *                           is negative or beyond the row (pos / block_size >= max_blocks_per_seq)
 * This is the flattening of the prepare_prefill example ("一个 prompt 的一生" §3.3.2: positions, cu_seqlens_q and
 * slot_mapping for two sequences with block_size 4) and the slot formula ("Nano-vLLM 架构详解" §1, Step2). For
 * a decode step pass num_new = 1 for every sequence.
 * total_q (host) must equal sum(num_new); batch <= 4096; num_blocks * block_size < 2^31.
 * Inputs num_cached, num_new [batch] and block_table [batch, max_blocks_per_seq] are device pointers.
 */
pa_status pa_build_metadata(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                            int32_t max_blocks_per_seq, int32_t batch, int32_t total_q, int32_t num_blocks,
                            int32_t block_size, int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                            int32_t* context_lens, int32_t* positions, int32_t* slot_mapping, void* stream);

/*
 * pa_store_kvcache -- write each new token's K and V into the cache at its slot.
 *
 * For every token i < num_tokens with slot_mapping[i] >= 0: flat_k_cache[slot_mapping[i]] = k[i] and
 * flat_v_cache[slot_mapping[i]] = v[i] (a bit copy of num_kv_heads * head_dim elements). Negative slots are
 * skipped. The write knows nothing about pages: it only follows slot_mapping ("一个 prompt 的一生" §3.3.2 and
 * §4; "Nano-vLLM 架构详解" §3.2, KV cache 写入函数).
 *   k, v        (device) [num_tokens, num_kv_heads, head_dim]; token i starts at element i * *_tok_stride and
 *               its num_kv_heads * head_dim elements are contiguous
 *   k_cache, v_cache (device) [num_blocks, block_size, num_kv_heads, head_dim]
 *   slot_mapping (device) [num_tokens]
 */
pa_status pa_store_kvcache(const void* k, int64_t k_tok_stride, const void* v, int64_t v_tok_stride,
                           void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                           pa_dtype dtype, void* stream);

/*
 * pa_build_metadata_store -- pa_build_metadata followed by pa_store_kvcache with its slot_mapping, in one launch.
 *
 * Computes every output of pa_build_metadata (same arguments, meanings and limits) and writes each new token's
 * K and V rows to the slot it computed, exactly as pa_store_kvcache would (bit copy, negative slots skipped). The
 * two steps run in this order at the start of every step of the engine ("一个 prompt 的一生" §3.3.2 and §4:
 * prepare the metadata, then each layer's store by slot_mapping); one launch saves the second launch and the wait
 * between them when the new K/V rows are already at hand. Token t's rows are k[t], v[t] in the flattened order of
 * the new tokens (sequence by sequence).
 *   k, v, k_tok_stride, v_tok_stride, k_cache, v_cache, num_kv_heads, head_dim, dtype as for pa_store_kvcache;
 *   they may be NULL when total_q == 0.
 */
pa_status pa_build_metadata_store(const int32_t* num_cached, const int32_t* num_new, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, int32_t batch, int32_t total_q, int32_t num_blocks,
                                  int32_t block_size, int32_t* cu_seqlens_q, int32_t* cu_seqlens_k,
                                  int32_t* context_lens, int32_t* positions, int32_t* slot_mapping, const void* k,
                                  int64_t k_tok_stride, const void* v, int64_t v_tok_stride, void* k_cache,
                                  void* v_cache, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                                  void* stream);

/*
 * pa_check_indices -- validate the index arrays of a call before making it (a debugging aid).
 *
 * The path trusts the indices it is given: an out-of-range slot or block id, or a length beyond the table, is
 * undefined behaviour there. This call reads only the index arrays (never the caches) and counts, per kind,
 * the entries that would make the path go out of bounds or compute the wrong rows:
 *   PA_CHECK_SLOT   slot_mapping[t] >= num_blocks * block_size (negative slots mean "skip" and are valid)
 *   PA_CHECK_TABLE  a used block-table entry (entries 0 .. ceil(k_len / block_size) - 1 of a sequence) outside
 *                   [0, num_blocks)
 *   PA_CHECK_LEN    a key length k_len < 0 or > max_blocks_per_seq * block_size (its table row is then not read)
 *   PA_CHECK_CU     cu_seqlens_q / cu_seqlens_k not starting at 0 or decreasing, or cu_seqlens_q[batch] !=
 *                   num_tokens
 *   PA_CHECK_Q_GT_K q_len > k_len for a sequence (prefill)
 * The key lengths come from context_lens (decode) or from cu_seqlens_k (prefill); give at most one of them.
 * Every array may be NULL to skip its checks (block_table is needed when key lengths are given).
 *   slot_mapping  (device) [num_tokens] or NULL
 *   block_table   (device) [batch, max_blocks_per_seq]
 *   context_lens  (device) [batch] or NULL; cu_seqlens_q, cu_seqlens_k (device) [batch + 1] or NULL
 *   report        (device) uint32 [2 * PA_CHECK_KINDS], written by the call: report[k] is the number of errors
 *                 of kind k, report[PA_CHECK_KINDS + k] the smallest offending index (token t, sequence s,
 *                 prefix index i, or s * max_blocks_per_seq + block for PA_CHECK_TABLE), 0xffffffff if none.
 * Asynchronous like every other call: read the report after the stream has passed it.
 */
typedef enum {
  PA_CHECK_SLOT = 0,
  PA_CHECK_TABLE = 1,
  PA_CHECK_LEN = 2,
  PA_CHECK_CU = 3,
  PA_CHECK_Q_GT_K = 4,
  PA_CHECK_KINDS = 5
} pa_check_kind;

pa_status pa_check_indices(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* block_table,
                           int32_t batch, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_blocks,
                           int32_t block_size, uint32_t* report, void* stream);

/*
 * pa_norm_rope_store_kvcache -- the layer's pre-attention step for the new tokens in one pass: k_norm, rotary
 * embedding and the store of K (and V) into the cache, plus q_norm and rotary embedding of Q when q is given.
 *
 * The layer runs q_norm -> k_norm -> rope -> store_kvcache before attention ("一个 prompt 的一生" §2.2.4, the
 * operators of one decoder layer), the rotation by table lookup (same page §3.3.2). Per token i and head h
 * (the pages name the steps; the formulas are the usual ones and are stated here):
 *   y = x / sqrt(mean over d of x[d]^2 + rms_eps) * weight[d]                      (RMSNorm over head_dim)
 *   out[d]       = y[d] * cos[d] - y[d + D/2] * sin[d]    for d < D/2               (rotate half)
 *   out[d + D/2] = y[d + D/2] * cos[d] + y[d] * sin[d]
 * with cos = cos_sin[pos][0 .. D/2), sin = cos_sin[pos][D/2 .. D) and pos = positions[i] (clamped to
 * [0, max_position - 1]). For slot_mapping[i] >= 0 the rotated key goes to flat_k_cache[slot] and v[i] to
 * flat_v_cache[slot] unchanged; negative slots store nothing. Arithmetic is fp32; bf16 results are rounded to
 * nearest even.
 *   k, v           (device) [num_tokens, num_kv_heads, head_dim], token stride *_tok_stride elements
 *   k_norm_weight  (device) [head_dim], dtype
 *   q              (device) [num_tokens, num_heads, head_dim] or NULL (then q_norm_weight, q_out and
 *                  num_heads are ignored)
 *   q_norm_weight  (device) [head_dim]; q_out (device) [num_tokens, num_heads, head_dim], contiguous, dtype
 *   positions      (device) [num_tokens] int32; cos_sin (device) [max_position, head_dim] float32
 *   k_cache, v_cache, slot_mapping as for pa_store_kvcache
 * head_dim must be a power of two in 16 .. 512; rms_eps >= 0; every pointer and token stride 16-byte aligned.
 */
pa_status pa_norm_rope_store_kvcache(const void* k, int64_t k_tok_stride, const void* v, int64_t v_tok_stride,
                                     const void* k_norm_weight, const void* q, int64_t q_tok_stride,
                                     const void* q_norm_weight, void* q_out, int32_t num_heads, float rms_eps,
                                     const int32_t* positions, const float* cos_sin, int32_t max_position,
                                     void* k_cache, void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                                     int32_t block_size, pa_dtype dtype, void* stream);

/*
 * pa_prefill_varlen -- causal attention of the new tokens of `batch` sequences over the paged cache.
 *
 * For sequence s, rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of q attend to its
 * k_len = cu_seqlens_k[s+1] - cu_seqlens_k[s] keys read through block_table row s, with
 * O = softmax(q K^T * softmax_scale + causal mask) V computed with float32 accumulation. Argument formats are
 * FlashAttention's varlen ones ("Nano-vLLM 架构详解" §3.2, Attention 运算: Q (total_q, nheads, headdim), cache
 * (num_blocks, page_block_size, nheads_k, headdim), cu_seqlens (batch+1,), max_seqlen, block_tables).
 *   q            (device) [total_q, num_heads, head_dim]; token i starts at element i * q_tok_stride
 *   cu_seqlens_q, cu_seqlens_k (device) [batch+1], cu_seqlens_q[0] = 0 and cu_seqlens_q[batch] = total_q
 *   block_table  (device) [batch, max_blocks_per_seq]
 *   max_seqlen_q (host) >= every q_len; max_seqlen_k (host) >= every k_len; with total_q they size the grid
 *                (for up to 64 sequences the grid counts the row blocks total_q can hold, so a total_q below
 *                cu_seqlens_q[batch] would leave rows uncomputed: it is a contract violation, as a q shorter
 *                than the rows cu_seqlens_q names is)
 *   out          (device) [total_q, num_heads, head_dim], contiguous, out_dtype
 *   workspace    (device) at least pa_prefill_workspace_bytes(...) bytes (may be NULL when that is 0)
 * With few query tiles over long keys (a small chunk after a long cached prefix, as in chunked prefill: fewer
 * 128-row tiles times heads than the chip runs at once), the bf16 head_dim-128 kernel splits each tile's keys into
 * up to 32 ranges of at least 1024 keys, chosen from the host sizes alone, and a second launch merges the
 * ranges' partial results with the log-sum-exp rule; the workspace then holds those partials (scratch: its
 * contents do not matter between calls). Results agree to rounding with and without splits.
 * Precision of the bf16 head_dim-128 kernel: q K^T multiplies the bf16 inputs exactly (bf16 matrix cores, float32
 * accumulation); the softmax weights and V enter the PV product as fp16 (float32 accumulation). V is converted
 * from bf16 to fp16 rounding toward zero: exact for magnitudes in [2^-14, 65504] (a bf16 significand fits an
 * fp16 one); larger finite magnitudes become +-65504; magnitudes in [2^-24, 2^-14) become fp16 subnormals
 * (truncated toward zero) and smaller ones zero. The weights (at most 256 before normalisation) are rounded to
 * nearest fp16, and the normaliser is the sum of the rounded weights. Other dtypes and head sizes compute in
 * float32 throughout.
 */
pa_status pa_prefill_varlen(const void* q, int64_t q_tok_stride, const void* k_cache, const void* v_cache,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* block_table,
                            int32_t max_blocks_per_seq, int32_t batch, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t num_blocks, int32_t block_size, float softmax_scale, pa_dtype dtype,
                            void* out, pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pa_prefill_varlen needs for these host sizes: 0 unless the call splits its keys (then
 * batch * ceil(max_seqlen_q / 128) * 128 * num_heads * splits rows of 132 floats). The query sees no dtype: for
 * head_dim 128 it answers for the bf16 kernel, and an fp32 call of the same sizes leaves the workspace unused. */
size_t pa_prefill_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, int32_t max_seqlen_q,
                                  int32_t max_seqlen_k);

/*
 * pa_decode -- one query token per sequence over its context_lens[s] cached keys (the new token included).
 *
 * Same arithmetic as prefill with q_len = 1 (the query at position context_lens[s] - 1 sees every key). With
 * split_tokens > 0 the keys of each sequence are cut into splits of split_tokens; each split yields an
 * unnormalised partial output with its running max and sum, and a second pass merges the partials of a sequence
 * with the log-sum-exp rule. With split_tokens == 0 the library chooses: for head_dim 128, at most 16 query heads
 * per KV head and a block_size that is a multiple of 32, a balanced decode (a fixed set of workers, each taking an
 * equal share of all (KV head, key) work, partials of cut sequences merged the same way); otherwise splits of
 * pa_decode_split_tokens(...) keys. Results agree to rounding whatever the split. FlashAttention's
 * KV-cache format: q (batch, 1, nheads, headdim), cache_seqlens, block_tables ("Nano-vLLM 架构详解" §3.2).
 *   q            (device) [batch, num_heads, head_dim]; sequence s starts at element s * q_tok_stride
 *   context_lens (device) [batch], each >= 1 and <= max_blocks_per_seq * block_size
 *   block_table  (device) [batch, max_blocks_per_seq]
 *   split_tokens (host) keys per split, a multiple of 32, or 0 to let the library choose from the host sizes
 *   out          (device) [batch, num_heads, head_dim], contiguous, out_dtype
 *   workspace    (device) at least pa_decode_workspace_bytes(...) bytes for the same host sizes
 */
pa_status pa_decode(const void* q, int64_t q_tok_stride, const void* k_cache, const void* v_cache,
                    const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks_per_seq,
                    int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                    int32_t block_size, float softmax_scale, pa_dtype dtype, void* out, pa_dtype out_dtype,
                    int32_t split_tokens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_append -- the decode step with the new token's K and V given: store them, then decode.
 *
 * The same as pa_store_kvcache of k_new[s], v_new[s] at position num_cached[s] of sequence s (slot
 * block_table[s][pos / block_size] * block_size + pos % block_size, pos = num_cached[s]) followed by pa_decode
 * over context_lens[s] = num_cached[s] + 1 keys, in the balanced decode's two launches (instead of the metadata
 * and store launches followed by those two): the worker whose slice holds a pair's new key writes that head of
 * the new rows and then reads them as part of its slice. FlashAttention's decode call takes the new k, v the same way and updates the cache in place ("Nano-vLLM
 * 架构详解" §3.2, flash_attn_with_kvcache; the step is store then attention, "一个 prompt 的一生" §4).
 *   q      (device) [batch, num_heads, head_dim]; k_new, v_new (device) [batch, num_kv_heads, head_dim], token
 *          stride *_tok_stride elements (a multiple of 8), 16-byte aligned
 *   num_cached (device) [batch] int32: keys already in the cache; the table row must hold num_cached[s] + 1
 *   workspace at least pa_decode_workspace_bytes(batch, ..., split_tokens = 0) bytes
 * Taken for the shapes the balanced decode takes (bf16, head_dim 128, at most 16 query heads per KV head, block
 * size a multiple of 32, batch <= 4096, 16-byte aligned pointers); PA_ERR_UNSUPPORTED otherwise, before any
 * launch (then call pa_build_metadata_store and pa_decode). As in pa_decode the indices are trusted: the row's
 * entries up to position num_cached[s] must be valid block ids (pa_check_indices with context_lens =
 * num_cached + 1 checks them).
 */
pa_status pa_decode_append(const void* q, int64_t q_tok_stride, const void* k_new, int64_t k_tok_stride,
                           const void* v_new, int64_t v_tok_stride, void* k_cache, void* v_cache,
                           const int32_t* num_cached, const int32_t* block_table, int32_t max_blocks_per_seq,
                           int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t num_blocks, int32_t block_size, float softmax_scale, pa_dtype dtype, void* out,
                           pa_dtype out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_append_noalloc -- pa_decode_append for callers that cannot allocate device memory: code recorded
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc. Same arguments, semantics, shapes and
 * error codes as pa_decode_append, without the workspace: its partial results go to a scratch array of fixed
 * size (51.1 MB: 3072 workers x 2 slots x 2080 floats) that the library holds in device memory, one per GPU it runs
 * on, until the process ends. No call allocates (no hipMalloc, hipFree or allocating library routine); the first
 * call on a device resolves the array's device address for that device (make it before capturing a graph).
 * The stream must belong to the current device (else PA_ERR_SHAPE). The array's size does not depend on the
 * call's sizes (every shape pa_decode_append takes fits it); its contents never need clearing, and calls that
 * overlap on one GPU (two streams at once) share it and race: serialise them.
 */
pa_status pa_decode_append_noalloc(const void* q, int64_t q_tok_stride, const void* k_new, int64_t k_tok_stride,
                                   const void* v_new, int64_t v_tok_stride, void* k_cache, void* v_cache,
                                   const int32_t* num_cached, const int32_t* block_table, int32_t max_blocks_per_seq,
                                   int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t num_blocks, int32_t block_size, float softmax_scale, pa_dtype dtype,
                                   void* out, pa_dtype out_dtype, void* stream);

/* Keys per split pa_decode uses for these host sizes when split_tokens == 0 and the balanced decode does not
 * apply. */
int32_t pa_decode_split_tokens(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_blocks_per_seq, int32_t block_size);

/* Workspace bytes pa_decode needs for these host sizes and split_tokens (0 = the library's choice). */
size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t block_size, int32_t split_tokens);

/*
 * pa_sample -- the next token of each sequence from its logits: temperature, softmax and Gumbel-max.
 *
 * The sampler divides the logits by the temperature, takes the softmax and draws with Gumbel-max ("Nano-vLLM
 * 架构详解" §2.4, sampling stage; "一个 prompt 的一生" §4). Since argmax_i (log softmax(l/T)_i + g_i) does not depend
 * on the softmax's normaliser, tokens[b] = argmax_i (logits[b][i] * (1 / T_b) + g_i) with g_i = -ln(-ln u_i);
 * T_b <= 0 is greedy (argmax_i logits[b][i]); ties go to the lower index. The uniforms come from Philox4x32-10
 * (Salmon et al., SC 2011) with counter (i / 4, b, offset mod 2^32, offset div 2^32) and key (seed mod 2^32,
 * seed div 2^32), word i % 4, u = ((x >> 9) + 1/2) * 2^-23: the same (seed, offset) gives the same tokens, and a
 * new offset per step gives fresh draws.
 *   logits       (device) [batch, vocab] float32, row b at element b * row_stride
 *   temperatures (device) [batch] float32
 *   tokens       (device) [batch] int32, written
 *   workspace    (device) at least pa_sample_workspace_bytes(batch, vocab) bytes
 * batch <= 65535. A row whose logits are all NaN gets token 0.
 */
pa_status pa_sample(const float* logits, int64_t row_stride, const float* temperatures, int32_t batch,
                    int32_t vocab, uint64_t seed, uint64_t offset, int32_t* tokens, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes pa_sample needs for these sizes. */
size_t pa_sample_workspace_bytes(int32_t batch, int32_t vocab);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
