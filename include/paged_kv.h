/*
 * paged_kv.h -- C ABI of the paged KV-cache decode path for AMD Instinct
 * MI355X (gfx950).
 *
 * One attention layer keeps its KV cache in a single device array
 *
 *     kv_cache[2][num_blocks][block_size][num_kv_heads][head_size]
 *
 * (index 0 of the first axis holds keys, index 1 values; the block id is the
 * paging index) -- the per-layer tensor shape described in the itan.pw
 * walk-through of vLLM's KVCacheManager, sections "BlockPoolの生成過程" and
 * "ブロックアロケーションの基本概念".  A sequence's tokens fill its logical blocks
 * left to right; token t sits at offset t % block_size of logical block
 * t / block_size, and the sequence's block table names the physical block of
 * each logical block (tech.blogsailing.com PagedAttention explainer, section 2;
 * studying-code.tistory.com vLLM review, memory-management sections).  A slot is
 * physical_block * block_size + offset.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated otherwise; arrays are
 *    row-major and contiguous in the shapes given.
 *  - The caller allocates and owns every buffer (cache, tables, slots, query,
 *    output, workspace).  The library allocates nothing, keeps no pointer
 *    after returning, and has no global mutable state except a thread-local
 *    error message.
 *  - All work is enqueued asynchronously on `stream` (0 = the null stream);
 *    the library never synchronises.  Argument errors are found on the host
 *    before anything is enqueued; the return value is a pkv_status and, when
 *    it is not PKV_OK, pkv_last_error() describes it.
 *  - Device-side contents (table entries, slots, context lengths) are not
 *    visible to the host check.  The kernels bound-check them and never read
 *    or write outside the arrays: an entry outside its range is skipped (write,
 *    slot mapping) or turns that sequence's output rows into NaN (attention).
 *  - Element types: PKV_F32 (IEEE binary32) or PKV_BF16 (bfloat16).  Cache,
 *    keys, values and queries share one element type.
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Flags of the attention entry points. */
enum {
  /* Blocks may be referenced by several sequences of the batch (shared
   * prefixes, parallel sampling, beam search): read K/V through the caches so
   * that sequences sharing a block can hit on it.  Without this flag K/V are
   * streamed with nontemporal loads, the faster way to read data used once. */
  PKV_ATTN_CACHED_KV = 1u
};

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* bad argument (null pointer, size, alignment)   */
  PKV_ERR_UNSUPPORTED = -2, /* valid but not built (head size, block size...) */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or too small                 */
  PKV_ERR_HIP = -4          /* the HIP runtime refused a launch               */
} pkv_status;

/* Message describing the last failed call on this thread ("" if none).  The
 * string is owned by the library and valid until the next call on the thread. */
const char* pkv_last_error(void);

/*
 * paged_kv_slot_mapping -- the slot each (sequence, position) pair occupies.
 *
 * The decode step records, for every newly generated token, which slot of the
 * physical cache it goes to (itan.pw walk-through, section
 * "ブロックアロケーションの基本概念", its last paragraph: slot_mapping).  For
 * i < num_tokens:
 *     s = seq_ids ? seq_ids[i] : i,   p = positions[i]
 *     slot_mapping[i] = block_tables[s][p / block_size] * block_size + p % block_size
 * and -1 when p < 0 (the sequence appends nothing).  It is also -1 when s is
 * outside [0, num_seqs), p / block_size >= table_width, or the table entry is
 * outside [0, num_blocks) -- such a token is then not written.
 *
 *   slot_mapping  int64 [num_tokens]                     (output)
 *   block_tables  int32 [num_seqs][table_width]
 *   seq_ids       int32 [num_tokens] or NULL (token i belongs to sequence i)
 *   positions     int32 [num_tokens]
 */
int paged_kv_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables, int table_width,
                          const int32_t* seq_ids, const int32_t* positions, int num_tokens,
                          int num_seqs, int block_size, int num_blocks, hipStream_t stream);

/*
 * paged_kv_write -- store each new token's key and value at its slot
 * (reshape-and-cache).
 *
 * Newly generated KV is stored into physical KV blocks during the forward pass
 * (studying-code.tistory.com vLLM review, section "디코딩 과정" (decoding); the
 * worked example's first decoding step writes into the free slot of block 1).
 * For t < num_tokens with 0 <= slot_mapping[t] < num_blocks * block_size:
 *     kv_cache[0][slot / B][slot % B][h][:] = key[t][h][:]
 *     kv_cache[1][slot / B][slot % B][h][:] = value[t][h][:]     for every h
 * A negative or out-of-range slot writes nothing.  The copy is bit-exact.
 * Distinct tokens must have distinct slots (else the result is unspecified).
 *
 *   key, value    dtype [num_tokens][num_kv_heads][head_size]
 *   kv_cache      dtype [2][num_blocks][block_size][num_kv_heads][head_size]   (in/out)
 *   slot_mapping  int64 [num_tokens]
 * head_size * element bytes must be a multiple of 16; pointers 16-byte aligned.
 */
int paged_kv_write(const void* key, const void* value, void* kv_cache, const int64_t* slot_mapping,
                   int num_tokens, int num_blocks, int block_size, int num_kv_heads,
                   int head_size, pkv_dtype dtype, hipStream_t stream);

/*
 * paged_kv_gather -- read every sequence's keys and values, in logical order,
 * through its block table into contiguous arrays (a checking path).
 *
 * The cache is accessed as kv_cache[:, table, ...] (itan.pw walk-through,
 * section "ブロック割当のロジック", the per-layer access with the table
 * [10, 21, 45, 67]).  For t < context_lens[s]:
 *     k_out[s][t] = kv_cache[0][table[s][t / B]][t % B],  v_out likewise;
 * rows t >= context_lens[s] are zero.  A sequence whose length exceeds
 * max_context_len or table_width * block_size, or whose table entry is out of
 * range, gets NaN rows instead.  Bit-exact copy.
 *
 *   k_out, v_out  dtype [num_seqs][max_context_len][num_kv_heads][head_size]  (output)
 */
int paged_kv_gather(void* k_out, void* v_out, const void* kv_cache, const int32_t* block_tables,
                    int table_width, const int32_t* context_lens, int num_seqs, int num_kv_heads,
                    int head_size, int block_size, int num_blocks, int max_context_len,
                    pkv_dtype dtype, hipStream_t stream);

/*
 * Partition size the decode kernel will use for these arguments.  A request
 * of 0 selects the split automatically.  bf16: whole sequences when the batch
 * has enough (sequence, kv-head group) work items to fill the GPU; otherwise
 * 0, the stream schedule: each wave of a persistent grid reads an equal share
 * of the batch's K/V, cutting contexts wherever the shares end.  fp32: 64
 * tokens.  A positive request is returned if it is a multiple of 32 and of
 * block_size (fp32: at most 512), else -1.  Host only.
 */
int paged_attention_partition_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                                   int block_size, int max_context_len, int partition_size,
                                   pkv_dtype dtype);

/*
 * Workspace bytes paged_attention_decode needs for these arguments (0 when
 * every sequence fits in one partition).  The stream schedule always needs
 * one, sized for the current device's compute units: query it on the device
 * the call will run on.  Host only.
 */
size_t paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_size, int block_size, int max_context_len,
                                       int partition_size, pkv_dtype dtype);

/*
 * paged_attention_decode -- one decoding token per sequence attends to its
 * sequence's cached keys and values, read block by block through the block
 * table (PagedAttention).
 *
 * Each query is multiplied with the keys of every block the table names, the
 * scores weight the values, and the per-block results are combined into the
 * output (studying-code.tistory.com vLLM review, section "PagedAttention";
 * garden.houmin.site notes, section "KV Cache 管理器", the algorithm figure).
 * Paging changes only where K/V live, so for each sequence s and query head h
 *     g      = h / (num_q_heads / num_kv_heads)         (contiguous head groups)
 *     z_t    = scale * dot(query[s][h], K_s[t][g]),      t < context_lens[s]
 *     out[s][h] = sum_t softmax(z)_t * V_s[t][g]
 * where K_s[t] = kv_cache[0][table[s][t / B]][t % B] and V_s likewise.
 * context_lens[s] counts every token attended, including the one written this
 * step; a sequence of length 0 gets zeros.  Long contexts are split into
 * partitions -- of `partition_size` tokens, or, under the stream schedule,
 * wherever one wave's share of the batch ends -- whose softmax statistics are
 * merged by the log-sum-exp rule; the result does not depend on the split
 * beyond rounding, and repeated calls on the same GPU model give identical
 * bits.  Accumulation is fp32.
 *
 *   out           out_dtype [num_seqs][num_q_heads][head_size]      (output)
 *   query         dtype [num_seqs][num_q_heads][head_size]
 *   kv_cache      dtype [2][num_blocks][block_size][num_kv_heads][head_size]
 *   block_tables  int32 [num_seqs][table_width]; entries past a sequence's
 *                 last block are never read
 *   context_lens  int32 [num_seqs], 0 <= L <= min(max_context_len, table_width*B)
 *   max_context_len  host int, an upper bound of context_lens (sizes the grid
 *                 of fixed partitions)
 *   partition_size   0 = chosen by the library (see
 *                 paged_attention_partition_size), else a multiple of 32 and of B
 *   flags         0 or PKV_ATTN_CACHED_KV
 *   workspace     device scratch of at least paged_attention_workspace_bytes()
 *                 bytes (may be NULL when that is 0), 256-byte aligned
 * Supported: head_size 64 or 128; block_size 16, 32 or 64 (PKV_BF16) and any
 * block_size from 1 to 256 (PKV_F32); num_q_heads a multiple of num_kv_heads.
 */
int paged_attention_decode(void* out, pkv_dtype out_dtype, const void* query,
                           const void* kv_cache, const int32_t* block_tables, int table_width,
                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_size, int block_size, int num_blocks,
                           float scale, int max_context_len, int partition_size, void* workspace,
                           size_t workspace_bytes, pkv_dtype dtype, unsigned flags,
                           hipStream_t stream);

/*
 * The two launches paged_attention_decode makes, exposed so that a caller can
 * time or schedule them separately.  paged_attention_partitions runs the
 * attention pass: it writes out[] directly for every sequence that fits in one
 * partition and the per-partition statistics (max score, exponent sum,
 * normalised partial output) into the workspace for the others.
 * paged_attention_merge then combines those statistics by the log-sum-exp
 * rule into out[]; it does nothing when every sequence fits in one partition.
 * Both take exactly paged_attention_decode's arguments and must be given the
 * same ones, in this order, on the same stream.
 */
int paged_attention_partitions(void* out, pkv_dtype out_dtype, const void* query,
                               const void* kv_cache, const int32_t* block_tables, int table_width,
                               const int32_t* context_lens, int num_seqs, int num_q_heads,
                               int num_kv_heads, int head_size, int block_size, int num_blocks,
                               float scale, int max_context_len, int partition_size,
                               void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                               unsigned flags, hipStream_t stream);

int paged_attention_merge(void* out, pkv_dtype out_dtype, const void* query,
                          const void* kv_cache, const int32_t* block_tables, int table_width,
                          const int32_t* context_lens, int num_seqs, int num_q_heads,
                          int num_kv_heads, int head_size, int block_size, int num_blocks,
                          float scale, int max_context_len, int partition_size, void* workspace,
                          size_t workspace_bytes, pkv_dtype dtype, unsigned flags,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
