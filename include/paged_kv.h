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
 *  - Pointers are DEVICE pointers unless stated otherwise (the block manager
 *    functions, pkv_bm_*, take host pointers); arrays are row-major and
 *    contiguous in the shapes given.
 *  - The caller allocates and owns every buffer (cache, tables, slots, query,
 *    output, workspace).  The library allocates no device memory, keeps no
 *    pointer after returning, and has no global mutable state except a
 *    thread-local error message; the only host memory it holds is inside
 *    block managers the caller creates and destroys.
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
  PKV_ERR_HIP = -4,         /* the HIP runtime refused a launch               */
  PKV_ERR_NO_BLOCKS = -5    /* block manager: not enough free blocks; nothing
                               was changed                                    */
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
 * paged_kv_write_positions -- paged_kv_slot_mapping and paged_kv_write in one
 * launch: each token's slot is derived from its sequence's table and its
 * position (the same rule and the same -1 cases as paged_kv_slot_mapping:
 * itan.pw walk-through, "ブロックアロケーションの基本概念", slot_mapping) and
 * its key and value are stored there (studying-code.tistory.com vLLM review,
 * "디코딩 과정").  A token whose slot is -1 writes nothing.  slot_mapping, if
 * not NULL, receives the slots.  Bit-exact; distinct tokens must have
 * distinct slots.
 *
 *   key, value    dtype [num_tokens][num_kv_heads][head_size]
 *   kv_cache      dtype [2][num_blocks][block_size][num_kv_heads][head_size]   (in/out)
 *   block_tables  int32 [num_seqs][table_width]
 *   seq_ids       int32 [num_tokens] or NULL (token i belongs to sequence i)
 *   positions     int32 [num_tokens]
 *   slot_mapping  int64 [num_tokens] (output) or NULL
 */
int paged_kv_write_positions(const void* key, const void* value, void* kv_cache,
                             const int32_t* block_tables, int table_width, const int32_t* seq_ids,
                             const int32_t* positions, int64_t* slot_mapping, int num_tokens,
                             int num_seqs, int num_blocks, int block_size, int num_kv_heads,
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
 * Supported: head_size 64 or 128; block_size 8, 16, 32 or 64 (PKV_BF16) and any
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
 * paged_attention_decode_noalloc -- paged_attention_decode for callers that
 * cannot allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without the
 * workspace.  Its workspace is a device array the library holds on every GPU
 * it runs on, PKV_NOALLOC_SCRATCH_BYTES bytes, from module load until the
 * process ends; the call allocates nothing (no hipMalloc or hipFree, no host
 * heap).  A batch whose workspace (paged_attention_workspace_bytes) exceeds
 * that returns PKV_ERR_WORKSPACE before anything is enqueued.  Every call on
 * one GPU uses that GPU's one array, so calls whose executions overlap on a
 * GPU (several streams, several threads) race: serialise them.  Results are
 * those of paged_attention_decode with the same arguments, bit for bit.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32 << 20)
int paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype, const void* query,
                                   const void* kv_cache, const int32_t* block_tables,
                                   int table_width, const int32_t* context_lens, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_size,
                                   int block_size, int num_blocks, float scale,
                                   int max_context_len, int partition_size, pkv_dtype dtype,
                                   unsigned flags, hipStream_t stream);

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

/*
 * paged_attention_decode_append -- a whole decode step in one call: each
 * sequence's newly generated key and value are stored into its KV block
 * (studying-code.tistory.com vLLM review, section "디코딩 과정" (decoding)) and
 * its query attends over all its tokens, the new one included (section
 * "PagedAttention").  Sequence s with context_lens[s] >= 1 appends key[s] and
 * value[s] at position context_lens[s] - 1, in the slot
 *     table[s][(L - 1) / B] * B + (L - 1) % B            (L = context_lens[s])
 * (itan.pw walk-through, "ブロックアロケーションの基本概念", slot_mapping; the
 * same -1 cases as paged_kv_write_positions: nothing is written), then
 * everything is as paged_attention_decode.  Cache and output are
 * bit-identical to paged_kv_write_positions (positions L - 1) followed by
 * paged_attention_decode.  With fp32 caches, and under the stream schedule
 * when few of its pieces hold a sequence's last step, the write happens
 * inside the attention launch (the waves that read a sequence's last token
 * store the new row first, then read it back like the rest: one launch
 * less); otherwise the library launches the write first.  Sequences whose last token is
 * already cached (e.g. a fork still on its shared prompt) must use the
 * separate calls.
 *
 *   key, value    dtype [num_seqs][num_kv_heads][head_size], 16-byte aligned
 *   kv_cache      dtype [2][num_blocks][block_size][num_kv_heads][head_size]   (in/out)
 *   other arguments as paged_attention_decode (same workspace size)
 */
int paged_attention_decode_append(void* out, pkv_dtype out_dtype, const void* query,
                                  const void* key, const void* value, void* kv_cache,
                                  const int32_t* block_tables, int table_width,
                                  const int32_t* context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_size, int block_size, int num_blocks,
                                  float scale, int max_context_len, int partition_size,
                                  void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                                  unsigned flags, hipStream_t stream);

/*
 * Whether paged_attention_decode_append with these arguments stores the new
 * tokens inside its attention launch (1: always with fp32 caches) or
 * launches the write first (0); -1 for inconsistent head counts or when the
 * device cannot be queried.
 * Needs the device the call will run on to be current.  Host only.
 */
int paged_attention_append_in_launch(int num_seqs, int num_q_heads, int num_kv_heads,
                                     int head_size, int block_size, int max_context_len,
                                     int partition_size, pkv_dtype dtype);

/*
 * The attention pass of paged_attention_decode_append alone (with the write);
 * follow it with paged_attention_merge given the same decode arguments.
 */
int paged_attention_append_partitions(void* out, pkv_dtype out_dtype, const void* query,
                                      const void* key, const void* value, void* kv_cache,
                                      const int32_t* block_tables, int table_width,
                                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_size, int block_size,
                                      int num_blocks, float scale, int max_context_len,
                                      int partition_size, void* workspace, size_t workspace_bytes,
                                      pkv_dtype dtype, unsigned flags, hipStream_t stream);

/*
 * paged_attention_prefix_groups -- find groups of consecutive sequences that
 * share their first blocks.  HOST pointers; host only.
 *
 * The samples of one prompt (parallel sampling, beam candidates) store the
 * prompt's K/V once: their tables name the same physical blocks, each with a
 * reference count above one, until a write into a shared block copies it
 * (studying-code.tistory.com vLLM review: the two-sample example with both
 * sequences' logical blocks 0 and 1 on physical blocks 7 and 1, section
 * "생성 단계에서의 Copy-on-Write", and "vLLM과 Beam Search의 KV 블록 관리";
 * tech.blogsailing.com explainer, section 3).  Sequences are scanned in batch
 * order; a sequence joins the current group when its table starts with the
 * same entries as the group's first sequence for at least as many tokens as
 * the group shares so far (and at least min_prefix_len), else it starts a new
 * group.  A group's prefix is its shared tokens, cut to a multiple of
 * lcm(32, block_size) and to its shortest member's length; a group of one
 * sequence has prefix 0.
 *
 *   block_tables   int32 [num_seqs][table_width], host
 *   context_lens   int32 [num_seqs], host
 *   group_starts   int32 [num_seqs + 1] (output, host): group g is sequences
 *                  [group_starts[g], group_starts[g + 1])
 *   prefix_lens    int32 [num_seqs] (output, host): prefix tokens of group g
 *   num_groups, max_prefix_len  (outputs, host)
 */
int paged_attention_prefix_groups(const int32_t* block_tables, int table_width,
                                  const int32_t* context_lens, int num_seqs, int block_size,
                                  int min_prefix_len, int32_t* group_starts, int32_t* prefix_lens,
                                  int* num_groups, int* max_prefix_len);

/*
 * Partition size (tokens) paged_attention_decode_shared uses for these
 * arguments: partition_size itself if it is valid (a multiple of 32 and of
 * block_size), or, for 0, a size giving prefix work items for about half
 * the workgroups resident on the current device; -1 if invalid.  Host only.
 */
int paged_attention_shared_partition_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                          int head_size, int block_size, int num_groups,
                                          int max_prefix_len, int partition_size);

/*
 * Workspace bytes paged_attention_decode_shared needs for these arguments
 * (partition_size as given to it, 0 = automatic).  Host only.
 */
size_t paged_attention_shared_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                              int head_size, int block_size, int num_groups,
                                              int max_context_len, int max_prefix_len,
                                              int partition_size);

/*
 * paged_attention_decode_shared -- paged_attention_decode for a batch whose
 * sequences come in groups sharing their first blocks (the case of
 * paged_attention_prefix_groups).  Same result as paged_attention_decode
 * (the same attention per sequence, up to rounding), but each group's shared
 * prefix is read once for all its members' query heads instead of once per
 * member; each sequence's remaining tokens are read on their own, and the
 * parts are merged by the log-sum-exp rule.  Two launches (attention pass,
 * merge) on `stream`.  bf16 only.
 *
 *   group_starts  int32 [num_groups + 1], device: group g is sequences
 *                 [group_starts[g], group_starts[g + 1]); 0 = first <= ... <=
 *                 last = num_seqs, else every output row is NaN
 *   prefix_lens   int32 [num_groups], device: tokens 0 .. prefix_lens[g] - 1
 *                 of every member of group g are read through the table of
 *                 the group's first member.  A multiple of lcm(32, block_size),
 *                 <= max_prefix_len, <= every member's context length; else
 *                 the group's rows are NaN.  A member whose own table entries
 *                 for those tokens differ from the first member's gets NaN.
 *   num_groups    1 .. num_seqs (num_seqs <= 512)
 *   max_prefix_len   host int >= every prefix_lens[g] (sizes the workspace)
 *   partition_size   0 = automatic, else a multiple of 32 and of block_size
 *   workspace     device scratch of paged_attention_shared_workspace_bytes()
 *                 bytes, 256-byte aligned; every byte read is written first
 *                 in the same call
 * Other arguments, layouts and limits as paged_attention_decode.
 */
int paged_attention_decode_shared(void* out, pkv_dtype out_dtype, const void* query,
                                  const void* kv_cache, const int32_t* block_tables,
                                  int table_width, const int32_t* context_lens,
                                  const int32_t* group_starts, const int32_t* prefix_lens,
                                  int num_groups, int num_seqs, int num_q_heads, int num_kv_heads,
                                  int head_size, int block_size, int num_blocks, float scale,
                                  int max_context_len, int max_prefix_len, int partition_size,
                                  void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                                  unsigned flags, hipStream_t stream);

/*
 * The two launches paged_attention_decode_shared makes, for timing or
 * scheduling them separately: the attention pass (partial results of every
 * prefix and suffix partition into the workspace) and the log-sum-exp merge
 * into out[].  Both take exactly paged_attention_decode_shared's arguments
 * and must be given the same ones, in this order, on the same stream.
 */
int paged_attention_shared_partitions(void* out, pkv_dtype out_dtype, const void* query,
                                      const void* kv_cache, const int32_t* block_tables,
                                      int table_width, const int32_t* context_lens,
                                      const int32_t* group_starts, const int32_t* prefix_lens,
                                      int num_groups, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_size, int block_size,
                                      int num_blocks, float scale, int max_context_len,
                                      int max_prefix_len, int partition_size, void* workspace,
                                      size_t workspace_bytes, pkv_dtype dtype, unsigned flags,
                                      hipStream_t stream);

int paged_attention_shared_merge(void* out, pkv_dtype out_dtype, const void* query,
                                 const void* kv_cache, const int32_t* block_tables,
                                 int table_width, const int32_t* context_lens,
                                 const int32_t* group_starts, const int32_t* prefix_lens,
                                 int num_groups, int num_seqs, int num_q_heads, int num_kv_heads,
                                 int head_size, int block_size, int num_blocks, float scale,
                                 int max_context_len, int max_prefix_len, int partition_size,
                                 void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                                 unsigned flags, hipStream_t stream);

/*
 * Shared-prefix decode with a plan made once per decode step.  Every layer
 * of a model reads its own cache through the same block tables (itan.pw
 * walk-through, "ブロック割当のロジック": in the decode phase each layer's
 * cache tensor is indexed by the one table), so the work list of
 * paged_attention_decode_shared -- which depends only on the tables,
 * context lengths and groups -- can be made once and read by every layer's
 * launches, which then start reading K/V one load after they begin instead
 * of first deriving the list.  Results are bit-identical to
 * paged_attention_decode_shared with the same arguments.
 *
 * Bytes of the plan for these arguments (0 if they are invalid); host only.
 */
size_t paged_attention_shared_plan_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int block_size, int num_groups, int max_context_len,
                                         int max_prefix_len, int partition_size);

/*
 * paged_attention_shared_plan -- make the plan: one launch on `stream`.
 *
 *   plan          device buffer of paged_attention_shared_plan_bytes() bytes,
 *                 256-byte aligned, owned by the caller; overwritten
 *   block_tables, table_width, context_lens, group_starts, prefix_lens,
 *   num_groups, num_seqs, num_q_heads, num_kv_heads, block_size,
 *   max_context_len, max_prefix_len, partition_size
 *                 as for paged_attention_decode_shared (device arrays)
 *
 * The plan holds the arguments it was made for, each sequence's part count,
 * group leader, prefix length and prefix-table check, and each work item's
 * description and first block-table window.  It describes the tables,
 * lengths and groups as they are when its launch runs: after any of them
 * changes, make a new plan.  Errors as paged_attention_decode_shared
 * (PKV_ERR_WORKSPACE for a plan buffer that is too small).
 */
int paged_attention_shared_plan(void* plan, size_t plan_bytes, const int32_t* block_tables,
                                int table_width, const int32_t* context_lens,
                                const int32_t* group_starts, const int32_t* prefix_lens,
                                int num_groups, int num_seqs, int num_q_heads, int num_kv_heads,
                                int block_size, int max_context_len, int max_prefix_len,
                                int partition_size, hipStream_t stream);

/*
 * paged_attention_decode_shared_planned -- paged_attention_decode_shared
 * (same arguments, same two launches, same output) reading its work list from
 * `plan` (made by paged_attention_shared_plan, read only) instead of
 * deriving it.  The kernels check that the plan was made for this call's
 * num_seqs, num_q_heads, num_kv_heads, block_size, table_width,
 * max_context_len, max_prefix_len, num_groups and (resolved) partition size,
 * and that it recorded every item; if not, every output row is NaN.  The
 * plan may be read by any number of calls (e.g. one per layer) until the
 * tables, lengths or groups change.  plan_bytes: its size, at least
 * paged_attention_shared_plan_bytes() for these arguments.
 */
int paged_attention_decode_shared_planned(void* out, pkv_dtype out_dtype, const void* query,
                                          const void* kv_cache, const int32_t* block_tables,
                                          int table_width, const int32_t* context_lens,
                                          const int32_t* group_starts,
                                          const int32_t* prefix_lens, int num_groups,
                                          int num_seqs, int num_q_heads, int num_kv_heads,
                                          int head_size, int block_size, int num_blocks,
                                          float scale, int max_context_len, int max_prefix_len,
                                          int partition_size, void* workspace,
                                          size_t workspace_bytes, pkv_dtype dtype, unsigned flags,
                                          const void* plan, size_t plan_bytes,
                                          hipStream_t stream);

/*
 * Its two launches separately (attention pass, merge), as
 * paged_attention_shared_partitions and paged_attention_shared_merge.
 */
int paged_attention_shared_planned_partitions(
    void* out, pkv_dtype out_dtype, const void* query, const void* kv_cache,
    const int32_t* block_tables, int table_width, const int32_t* context_lens,
    const int32_t* group_starts, const int32_t* prefix_lens, int num_groups, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_size, int block_size, int num_blocks, float scale,
    int max_context_len, int max_prefix_len, int partition_size, void* workspace,
    size_t workspace_bytes, pkv_dtype dtype, unsigned flags, const void* plan, size_t plan_bytes,
    hipStream_t stream);

int paged_attention_shared_planned_merge(
    void* out, pkv_dtype out_dtype, const void* query, const void* kv_cache,
    const int32_t* block_tables, int table_width, const int32_t* context_lens,
    const int32_t* group_starts, const int32_t* prefix_lens, int num_groups, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_size, int block_size, int num_blocks, float scale,
    int max_context_len, int max_prefix_len, int partition_size, void* workspace,
    size_t workspace_bytes, pkv_dtype dtype, unsigned flags, const void* plan, size_t plan_bytes,
    hipStream_t stream);

/*
 * paged_attention_prefill -- causal attention of chunks of query tokens over
 * their paged sequences: the prompt step (prefill) and chunked prefill.
 *
 * A prompt is processed with ordinary self-attention, every token attending
 * to itself and the tokens before it (studying-code.tistory.com vLLM review,
 * "프리필(Prefill) 단계"); the input tokens of all requests of an iteration
 * are joined into one sequence, and the kernel reads earlier K/V through the
 * block tables (the same review, "디코딩 과정"); each joined request keeps
 * its own positions from 0 and attends only to itself (itan.pw walk-through,
 * "ブロックアロケーションの基本概念").  Sequence s's chunk is query rows
 * [query_start[s], query_start[s+1]); its K/V must already be in the cache
 * (written with paged_kv_write), so the chunk is the last chunk_len tokens of
 * the sequence: row i sits at position context_lens[s] - chunk_len + i and
 * attends keys 0 .. that position.  A whole prompt is the chunk with
 * chunk_len == context_len; a chunk continuing cached tokens (an earlier
 * chunk, or prefix-cache hits) has chunk_len < context_len; decode is
 * chunk_len == 1.
 *
 *   out          out_dtype [num_tokens][num_q_heads][head_size]; rows outside
 *                every chunk are not written
 *   query        dtype [num_tokens][num_q_heads][head_size]
 *   query_start  int32 [num_seqs + 1], device, non-decreasing, last <= num_tokens
 *   max_query_len  host int >= every chunk length (sizes the grid); a longer
 *                chunk, a chunk longer than its sequence, or a sequence longer
 *                than table_width * block_size gives NaN rows; an
 *                out-of-range table entry gives NaN for the rows reading it
 *   kv_cache, block_tables, table_width, context_lens, num_blocks: as for
 *                paged_attention_decode
 * Supported: head_size 64 or 128; bf16: block_size 8, 16, 32 or 64 (matrix
 * cores; scores and the weighted sum accumulate in fp32), at most 5453
 * (head_size 64) or 10914 (head_size 128) sequences per call, else
 * PKV_ERR_UNSUPPORTED; fp32: any block_size (vector ALU).  Needs no workspace
 * and no clearing.
 */
int paged_attention_prefill(void* out, pkv_dtype out_dtype, const void* query,
                            const int32_t* query_start, int num_tokens, int max_query_len,
                            const void* kv_cache, const int32_t* block_tables, int table_width,
                            const int32_t* context_lens, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_size, int block_size, int num_blocks,
                            float scale, pkv_dtype dtype, hipStream_t stream);

/*
 * paged_kv_copy_blocks -- copy whole blocks (keys and values) between two
 * pools of the same geometry: dst_cache[:, dst_blocks[i]] =
 * src_cache[:, src_blocks[i]] for every i.
 *
 * Serves copy-on-write (dst_cache == src_cache: a forked sample about to
 * write into a shared block first copies it to its own; studying-code.tistory.com
 * vLLM review, "생성 단계에서의 Copy-on-Write", and "메모리 복사 오버헤드의
 * 최적화": only that one block is copied) and swapping (one pool in device
 * memory, the other in pinned host memory from hipHostMalloc, which the
 * kernel reads or writes over PCIe).  Bit-exact copy.  Each pointer is
 * checked with hipPointerGetAttributes: pinned host memory is used through
 * its mapped device address, and pageable host memory gives PKV_ERR_INVALID
 * before anything is launched.
 *
 *   dst_cache    dtype [2][dst_num_blocks][block_size][num_kv_heads][head_size]
 *   src_cache    dtype [2][src_num_blocks][block_size][num_kv_heads][head_size]
 *   src_blocks, dst_blocks  int32 [num_copies], device or pinned host memory;
 *                a pair with an id out of its pool's range is skipped
 * The copies are independent: no destination may also be a source, and no
 * block may be a destination twice (the block manager's copy lists obey this).
 * Supported: head_size * element bytes a multiple of 16; pools 16-byte aligned.
 */
int paged_kv_copy_blocks(void* dst_cache, int dst_num_blocks, const void* src_cache,
                         int src_num_blocks, const int32_t* src_blocks, const int32_t* dst_blocks,
                         int num_copies, int block_size, int num_kv_heads, int head_size,
                         pkv_dtype dtype, hipStream_t stream);

/*
 * Block manager (host).  Hands out the block tables and slots the kernels
 * above consume, for one pool of num_blocks physical blocks of block_size
 * tokens (every layer's cache uses the same table):
 *
 *  - each physical block has a reference count, one per logical block that
 *    maps to it (studying-code.tistory.com vLLM review, "요청 완료 후 메모리
 *    관리": two samples share blocks 7 and 1, counts 2);
 *  - free blocks wait in a queue: allocation takes its head, a freed sequence
 *    returns the blocks whose count reaches zero to its tail, last block first
 *    (itan.pw walk-through, "プレイフィックスキャッシュの詳細", times 4-6);
 *  - a prompt of n tokens takes ceil(n / block_size) blocks; decoding fills
 *    the last block and takes a new one when it is full (the walk-through,
 *    overall allocation flow and "ブロック割当のロジック");
 *  - fork shares every block of the parent (counts + 1); writing a token
 *    into a block whose count is above 1 first moves the writer to a fresh
 *    block and reports the copy the caller must make with
 *    paged_kv_copy_blocks before the write (the review, "생성 단계에서의
 *    Copy-on-Write"; tech.blogsailing.com explainer, section 3);
 *  - with prefix caching, every full block is registered under the chain hash
 *    SHA-256(previous block's hash, or 32 zero bytes, || its token ids as
 *    little-endian int32); a new request reuses the cached blocks of its
 *    leading full blocks, at most (n - 1) / block_size of them, up to the
 *    first miss; a cached block taken from the free queue for other data
 *    loses its entry (the walk-through, "プレイフィックスキャッシュの詳細");
 *  - a group of sequences (every sequence sharing a block with another must
 *    be in it) is swapped out to, and back in from, a pool of num_cpu_blocks
 *    host blocks, all or nothing; the caller makes the reported copies
 *    (studying-code.tistory.com vLLM review, "All-or-Nothing Eviction" and
 *    "스와핑(Swapping)").
 *
 * A request the pool cannot satisfy returns PKV_ERR_NO_BLOCKS and changes
 * nothing.  Sequences are named by caller-chosen int64 ids.  A manager is not
 * thread-safe.  All pointers here are host pointers.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* NULL on bad sizes.  prefix_caching: 0 or 1. */
pkv_block_manager* pkv_bm_create(int num_blocks, int block_size, int prefix_caching,
                                 int num_cpu_blocks);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Replace the initial free-queue order (a permutation of all blocks) of a
 * manager that has no sequence yet. */
int pkv_bm_set_free_order(pkv_block_manager* bm, const int32_t* order, int n);

/* Admit sequence `seq` with its prompt tokens[num_tokens]; *num_cached_tokens
 * receives how many leading tokens came from the prefix cache (their K/V are
 * already in the pool; the caller writes positions from there on). */
int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int num_tokens,
                    int* num_cached_tokens);

/* Append n generated tokens to `seq`.  slots[n] receives each token's slot
 * (for paged_kv_slot_mapping's consumers: paged_kv_write); copy_src[n] and
 * copy_dst[n] receive *num_copies copy-on-write block copies to make first. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int n,
                  int64_t* slots, int32_t* copy_src, int32_t* copy_dst, int* num_copies);

/* `child` shares every block of `parent`. */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Release a sequence (swapped out or not). */
int pkv_bm_free(pkv_block_manager* bm, int64_t seq);

/* Swap the group seqs[num_seqs] out to host blocks (gpu_blocks[i] ->
 * cpu_blocks[i], *num_copies pairs, at most `capacity`), or back in
 * (cpu_blocks[i] -> gpu_blocks[i]). */
int pkv_bm_swap_out(pkv_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* gpu_blocks,
                    int32_t* cpu_blocks, int capacity, int* num_copies);
int pkv_bm_swap_in(pkv_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* cpu_blocks,
                   int32_t* gpu_blocks, int capacity, int* num_copies);

/* Views.  Counts are returned (>= 0) or a negative status. */
int pkv_bm_num_tokens(pkv_block_manager* bm, int64_t seq);
int pkv_bm_is_swapped(pkv_block_manager* bm, int64_t seq);
/* the sequence's block ids (CPU block ids while swapped out); returns the
 * count and fills at most `capacity` entries */
int pkv_bm_block_table(pkv_block_manager* bm, int64_t seq, int32_t* out, int capacity);
/* slots of positions [begin, end) of a resident sequence */
int pkv_bm_slots(pkv_block_manager* bm, int64_t seq, int begin, int end, int64_t* out);
/* block tables [num_seqs][table_width] (INT32_MIN past each sequence's last
 * block) and context lengths [num_seqs] of resident sequences, for the
 * attention entry points (copy them to the device) */
int pkv_bm_batch_tables(pkv_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* tables,
                        int table_width, int32_t* context_lens);
int pkv_bm_ref_count(pkv_block_manager* bm, int block);
int pkv_bm_num_free(pkv_block_manager* bm);
/* the free queue, head first; returns its length, fills at most `capacity` */
int pkv_bm_free_queue(pkv_block_manager* bm, int32_t* out, int capacity);
/* 1 and the block's 32-byte chain hash in out, or 0 when it has none */
int pkv_bm_block_hash(pkv_block_manager* bm, int block, uint8_t* out);
/* 1 when the prefix cache maps the block's hash to this block */
int pkv_bm_is_cached(pkv_block_manager* bm, int block);

/*
 * pkv_read_ceiling -- a measurement utility, not part of the decode path:
 * read `bytes` (a multiple of 16) of device memory at `buf` (16-byte
 * aligned) once, with `grid` workgroups of 256 threads each keeping
 * `loads_in_flight` (1, 2, 4 or 8) nontemporal 16-byte loads in flight, and
 * write one word per workgroup to sink[0 .. grid) (device).  Timed by the
 * caller, it gives the streaming-read rate the decode kernels' HBM rates are
 * compared with at the same bytes per launch.  Errors: PKV_ERR_INVALID (null
 * pointers, alignment, grid outside [1, 2^20]), PKV_ERR_UNSUPPORTED.
 */
int pkv_read_ceiling(const void* buf, size_t bytes, int grid, int loads_in_flight, unsigned* sink,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
