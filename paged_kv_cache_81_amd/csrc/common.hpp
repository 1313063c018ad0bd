// Internal helpers shared by the HIP sources of the paged KV library (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "paged_kv.h"

namespace pkv {

// ---------------------------------------------------------------- host side

// Records the message returned by pkv_last_error() for this thread.
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

// Turns the last launch error into PKV_ERR_HIP (or PKV_OK).
int check_launch(const char* what);

// Lets kernel kern use `bytes` of dynamic LDS (default bf16_lds_limit()) on
// the current device (once per kernel and device; thread-safe).
int raise_lds_limit(const void* kern, int bytes = 0);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- device side

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Kernel launchers (one per source file), called from api.hip after the
// arguments have been checked.
int launch_slot_mapping(int64_t* slot_mapping, const int32_t* tables, int width,
                        const int32_t* seq_ids, const int32_t* positions, int T, int S, int B,
                        int NB, hipStream_t stream);
int launch_write(const void* key, const void* value, void* kv, const int64_t* slots, int T, int NB,
                 int B, int Hkv, int D, int elem_bytes, hipStream_t stream);
int launch_write_positions(const void* key, const void* value, void* kv, const int32_t* tables,
                           int width, const int32_t* seq_ids, const int32_t* positions,
                           int pos_offset, int64_t* slots_out, int T, int S, int NB, int B,
                           int Hkv, int D, int elem_bytes, hipStream_t stream);
int launch_copy_blocks(void* dst, int dst_nb, const void* src, int src_nb, const int32_t* src_ids,
                       const int32_t* dst_ids, int n, int64_t half_bytes, hipStream_t stream);
int launch_gather(void* k_out, void* v_out, const void* kv, const int32_t* tables, int width,
                  const int32_t* lens, int S, int Hkv, int D, int B, int NB, int max_len,
                  int elem_bytes, hipStream_t stream);

struct AttnArgs {
  void* out;          // [S][Hq][D] fp32 or bf16
  float* ws_o;        // [S][max_parts][Hq][D]   (split path only)
  float* ws_ml;       // [S][max_parts][Hq][2]   (m in log2 units, l)
  const void* query;  // [S][Hq][D]
  const void* kv;     // [2][NB][B][Hkv][D]
  const int32_t* tables;
  const int32_t* lens;
  int width, S, Hq, Hkv, D, B, NB;
  int partition;      // tokens per partition
  int max_parts;      // partitions the grid covers per sequence
  float scale_log2;   // scale * log2(e)
  int out_bf16;
  int nontemporal;    // stream K/V past the caches
  int parts_per_wg;   // partitions one workgroup covers (bf16 path)
  int longest_first;  // map workgroups to sequences in decreasing length
  int k_via_lds;      // load keys row-wise and rearrange them through LDS
  int compact;        // bf16: workgroups walk a compact list of work items
  int xcd_blocked;    // bf16 dense grid: each XCD takes a contiguous eighth of the items
  // stream schedule (bf16, automatic partitioning)
  int stream;              // use it
  int stream_waves;        // waves of the persistent grid (a multiple of 4)
  int stream_slots;        // finished results a wave keeps in LDS before storing
  int stream_wave_floats;  // LDS floats of one wave
  int* ws_pref;            // [S + 1] first stream step of each sequence
  int max_len;             // longest valid context (longer ones give NaN)
  // shared-prefix schedule (sequences in groups that read their first
  // prefix_lens[g] tokens through identical table entries)
  const int32_t* group_starts;  // [num_groups + 1]
  const int32_t* prefix_lens;   // [num_groups]
  int num_groups;
  int max_prefix;               // longest valid prefix (longer ones give NaN)
  int* ws_seq;                  // [4][S]: parts of each sequence (or -1), its group's
                                // first sequence, its prefix length, table mismatch
  // decode step with its write (stream schedule): sequence s's new token,
  // rows [s][Hkv][D] of k_new and v_new, sits at position lens[s] - 1; it is
  // written to the cache and folded in from these rows (nullptr: none)
  const void* k_new;
  const void* v_new;
  // shared-prefix schedule with a plan made beforehand (nullptr: every
  // workgroup of the attention launch makes its own), and the item records
  // its buffer holds room for
  const int32_t* plan;
  int64_t plan_capacity;
};

// Stream schedule: wave w of W reads stream steps [start(w), start(w + 1))
// of the T in the batch.  With T >= W every piece has floor(T/W) or one more
// steps; with fewer steps than waves, wave w < T gets step w alone and the
// rest none -- never an empty piece between two others.
__host__ __device__ inline int stream_piece_start(int64_t w, int64_t T, int64_t W) {
  return static_cast<int>(T >= W ? w * T / W : (w < T ? w : T));
}
// The wave whose piece holds step x (0 <= x < T).
__host__ __device__ inline int64_t stream_wave_of(int64_t x, int64_t T, int64_t W) {
  return T >= W ? ((x + 1) * W - 1) / T : x;
}

// largest batch whose bf16 workgroups rank the sequences by length
constexpr int kMaxRankedSeqs = 128;
// largest batch whose bf16 workgroups can number the work items themselves
constexpr int kMaxCompactSeqs = 512;
// most groups (and sequences, kMaxCompactSeqs) the shared-prefix schedule takes
constexpr int kMaxSharedGroups = 512;
// largest batch the stream schedule takes (its workgroups scan the lengths);
// it serves batches of fewer than 512 (sequence, kv-head group) units
constexpr int kMaxStreamSeqs = 512;

// kv heads per bf16 workgroup: 4 when they divide Hkv, else 2, else 1
__host__ __device__ inline int bf16_heads_per_group(int Hkv) { return Hkv % 4 == 0 ? 4 : (Hkv % 2 == 0 ? 2 : 1); }

// LDS of one bf16 workgroup: for each of its 4 waves, a 32-token K tile
// (32 x D bf16), then pps partition slots of min(16, G) head rows (D + 4
// floats), then an (m, l) pair per row, padded to a multiple of 4 floats so
// every wave's area stays 16-byte aligned.
__host__ __device__ inline int bf16_lds_k_floats(int D) { return 16 * D; }
__host__ __device__ inline int bf16_lds_wave_floats(int pps, int G, int D, bool k_tile) {
  const int nhs = G < 16 ? G : 16;
  return (k_tile ? bf16_lds_k_floats(D) : 0) + pps * nhs * (D + 4) + (pps * nhs * 2 + 3) / 4 * 4;
}
inline size_t bf16_lds_bytes(int pps, int G, int D, bool k_tile) {
  return static_cast<size_t>(4) * bf16_lds_wave_floats(pps, G, D, k_tile) * sizeof(float);
}
// at most this much (plus ~2 KB of static LDS), so that two workgroups fit
// in a CU's 160 KB
inline size_t bf16_lds_limit() { return 77 * 1024; }

// Stream schedule: workgroups per CU of the persistent grid (what the
// kernel's registers allow: 3 for head size 64, 2 for 128).
inline int stream_wgs_per_cu(int D) { return D == 64 ? 3 : 2; }
// Ints describing where a stream result slot goes.
constexpr int kStreamMeta = 3;
// LDS floats per result slot: nhs rows of D + 4, their (m, l), and the
// slot's description.
inline int stream_slot_floats(int G, int D) {
  const int nhs = G < 16 ? G : 16;
  return nhs * (D + 4) + 2 * nhs + kStreamMeta;
}
// Result slots per wave and LDS floats per wave: what is left of the CU's
// 160 KB, shared by the resident workgroups, after the static scan array and
// the K tile; at most 16 slots.
inline void stream_lds_plan(int G, int D, bool k_tile, int* slots, int* wave_floats) {
  const size_t static_bytes = (kMaxStreamSeqs + 1 + 4) * sizeof(int) + 256;
  size_t per_wg = 160 * 1024 / stream_wgs_per_cu(D) - static_bytes;
  if (per_wg > bf16_lds_limit()) per_wg = bf16_lds_limit();
  const int per_wave = static_cast<int>(per_wg / 4 / sizeof(float));
  const int tile = k_tile ? 16 * D : 0;
  int k = (per_wave - tile) / stream_slot_floats(G, D);
  k = k < 1 ? 1 : (k > 16 ? 16 : k);
  *slots = k;
  *wave_floats = (tile + k * stream_slot_floats(G, D) + 3) / 4 * 4;
}

// Shared-prefix schedule: static LDS of a workgroup's plan (group starts,
// item scans, prefix lengths, sequence lengths), ints describing where a
// finished result goes, and the LDS floats of one result (16 rows of D + 4,
// their (m, l), its description).  Two workgroups per CU (registers).
constexpr int kSharedPlanInts = 2 * (kMaxSharedGroups + 1) + 3 * kMaxCompactSeqs + 5 +
                                (kMaxSharedGroups + 1 + kMaxCompactSeqs + 1) / 2;
constexpr int kSharedMeta = 8;
constexpr int kSharedWgsPerCu = 2;
inline int shared_slot_floats(int D) { return 16 * (D + 4) + 2 * 16 + kSharedMeta; }
// Finished results each wave keeps in LDS (1 .. 4) and LDS floats per wave.
inline void shared_lds_plan(int D, bool k_tile, int* slots, int* wave_floats) {
  size_t per_wg = 160 * 1024 / kSharedWgsPerCu - kSharedPlanInts * sizeof(int) - 256;
  if (per_wg > bf16_lds_limit()) per_wg = bf16_lds_limit();
  const int per_wave = static_cast<int>(per_wg / 4 / sizeof(float));
  const int tile = k_tile ? 16 * D : 0;
  int k = (per_wave - tile) / shared_slot_floats(D);
  k = k < 1 ? 1 : (k > 4 ? 4 : k);
  *slots = k;
  *wave_floats = (tile + k * shared_slot_floats(D) + 3) / 4 * 4;
}

// Shared-prefix plan, made once for a batch's tables, lengths and groups and
// read by every attention and merge launch over them (every layer of a
// decode step): a header of kPlanHeaderInts ints, the per-sequence records
// the merge reads ([4][S], as ws_seq, padded to 64 ints), then one record of
// kPlanItemInts ints per work item -- its description (part, sequence, first
// kv head, first score column or -1, columns, first and end token, query-head
// chunk) and the first block-table window its waves read.
enum PlanField {
  kPlMagic, kPlS, kPlHq, kPlHkv, kPlB, kPlWidth, kPlMaxLen, kPlMaxPrefix, kPlGroups,
  kPlPartition, kPlStatus, kPlPrefixItems, kPlItems, kPlFields
};
constexpr int kPlanHeaderInts = 64;
constexpr int kPlanItemInts = 72;
constexpr int kPlanItemFields = 8;
constexpr int32_t kPlanMagic = 0x53504b50;
__host__ __device__ inline int64_t plan_items_off(int S) {
  return kPlanHeaderInts + (static_cast<int64_t>(4) * S + 63) / 64 * 64;
}
// Does the plan describe a batch of these arguments, with every item
// recorded?  (kPlStatus: 0, or 1 when the items exceeded the capacity.)
// Its per-sequence records are copied into the workspace by the attention
// launch, so the merge reads them as without a plan.
__device__ inline bool plan_matches(const AttnArgs& a) {
  const int32_t* h = a.plan;
  return h[kPlMagic] == kPlanMagic && h[kPlS] == a.S && h[kPlHq] == a.Hq && h[kPlHkv] == a.Hkv &&
         h[kPlB] == a.B && h[kPlWidth] == a.width && h[kPlMaxLen] == a.max_len &&
         h[kPlMaxPrefix] == a.max_prefix && h[kPlGroups] == a.num_groups &&
         h[kPlPartition] == a.partition && h[kPlStatus] == 0;
}

// Prefill (chunked) attention: sequence s's chunk is query rows
// [qstart[s], qstart[s + 1]) at positions lens[s] - chunk_len .. lens[s] - 1.
struct PrefillArgs {
  void* out;             // [T][Hq][D] fp32 or bf16
  const void* query;     // [T][Hq][D]
  const void* kv;        // [2][NB][B][Hkv][D]
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* qstart;  // [S + 1]
  int width, S, T, Hq, Hkv, D, B, NB;
  float scale_log2;
  int out_bf16;
  int max_q;           // longest chunk the grid covers (longer ones give NaN)
  int qtiles;          // tiles of query vectors per (sequence, kv head) at most
  int total;           // work items (workgroups): tiles x Hkv
};

int launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// most sequences one bf16 prefill launch takes (its work ranking lives in LDS)
int prefill_max_seqs(int head_size);
// query vectors per bf16 prefill tile (one workgroup each)
int prefill_tile_vectors(int head_size);
int launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

int launch_attention_bf16(const AttnArgs& a, hipStream_t stream);
int launch_attention_bf16_shared(const AttnArgs& a, hipStream_t stream);
// the plan launch: a's schedule fields, the plan, its item capacity
int launch_shared_plan(const AttnArgs& a, int32_t* plan, int64_t capacity, hipStream_t stream);
int launch_reduce_shared(const AttnArgs& a, hipStream_t stream);
int launch_attention_bf16_stream(const AttnArgs& a, hipStream_t stream);
int launch_attention_f32(const AttnArgs& a, hipStream_t stream);
int launch_reduce(const AttnArgs& a, hipStream_t stream);

}  // namespace pkv
