// C ABI entry points: host-side argument checks, partition choice and
// dispatch to the kernels.  Nothing here touches device memory contents.
#include "common.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <mutex>

namespace pkv {

// (a fixed buffer: reporting an error allocates nothing)
static thread_local char g_error[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
}

void clear_error() { g_error[0] = '\0'; }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

int raise_lds_limit(const void* kern, int bytes) {
  if (bytes <= 0) bytes = static_cast<int>(bf16_lds_limit());
  // (kernel, device) pairs already raised, in fixed storage (the launch
  // path allocates nothing); a pair that finds the table full is raised
  // again on every launch, which is correct, only slower
  struct Done {
    const void* kern;
    int dev;
  };
  constexpr int kMaxDone = 1024;
  static Done done[kMaxDone];
  static int ndone = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_error("cannot query the current device");
    return PKV_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < ndone; ++i)
    if (done[i].kern == kern && done[i].dev == dev) return PKV_OK;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) {
    (void)hipGetLastError();
    set_error("cannot raise a kernel's LDS limit to %d bytes", bytes);
    return PKV_ERR_HIP;
  }
  if (ndone < kMaxDone) done[ndone++] = Done{kern, dev};
  return PKV_OK;
}

namespace {

constexpr int kMaxParts = 8192;  // partitions per sequence the merge supports
constexpr int kGridYZ = 65535;

int elem_bytes(pkv_dtype t) { return t == PKV_F32 ? 4 : (t == PKV_BF16 ? 2 : 0); }

int gcd(int a, int b) { return b ? gcd(b, a % b) : a; }

// The address a kernel uses for p: p itself for device memory, the mapped
// device address for pinned host memory.  Pageable host memory (or an
// unknown pointer) is refused here rather than faulting in the kernel.
bool device_address(const void* p, const char* what, void** out) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    set_error("%s: not device memory or pinned host memory", what);
    return false;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = const_cast<void*>(p);
    return true;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer) {
    *out = attr.devicePointer;
    return true;
  }
  set_error("%s: not device memory or pinned host memory (type %d)", what,
            static_cast<int>(attr.type));
  return false;
}

// Partitions are whole 32-token wave steps and whole blocks.
int partition_unit(int B) { return 32 / gcd(32, B) * B; }

bool shape_ok(int S, int Hq, int Hkv, int D, int B, int max_len, pkv_dtype dtype) {
  if (elem_bytes(dtype) == 0) { set_error("unknown dtype %d", static_cast<int>(dtype)); return false; }
  if (S < 0 || S > kGridYZ) { set_error("num_seqs %d outside [0, %d]", S, kGridYZ); return false; }
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) {
    set_error("num_q_heads %d must be a positive multiple of num_kv_heads %d", Hq, Hkv);
    return false;
  }
  if (max_len < 0) { set_error("max_context_len %d < 0", max_len); return false; }
  if (B <= 0) { set_error("block_size %d <= 0", B); return false; }
  (void)D;
  return true;
}

constexpr int kResidentGroups = 512;  // workgroups of the bf16 kernel resident at once (2 per CU)

// (sequence, kv-head group, query-head chunk) work units of the bf16 kernel
int64_t bf16_units(int S, int Hq, int Hkv) {
  const int G = Hq / Hkv;
  return static_cast<int64_t>(S) * (Hkv / bf16_heads_per_group(Hkv)) * ((G + 15) / 16);
}

// Partition size: a request is checked; 0 picks one.  The bf16 kernel keeps
// whole sequences in one partition (no merge pass) when there are enough work
// units to fill the GPU without splitting; otherwise contexts are split into
// 256-token partitions, short enough that the longest sequence of a ragged
// batch is spread over many workgroups.  fp32 uses 64-token partitions.
int resolve_partition(int S, int Hq, int Hkv, int D, int B, int max_len, int req, pkv_dtype dtype) {
  (void)D;
  const int unit = partition_unit(B);
  const int cap = dtype == PKV_F32 ? 512 : (1 << 20);
  if (req < 0) return -1;
  if (req > 0) return (req % unit == 0 && req <= cap) ? req : -1;
  const int whole = static_cast<int>(cdiv64(std::max(max_len, 1), unit) * unit);
  if (dtype == PKV_F32) return std::min(whole, std::max(unit, 64 / unit * unit));
  if (bf16_units(S, Hq, Hkv) >= kResidentGroups && whole <= (1 << 20)) return whole;
  return std::min(whole, std::max(unit, 256 / unit * unit));
}

// Partitions one bf16 workgroup covers.  A small batch of long sequences
// (at most 32) gets as many per wave as keep one full round of resident
// workgroups, so each wave streams a long token range; a larger batch gets one
// per wave, since its lengths may be ragged and a long run on its longest
// sequence would become the critical path.  Capped by what the waves can hold
// in LDS until they write it.
int bf16_parts_per_wg(int S, int Hq, int Hkv, int D, int max_parts, bool k_tile) {
  const int nslot = 4 / bf16_heads_per_group(Hkv);
  const int64_t units = bf16_units(S, Hq, Hkv);
  if (S > 32) return nslot;
  int64_t pps = units * max_parts / (static_cast<int64_t>(kResidentGroups) * nslot);
  pps = std::max<int64_t>(1, std::min<int64_t>(pps, cdiv64(max_parts, nslot)));
  while (pps > 1 && bf16_lds_bytes(static_cast<int>(pps), Hq / Hkv, D, k_tile) > bf16_lds_limit()) --pps;
  return static_cast<int>(pps) * nslot;
}

// The stream schedule serves bf16 caches with automatic partitioning when
// whole sequences would leave the GPU partly idle -- too few (sequence,
// kv-head group) work units to fill it, or a partial last round of them --
// and every sequence's length fits its scan.
bool uses_stream(int S, int Hq, int Hkv, int max_len, int req, pkv_dtype dtype) {
  if (dtype != PKV_BF16 || req != 0 || S > kMaxStreamSeqs) return false;
  // Whole sequences (no merge pass) when the batch fills the GPU in whole
  // rounds of resident workgroups, or in enough rounds that dispatch order
  // evens out the lengths, or when the merge would have many rows; the
  // stream otherwise -- a partial last round of whole sequences leaves most
  // of the GPU idle at the end.
  const int64_t units = bf16_units(S, Hq, Hkv);
  if (units >= kResidentGroups &&
      (units % kResidentGroups == 0 || units >= 4 * kResidentGroups ||
       static_cast<int64_t>(S) * Hq > 4096))
    return false;
  // stream steps are counted in 32-bit integers
  const int G = Hq / Hkv;
  const int64_t steps = static_cast<int64_t>(S) * Hkv * ((G + 15) / 16) * (max_len / 32 + 1);
  return steps < (int64_t{1} << 31);
}

// Under the stream schedule, new tokens are stored by the attention launch
// itself when few of its pieces hold a sequence's last step: each such piece
// stores the row and reads it back mid-piece, which cost the OPT-13B-shaped
// batch (most pieces hold one) more than the write launch it saves, while
// the Qwen2-shaped one (one piece in six) gains that launch.
bool stream_writes_in_launch(int S, int Hq, int Hkv, int waves) {
  const int HG = bf16_heads_per_group(Hkv);
  const int64_t units = static_cast<int64_t>(S) * (Hkv / HG) * ((Hq / Hkv + 15) / 16);
  return 2 * units <= waves / HG;
}

// Compute units of the current device (0 if it cannot be queried), asked of
// the runtime once per device.
int device_cus() {
  constexpr int kDevices = 64;
  static std::atomic<int> cached[kDevices];  // 0: not yet asked
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < kDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 0;
  if (dev >= 0 && dev < kDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Waves of the stream schedule's persistent grid on the current device.
int stream_waves(int D) { return device_cus() * stream_wgs_per_cu(D) * 4; }

// Workspace of the stream schedule: one partial-result slot (nhs rows of D
// floats and their (m, l)) per wave and per (sequence, kv head, query-head
// chunk) -- a piece of the stream is named by piece + pair, so that many
// slots cover every piece -- then the scan of the lengths, which tells the
// merge where each unit was cut.
struct StreamLayout {
  int64_t ml_off, pref_off, bytes;
};
StreamLayout stream_layout(int S, int Hq, int Hkv, int D, int waves) {
  const int G = Hq / Hkv;
  const int64_t units = static_cast<int64_t>(S) * Hkv * ((G + 15) / 16);
  const int64_t rows = (static_cast<int64_t>(waves) + units) * std::min(16, G);
  auto up256 = [](int64_t b) { return (b + 255) / 256 * 256; };
  StreamLayout l;
  l.ml_off = up256(rows * D * 4);
  l.pref_off = l.ml_off + up256(rows * 2 * 4);
  l.bytes = l.pref_off + up256(static_cast<int64_t>(S + 1) * 4);
  return l;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

const char* pkv_last_error(void) { return g_error; }

int paged_kv_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables, int table_width,
                          const int32_t* seq_ids, const int32_t* positions, int num_tokens,
                          int num_seqs, int block_size, int num_blocks, hipStream_t stream) {
  clear_error();
  if (num_tokens < 0 || num_seqs < 0 || table_width <= 0 || block_size <= 0 || num_blocks <= 0) {
    set_error("slot mapping: bad sizes (tokens %d, seqs %d, width %d, block %d, blocks %d)",
              num_tokens, num_seqs, table_width, block_size, num_blocks);
    return PKV_ERR_INVALID;
  }
  if (num_tokens > 0 && (!slot_mapping || !block_tables || !positions)) {
    set_error("slot mapping: null pointer");
    return PKV_ERR_INVALID;
  }
  return launch_slot_mapping(slot_mapping, block_tables, table_width, seq_ids, positions,
                             num_tokens, num_seqs, block_size, num_blocks, stream);
}

int paged_kv_write(const void* key, const void* value, void* kv_cache, const int64_t* slot_mapping,
                   int num_tokens, int num_blocks, int block_size, int num_kv_heads,
                   int head_size, pkv_dtype dtype, hipStream_t stream) {
  clear_error();
  const int eb = elem_bytes(dtype);
  if (eb == 0) { set_error("kv write: unknown dtype"); return PKV_ERR_INVALID; }
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_size <= 0) {
    set_error("kv write: bad sizes");
    return PKV_ERR_INVALID;
  }
  if ((head_size * eb) % 16) {
    set_error("kv write: head_size*%d bytes must be a multiple of 16", eb);
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !kv_cache || !slot_mapping) { set_error("kv write: null pointer"); return PKV_ERR_INVALID; }
  if (!aligned16(key) || !aligned16(value) || !aligned16(kv_cache)) {
    set_error("kv write: key, value and cache must be 16-byte aligned");
    return PKV_ERR_INVALID;
  }
  return launch_write(key, value, kv_cache, slot_mapping, num_tokens, num_blocks, block_size,
                      num_kv_heads, head_size, eb, stream);
}

int paged_kv_write_positions(const void* key, const void* value, void* kv_cache,
                             const int32_t* block_tables, int table_width, const int32_t* seq_ids,
                             const int32_t* positions, int64_t* slot_mapping, int num_tokens,
                             int num_seqs, int num_blocks, int block_size, int num_kv_heads,
                             int head_size, pkv_dtype dtype, hipStream_t stream) {
  clear_error();
  const int eb = elem_bytes(dtype);
  if (eb == 0) { set_error("kv write: unknown dtype"); return PKV_ERR_INVALID; }
  if (num_tokens < 0 || num_seqs < 0 || table_width <= 0 || num_blocks <= 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_size <= 0) {
    set_error("kv write: bad sizes");
    return PKV_ERR_INVALID;
  }
  if ((head_size * eb) % 16) {
    set_error("kv write: head_size*%d bytes must be a multiple of 16", eb);
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !kv_cache || !block_tables || !positions) {
    set_error("kv write: null pointer");
    return PKV_ERR_INVALID;
  }
  if (!aligned16(key) || !aligned16(value) || !aligned16(kv_cache)) {
    set_error("kv write: key, value and cache must be 16-byte aligned");
    return PKV_ERR_INVALID;
  }
  return launch_write_positions(key, value, kv_cache, block_tables, table_width, seq_ids, positions,
                                0, slot_mapping, num_tokens, num_seqs, num_blocks, block_size,
                                num_kv_heads, head_size, eb, stream);
}

int paged_kv_gather(void* k_out, void* v_out, const void* kv_cache, const int32_t* block_tables,
                    int table_width, const int32_t* context_lens, int num_seqs, int num_kv_heads,
                    int head_size, int block_size, int num_blocks, int max_context_len,
                    pkv_dtype dtype, hipStream_t stream) {
  clear_error();
  const int eb = elem_bytes(dtype);
  if (eb == 0) { set_error("kv gather: unknown dtype"); return PKV_ERR_INVALID; }
  if (num_seqs < 0 || num_seqs > kGridYZ || table_width <= 0 || num_kv_heads <= 0 ||
      head_size <= 0 || block_size <= 0 || num_blocks <= 0 || max_context_len < 0) {
    set_error("kv gather: bad sizes");
    return PKV_ERR_INVALID;
  }
  if ((head_size * eb) % 16) { set_error("kv gather: head_size bytes must be a multiple of 16"); return PKV_ERR_UNSUPPORTED; }
  if (num_seqs == 0 || max_context_len == 0) return PKV_OK;
  if (!k_out || !v_out || !kv_cache || !block_tables || !context_lens) {
    set_error("kv gather: null pointer");
    return PKV_ERR_INVALID;
  }
  if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(kv_cache)) {
    set_error("kv gather: buffers must be 16-byte aligned");
    return PKV_ERR_INVALID;
  }
  return launch_gather(k_out, v_out, kv_cache, block_tables, table_width, context_lens, num_seqs,
                       num_kv_heads, head_size, block_size, num_blocks, max_context_len, eb, stream);
}

int paged_kv_copy_blocks(void* dst_cache, int dst_num_blocks, const void* src_cache,
                         int src_num_blocks, const int32_t* src_blocks, const int32_t* dst_blocks,
                         int num_copies, int block_size, int num_kv_heads, int head_size,
                         pkv_dtype dtype, hipStream_t stream) {
  clear_error();
  const int eb = elem_bytes(dtype);
  if (eb == 0) { set_error("copy blocks: unknown dtype"); return PKV_ERR_INVALID; }
  if (num_copies < 0 || num_copies > (1 << 30) || dst_num_blocks <= 0 || src_num_blocks <= 0 ||
      block_size <= 0 || num_kv_heads <= 0 || head_size <= 0) {
    set_error("copy blocks: bad sizes");
    return PKV_ERR_INVALID;
  }
  if ((static_cast<int64_t>(head_size) * eb) % 16) {
    set_error("copy blocks: head_size*%d bytes must be a multiple of 16", eb);
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_copies == 0) return PKV_OK;
  if (!dst_cache || !src_cache || !src_blocks || !dst_blocks) {
    set_error("copy blocks: null pointer");
    return PKV_ERR_INVALID;
  }
  if (!aligned16(dst_cache) || !aligned16(src_cache)) {
    set_error("copy blocks: pools must be 16-byte aligned");
    return PKV_ERR_INVALID;
  }
  void *dst = nullptr, *src = nullptr, *src_ids = nullptr, *dst_ids = nullptr;
  if (!device_address(dst_cache, "copy blocks: dst_cache", &dst) ||
      !device_address(src_cache, "copy blocks: src_cache", &src) ||
      !device_address(src_blocks, "copy blocks: src_blocks", &src_ids) ||
      !device_address(dst_blocks, "copy blocks: dst_blocks", &dst_ids)) {
    return PKV_ERR_INVALID;
  }
  const int64_t half = static_cast<int64_t>(block_size) * num_kv_heads * head_size * eb;
  return launch_copy_blocks(dst, dst_num_blocks, src, src_num_blocks,
                            static_cast<const int32_t*>(src_ids),
                            static_cast<const int32_t*>(dst_ids), num_copies, half, stream);
}

int paged_attention_partition_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_size,
                                   int block_size, int max_context_len, int partition_size,
                                   pkv_dtype dtype) {
  clear_error();
  if (!shape_ok(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, max_context_len, dtype))
    return -1;
  if (uses_stream(num_seqs, num_q_heads, num_kv_heads, max_context_len, partition_size, dtype))
    return 0;
  const int P = resolve_partition(num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                                  max_context_len, partition_size, dtype);
  if (P < 0) set_error("partition_size %d is not a positive multiple of %d (fp32: at most 512)",
                       partition_size, partition_unit(block_size));
  return P;
}

size_t paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_size, int block_size, int max_context_len,
                                       int partition_size, pkv_dtype dtype) {
  const int P = paged_attention_partition_size(num_seqs, num_q_heads, num_kv_heads, head_size,
                                               block_size, max_context_len, partition_size, dtype);
  if (P == 0 && num_seqs > 0) {
    const int waves = stream_waves(head_size);
    return waves > 0 ? static_cast<size_t>(
                           stream_layout(num_seqs, num_q_heads, num_kv_heads, head_size, waves).bytes)
                     : 0;
  }
  if (P <= 0) return 0;
  const int64_t parts = cdiv64(std::max(max_context_len, 1), P);
  if (parts <= 1) return 0;
  const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads * parts;
  const int64_t o_bytes = (rows * head_size * 4 + 255) / 256 * 256;
  return static_cast<size_t>(o_bytes + rows * 2 * 4);
}

}  // extern "C"

namespace {

enum Phase { kAttend = 1, kMerge = 2 };

// The stream schedule (arguments already checked).
int decode_stream(int phases, void* out, pkv_dtype out_dtype, const void* query,
                  const void* kv_cache, const int32_t* block_tables, int table_width,
                  const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                  int head_size, int block_size, int num_blocks, float scale, int max_context_len,
                  void* workspace, size_t workspace_bytes, pkv_dtype dtype, unsigned flags,
                  hipStream_t stream, const void* key_new, const void* value_new) {
  const int waves = stream_waves(head_size);
  if (waves <= 0) {
    set_error("cannot query the current device");
    return PKV_ERR_HIP;
  }
  const StreamLayout lay = stream_layout(num_seqs, num_q_heads, num_kv_heads, head_size, waves);
  if (!workspace || workspace_bytes < static_cast<size_t>(lay.bytes)) {
    set_error("workspace of %zu bytes is smaller than the %lld needed", workspace_bytes,
              static_cast<long long>(lay.bytes));
    return PKV_ERR_WORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) {
    set_error("workspace must be 256-byte aligned");
    return PKV_ERR_INVALID;
  }
  AttnArgs a{};
  a.out = out;
  a.query = query;
  a.kv = kv_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.width = table_width;
  a.S = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.D = head_size;
  a.B = block_size;
  a.NB = num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = out_dtype == PKV_BF16 ? 1 : 0;
  a.nontemporal = (flags & PKV_ATTN_CACHED_KV) ? 0 : 1;
  a.k_via_lds = static_cast<int64_t>(num_kv_heads) * head_size * elem_bytes(dtype) >= 4096;
  a.max_len = max_context_len;
  // New tokens: stored by the attention launch itself or by a write launch
  // first (stream_writes_in_launch).
  if (key_new) {
    if (stream_writes_in_launch(num_seqs, num_q_heads, num_kv_heads, waves)) {
      a.k_new = key_new;
      a.v_new = value_new;
    } else if (phases & kAttend) {
      const int rc = launch_write_positions(key_new, value_new, const_cast<void*>(kv_cache),
                                            block_tables, table_width, nullptr, context_lens, -1,
                                            nullptr, num_seqs, num_seqs, num_blocks, block_size,
                                            num_kv_heads, head_size, elem_bytes(dtype), stream);
      if (rc != PKV_OK) return rc;
    }
  }
  a.stream = 1;
  a.stream_waves = waves;
  stream_lds_plan(num_q_heads / num_kv_heads, head_size, a.k_via_lds != 0, &a.stream_slots,
                  &a.stream_wave_floats);
  char* ws = static_cast<char*>(workspace);
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(ws + lay.ml_off);
  a.ws_pref = reinterpret_cast<int*>(ws + lay.pref_off);
  if (phases & kAttend) {
    const int rc = launch_attention_bf16(a, stream);
    if (rc != PKV_OK) return rc;
  }
  if (phases & kMerge) return launch_reduce(a, stream);
  return PKV_OK;
}

int decode_impl(int phases, void* out, pkv_dtype out_dtype, const void* query,
                const void* kv_cache, const int32_t* block_tables, int table_width,
                const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                int head_size, int block_size, int num_blocks, float scale, int max_context_len,
                int partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                unsigned flags, hipStream_t stream, const void* key_new = nullptr,
                const void* value_new = nullptr) {
  clear_error();
  if (!shape_ok(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, max_context_len, dtype))
    return PKV_ERR_INVALID;
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) { set_error("unknown out_dtype"); return PKV_ERR_INVALID; }
  if (head_size != 64 && head_size != 128) {
    set_error("head_size %d is not built (64 or 128)", head_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (dtype == PKV_BF16 && block_size != 8 && block_size != 16 && block_size != 32 &&
      block_size != 64) {
    set_error("bf16 path: block_size %d is not built (8, 16, 32 or 64)", block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (dtype == PKV_F32 && block_size > 256) {
    set_error("fp32 path: block_size %d above 256", block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (table_width <= 0 || num_blocks <= 0) { set_error("table_width and num_blocks must be positive"); return PKV_ERR_INVALID; }
  if (!std::isfinite(scale)) { set_error("scale is not finite"); return PKV_ERR_INVALID; }
  if (flags & ~static_cast<unsigned>(PKV_ATTN_CACHED_KV)) {
    set_error("unknown flags 0x%x", flags);
    return PKV_ERR_INVALID;
  }
  const int G = num_q_heads / num_kv_heads;
  if (static_cast<int64_t>(num_kv_heads) * ((G + 15) / 16) > kGridYZ) {
    set_error("too many kv heads for the grid");
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !kv_cache || !block_tables || !context_lens) {
    set_error("null pointer argument");
    return PKV_ERR_INVALID;
  }
  if (!aligned16(out) || !aligned16(query) || !aligned16(kv_cache)) {
    set_error("out, query and kv_cache must be 16-byte aligned");
    return PKV_ERR_INVALID;
  }
  if (key_new || value_new) {
    if (!key_new || !value_new) {
      set_error("key and value of the new tokens: null pointer");
      return PKV_ERR_INVALID;
    }
    if (!aligned16(key_new) || !aligned16(value_new)) {
      set_error("key and value of the new tokens must be 16-byte aligned");
      return PKV_ERR_INVALID;
    }
  }
  if (uses_stream(num_seqs, num_q_heads, num_kv_heads, max_context_len, partition_size, dtype))
    return decode_stream(phases, out, out_dtype, query, kv_cache, block_tables, table_width,
                         context_lens, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                         num_blocks, scale, max_context_len, workspace, workspace_bytes, dtype,
                         flags, stream, key_new, value_new);
  const int P = resolve_partition(num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                                  max_context_len, partition_size, dtype);
  if (P <= 0) {
    set_error("partition_size %d is not a positive multiple of %d (fp32: at most 512)",
              partition_size, partition_unit(block_size));
    return PKV_ERR_INVALID;
  }
  const int64_t parts = cdiv64(std::max(max_context_len, 1), P);
  if (parts > kMaxParts) {
    set_error("%lld partitions per sequence exceed %d; use a larger partition_size",
              static_cast<long long>(parts), kMaxParts);
    return PKV_ERR_UNSUPPORTED;
  }
  AttnArgs a{};
  a.out = out;
  a.query = query;
  a.kv = kv_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.width = table_width;
  a.S = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.D = head_size;
  a.B = block_size;
  a.NB = num_blocks;
  a.partition = P;
  a.max_parts = static_cast<int>(parts);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = out_dtype == PKV_BF16 ? 1 : 0;
  a.nontemporal = (flags & PKV_ATTN_CACHED_KV) ? 0 : 1;
  // Longest sequences first, so the longest work starts earliest and short
  // sequences fill the tail -- except when blocks are shared: sequences that
  // share blocks come adjacent in a batch and should run together to hit in
  // the caches.  Each workgroup ranks the lengths itself, so only for small
  // batches.
  a.longest_first = !(flags & PKV_ATTN_CACHED_KV) && num_seqs <= kMaxRankedSeqs;
  // Shared blocks are read once per L2 when the sequences sharing them run
  // on one XCD.
  a.xcd_blocked = (flags & PKV_ATTN_CACHED_KV) ? 1 : 0;
  // Keys take the LDS path when a token's row across all kv heads is long
  // (>= 4 KB): one head's 64-byte pieces of such rows stream poorly, while
  // for short rows the direct MFMA-layout load is faster.
  a.k_via_lds = static_cast<int64_t>(num_kv_heads) * head_size * elem_bytes(dtype) >= 4096;
  a.parts_per_wg = dtype == PKV_BF16
                       ? bf16_parts_per_wg(num_seqs, num_q_heads, num_kv_heads, head_size, a.max_parts,
                                           a.k_via_lds != 0)
                       : 1;
  // When contexts are split into several workgroup runs, a ragged batch
  // leaves most of a grid sized by the longest context empty, and dispatching
  // the empty workgroups takes longer than the work: workgroups then number
  // the real work items themselves and walk that list instead.
  a.compact = dtype == PKV_BF16 && num_seqs <= kMaxCompactSeqs &&
              cdiv64(a.max_parts, a.parts_per_wg) > 1;
  if (a.compact) a.longest_first = 0;
  if (parts > 1) {
    const size_t need = paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                        head_size, block_size, max_context_len,
                                                        P, dtype);
    if (!workspace || workspace_bytes < need) {
      set_error("workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
      return PKV_ERR_WORKSPACE;
    }
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) {
      set_error("workspace must be 256-byte aligned");
      return PKV_ERR_INVALID;
    }
    const int64_t rows = static_cast<int64_t>(num_seqs) * num_q_heads * parts;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       (rows * head_size * 4 + 255) / 256 * 256);
  }
  // fp32: the attention launch stores the new tokens itself (each
  // sequence's at position context_lens[s] - 1); the bf16 fixed partitions
  // write them first, then read them like the rest
  if (key_new && dtype == PKV_F32) {
    a.k_new = key_new;
    a.v_new = value_new;
  }
  if (phases & kAttend) {
    if (key_new && dtype != PKV_F32) {
      const int rc = launch_write_positions(key_new, value_new, const_cast<void*>(kv_cache),
                                            block_tables, table_width, nullptr, context_lens, -1,
                                            nullptr, num_seqs, num_seqs, num_blocks, block_size,
                                            num_kv_heads, head_size, elem_bytes(dtype), stream);
      if (rc != PKV_OK) return rc;
    }
    const int rc = dtype == PKV_BF16 ? launch_attention_bf16(a, stream) : launch_attention_f32(a, stream);
    if (rc != PKV_OK) return rc;
  }
  if (phases & kMerge) return launch_reduce(a, stream);
  return PKV_OK;
}

}  // namespace

#define PKV_DECODE_ARGS                                                                        \
  out, out_dtype, query, kv_cache, block_tables, table_width, context_lens, num_seqs,          \
      num_q_heads, num_kv_heads, head_size, block_size, num_blocks, scale, max_context_len,    \
      partition_size, workspace, workspace_bytes, dtype, flags, stream

#define PKV_DECODE_PARAMS                                                                      \
  void *out, pkv_dtype out_dtype, const void *query, const void *kv_cache,                     \
      const int32_t *block_tables, int table_width, const int32_t *context_lens, int num_seqs, \
      int num_q_heads, int num_kv_heads, int head_size, int block_size, int num_blocks,        \
      float scale, int max_context_len, int partition_size, void *workspace,                   \
      size_t workspace_bytes, pkv_dtype dtype, unsigned flags, hipStream_t stream

extern "C" {

int paged_attention_prefill(void* out, pkv_dtype out_dtype, const void* query,
                            const int32_t* query_start, int num_tokens, int max_query_len,
                            const void* kv_cache, const int32_t* block_tables, int table_width,
                            const int32_t* context_lens, int num_seqs, int num_q_heads,
                            int num_kv_heads, int head_size, int block_size, int num_blocks,
                            float scale, pkv_dtype dtype, hipStream_t stream) {
  clear_error();
  if (!shape_ok(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, 0, dtype))
    return PKV_ERR_INVALID;
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) { set_error("unknown out_dtype"); return PKV_ERR_INVALID; }
  if (num_tokens < 0 || max_query_len < 0) {
    set_error("num_tokens %d and max_query_len %d must be >= 0", num_tokens, max_query_len);
    return PKV_ERR_INVALID;
  }
  if (head_size != 64 && head_size != 128) {
    set_error("head_size %d is not built (64 or 128)", head_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (dtype == PKV_BF16 && block_size != 8 && block_size != 16 && block_size != 32 &&
      block_size != 64) {
    set_error("bf16 prefill: block_size %d is not built (8, 16, 32 or 64)", block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (table_width <= 0 || num_blocks <= 0) { set_error("table_width and num_blocks must be positive"); return PKV_ERR_INVALID; }
  if (!std::isfinite(scale)) { set_error("scale is not finite"); return PKV_ERR_INVALID; }
  if (num_q_heads > kGridYZ) { set_error("num_q_heads %d above %d", num_q_heads, kGridYZ); return PKV_ERR_UNSUPPORTED; }
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !query || !query_start || !kv_cache || !block_tables || !context_lens) {
    set_error("null pointer argument");
    return PKV_ERR_INVALID;
  }
  if (!aligned16(out) || !aligned16(query) || !aligned16(kv_cache)) {
    set_error("out, query and kv_cache must be 16-byte aligned");
    return PKV_ERR_INVALID;
  }
  PrefillArgs a{};
  a.out = out;
  a.query = query;
  a.kv = kv_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.qstart = query_start;
  a.width = table_width;
  a.S = num_seqs;
  a.T = num_tokens;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.D = head_size;
  a.B = block_size;
  a.NB = num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = out_dtype == PKV_BF16;
  a.max_q = max_query_len;
  if (dtype == PKV_F32) return launch_prefill_f32(a, stream);
  // One workgroup per (tile, kv head); a tile is a run of query vectors of
  // one kv head (rows x its G query heads).  A chunk has at most qtiles
  // tiles, and chunks that follow each other in [0, num_tokens) (query_start
  // non-decreasing) have at most one per tile's vectors plus one each.
  const int64_t G = num_q_heads / num_kv_heads;
  if (static_cast<int64_t>(num_tokens) * G >= (int64_t{1} << 31) ||
      static_cast<int64_t>(max_query_len) * G >= (int64_t{1} << 31)) {
    set_error("prefill: %d tokens x %lld query heads per kv head is too large", num_tokens,
              static_cast<long long>(G));
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_seqs > prefill_max_seqs(head_size)) {
    set_error("bf16 prefill takes at most %d sequences per launch (got %d)",
              prefill_max_seqs(head_size), num_seqs);
    return PKV_ERR_UNSUPPORTED;
  }
  const int tile = prefill_tile_vectors(head_size);
  a.qtiles = static_cast<int>(cdiv64(static_cast<int64_t>(max_query_len) * G, tile));
  const int64_t tiles = std::min<int64_t>(static_cast<int64_t>(num_seqs) * a.qtiles,
                                          cdiv64(static_cast<int64_t>(num_tokens) * G, tile) + num_seqs);
  const int64_t total = tiles * num_kv_heads;
  if (total > (int64_t{1} << 30)) {
    set_error("prefill grid of %lld work items is too large", static_cast<long long>(total));
    return PKV_ERR_UNSUPPORTED;
  }
  a.total = static_cast<int>(total);
  return launch_prefill_bf16(a, stream);
}

int paged_attention_decode(PKV_DECODE_PARAMS) { return decode_impl(kAttend | kMerge, PKV_DECODE_ARGS); }

}  // extern "C"

// ---------------------------------------------------------------- no allocation

namespace pkv {
namespace {

// The workspace of paged_attention_decode_noalloc: a device array of the
// library's own, present on every GPU the library runs on from module load
// to process end.  Host code never uses its name as an address (on the host
// that names a stand-in, not device memory): the array's device address is
// looked up once per device and kept in scratch_ptr.
__device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The array's address on the current device (nullptr, with the error set,
// if it cannot be found).
void* scratch_on_device() {
  static void* ptr[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("no-allocation decode: cannot query the current device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      set_error("no-allocation decode: cannot find the scratch array on device %d", dev);
      return nullptr;
    }
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace
}  // namespace pkv

extern "C" {

int paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype, const void* query,
                                   const void* kv_cache, const int32_t* block_tables,
                                   int table_width, const int32_t* context_lens, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_size,
                                   int block_size, int num_blocks, float scale,
                                   int max_context_len, int partition_size, pkv_dtype dtype,
                                   unsigned flags, hipStream_t stream) {
  clear_error();
  const size_t need = paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                      head_size, block_size, max_context_len,
                                                      partition_size, dtype);
  if (need > static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES)) {
    set_error("no-allocation decode: this batch needs %zu bytes of workspace, above the %d the "
              "library holds; use paged_attention_decode with a workspace",
              need, PKV_NOALLOC_SCRATCH_BYTES);
    return PKV_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_device();
    if (ws == nullptr) return PKV_ERR_HIP;
  }
  return decode_impl(kAttend | kMerge, out, out_dtype, query, kv_cache, block_tables, table_width,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,
                     num_blocks, scale, max_context_len, partition_size, ws,
                     static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES), dtype, flags, stream);
}

int paged_attention_partitions(PKV_DECODE_PARAMS) { return decode_impl(kAttend, PKV_DECODE_ARGS); }

int paged_attention_merge(PKV_DECODE_PARAMS) { return decode_impl(kMerge, PKV_DECODE_ARGS); }

#define PKV_APPEND_PARAMS                                                                      \
  void *out, pkv_dtype out_dtype, const void *query, const void *key, const void *value,      \
      void *kv_cache, const int32_t *block_tables, int table_width, const int32_t *context_lens, \
      int num_seqs, int num_q_heads, int num_kv_heads, int head_size, int block_size,          \
      int num_blocks, float scale, int max_context_len, int partition_size, void *workspace,   \
      size_t workspace_bytes, pkv_dtype dtype, unsigned flags, hipStream_t stream

int paged_attention_append_in_launch(int num_seqs, int num_q_heads, int num_kv_heads,
                                     int head_size, int block_size, int max_context_len,
                                     int partition_size, pkv_dtype dtype) {
  (void)block_size;
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || num_seqs < 0) return -1;
  if (dtype == PKV_F32) return 1;
  if (!uses_stream(num_seqs, num_q_heads, num_kv_heads, max_context_len, partition_size, dtype))
    return 0;
  const int waves = stream_waves(head_size);
  if (waves <= 0) return -1;
  return stream_writes_in_launch(num_seqs, num_q_heads, num_kv_heads, waves) ? 1 : 0;
}

int paged_attention_decode_append(PKV_APPEND_PARAMS) {
  return decode_impl(kAttend | kMerge, PKV_DECODE_ARGS, key, value);
}

int paged_attention_append_partitions(PKV_APPEND_PARAMS) {
  return decode_impl(kAttend, PKV_DECODE_ARGS, key, value);
}

}  // extern "C"

// ---------------------------------------------------------------- shared prefixes

namespace pkv {
namespace {

// Workgroups of the shared-prefix kernel resident at once on the current
// device (0 if it cannot be queried).
int shared_resident_wgs() { return device_cus() * kSharedWgsPerCu; }

// Items of a group's prefix partition: (kv-head groups) x (16-column blocks
// of its members' query heads); estimated for groups of equal size.
int64_t shared_items_per_partition(int S, int Hq, int Hkv, int num_groups) {
  const int G = Hq / Hkv;
  const int64_t per_group = cdiv64(cdiv64(S, num_groups) * G, 16);
  return static_cast<int64_t>(Hkv / bf16_heads_per_group(Hkv)) * per_group * num_groups;
}

// A requested partition size is checked; 0 picks the largest one that still
// gives prefix items for about half the resident item slots (the suffix
// items fill the rest; longer prefix partitions leave fewer parts to merge,
// and measured no slower), or 256 tokens when there is no prefix.
int resolve_shared_partition(int S, int Hq, int Hkv, int B, int num_groups, int max_prefix,
                             int req) {
  const int unit = partition_unit(B);
  if (req < 0) return -1;
  if (req > 0) return req % unit == 0 ? req : -1;
  if (max_prefix <= 0 || S <= 0 || num_groups <= 0) return std::max(unit, 256 / unit * unit);
  const int64_t slots = static_cast<int64_t>(shared_resident_wgs()) * (4 / bf16_heads_per_group(Hkv));
  const int64_t per_part = std::max<int64_t>(1, shared_items_per_partition(S, Hq, Hkv, num_groups));
  const int64_t parts = std::max<int64_t>(1, cdiv64(slots, 2 * per_part));
  const int64_t P = max_prefix / parts / unit * unit;
  return static_cast<int>(std::max<int64_t>(unit, std::min<int64_t>(P, cdiv64(max_prefix, unit) * unit)));
}

struct SharedLayout {
  int64_t parts, ml_off, seq_off, bytes;
};
// Partial results [parts][S][Hq][D] floats, their (m, l) [parts][S][Hq][2],
// then per sequence: parts, group leader, prefix length, table mismatch
// (int32 [4][S]).
SharedLayout shared_layout(int S, int Hq, int D, int max_len, int max_prefix, int P) {
  auto up256 = [](int64_t b) { return (b + 255) / 256 * 256; };
  SharedLayout l;
  l.parts = cdiv64(std::max(max_prefix, 0), P) + cdiv64(std::max(max_len, 1), P);
  const int64_t rows = l.parts * S * Hq;
  l.ml_off = up256(rows * D * 4);
  l.seq_off = l.ml_off + up256(rows * 2 * 4);
  l.bytes = l.seq_off + up256(static_cast<int64_t>(4) * S * 4);
  return l;
}

// Work items at most: prefix items are at most (kv-head groups) x (column
// blocks, at most S*G/16 + groups) x parts, suffix items (kv-head groups) x
// (head chunks) x parts per sequence.
int64_t shared_item_bound(int S, int Hq, int Hkv, int num_groups, int max_len, int max_prefix,
                          int P) {
  const int G = Hq / Hkv;
  const int64_t hgn = Hkv / bf16_heads_per_group(Hkv);
  return hgn * (cdiv64(static_cast<int64_t>(S) * G, 16) + num_groups) * cdiv64(max_prefix, P) +
         static_cast<int64_t>(S) * hgn * cdiv64(G, 16) * cdiv64(std::max(max_len, 1), P);
}

// Bytes of a plan: header, per-sequence records, one record per item.
int64_t shared_plan_bytes(int S, int64_t items) {
  return (plan_items_off(S) + items * kPlanItemInts) * static_cast<int64_t>(sizeof(int32_t));
}

}  // namespace
}  // namespace pkv

extern "C" {

int paged_attention_prefix_groups(const int32_t* block_tables, int table_width,
                                  const int32_t* context_lens, int num_seqs, int block_size,
                                  int min_prefix_len, int32_t* group_starts, int32_t* prefix_lens,
                                  int* num_groups, int* max_prefix_len) {
  clear_error();
  if (num_seqs < 0 || block_size <= 0 || table_width < 0) {
    set_error("num_seqs %d, block_size %d, table_width %d: invalid", num_seqs, block_size,
              table_width);
    return PKV_ERR_INVALID;
  }
  if (!group_starts || !num_groups || !max_prefix_len ||
      (num_seqs > 0 && (!block_tables || !context_lens || !prefix_lens || table_width == 0))) {
    set_error("null pointer argument");
    return PKV_ERR_INVALID;
  }
  const int unit = partition_unit(block_size);
  // whole partition units of the first `blocks` blocks, within length L
  auto usable = [&](int64_t blocks, int L) {
    const int64_t t = std::min<int64_t>(blocks * block_size, L);
    return static_cast<int>(t / unit * unit);
  };
  auto nblocks = [&](int L) {
    return static_cast<int>(std::min<int64_t>(cdiv64(L, block_size), table_width));
  };
  int ng = 0, maxp = 0;
  group_starts[0] = 0;
  if (num_seqs > 0) {
    int lead = 0;
    int64_t common = -1;  // blocks every member shares with the leader (-1: one member)
    int min_len = std::max(context_lens[0], 0);
    auto close = [&](int end) {
      const int p = (end - group_starts[ng] >= 2 && common > 0) ? usable(common, min_len) : 0;
      prefix_lens[ng] = p;
      maxp = std::max(maxp, p);
      group_starts[++ng] = end;
    };
    for (int s = 1; s < num_seqs; ++s) {
      const int L = std::max(context_lens[s], 0);
      const int n = std::min(nblocks(L), nblocks(std::max(context_lens[lead], 0)));
      const int32_t* a = block_tables + static_cast<int64_t>(s) * table_width;
      const int32_t* b = block_tables + static_cast<int64_t>(lead) * table_width;
      int64_t k = 0;
      while (k < n && a[k] == b[k]) ++k;
      const int64_t cand = common < 0 ? k : std::min(common, k);
      const int tok = usable(cand, std::min(min_len, L));
      const int cur = common < 0 ? 0 : usable(common, min_len);
      if (tok > 0 && tok >= min_prefix_len && tok >= cur) {
        common = cand;
        min_len = std::min(min_len, L);
      } else {
        close(s);
        lead = s;
        common = -1;
        min_len = L;
      }
    }
    close(num_seqs);
  }
  *num_groups = ng;
  *max_prefix_len = maxp;
  return PKV_OK;
}

int paged_attention_shared_partition_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                          int head_size, int block_size, int num_groups,
                                          int max_prefix_len, int partition_size) {
  clear_error();
  if (!shape_ok(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, 0, PKV_BF16)) return -1;
  const int P = resolve_shared_partition(num_seqs, num_q_heads, num_kv_heads, block_size,
                                         num_groups, max_prefix_len, partition_size);
  if (P < 0) set_error("partition_size %d is not a positive multiple of %d", partition_size,
                       partition_unit(block_size));
  return P;
}

size_t paged_attention_shared_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                              int head_size, int block_size, int num_groups,
                                              int max_context_len, int max_prefix_len,
                                              int partition_size) {
  const int P = paged_attention_shared_partition_size(num_seqs, num_q_heads, num_kv_heads,
                                                      head_size, block_size, num_groups,
                                                      max_prefix_len, partition_size);
  if (P <= 0 || num_seqs <= 0) return 0;
  return static_cast<size_t>(
      shared_layout(num_seqs, num_q_heads, head_size, max_context_len, max_prefix_len, P).bytes);
}

size_t paged_attention_shared_plan_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                         int block_size, int num_groups, int max_context_len,
                                         int max_prefix_len, int partition_size) {
  clear_error();
  if (!shape_ok(num_seqs, num_q_heads, num_kv_heads, 0, block_size, max_context_len, PKV_BF16) ||
      max_prefix_len < 0 || num_seqs == 0 || num_groups < 1 || num_groups > num_seqs)
    return 0;
  const int P = resolve_shared_partition(num_seqs, num_q_heads, num_kv_heads, block_size,
                                         num_groups, max_prefix_len, partition_size);
  if (P <= 0) return 0;
  return static_cast<size_t>(shared_plan_bytes(
      num_seqs, shared_item_bound(num_seqs, num_q_heads, num_kv_heads, num_groups, max_context_len,
                                  max_prefix_len, P)));
}

int paged_attention_shared_plan(void* plan, size_t plan_bytes, const int32_t* block_tables,
                                int table_width, const int32_t* context_lens,
                                const int32_t* group_starts, const int32_t* prefix_lens,
                                int num_groups, int num_seqs, int num_q_heads, int num_kv_heads,
                                int block_size, int max_context_len, int max_prefix_len,
                                int partition_size, hipStream_t stream) {
  clear_error();
  if (!shape_ok(num_seqs, num_q_heads, num_kv_heads, 0, block_size, max_context_len, PKV_BF16))
    return PKV_ERR_INVALID;
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64) {
    set_error("block_size %d is not built (8, 16, 32 or 64)", block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_seqs > kMaxCompactSeqs) {
    set_error("shared-prefix plan: num_seqs %d above %d", num_seqs, kMaxCompactSeqs);
    return PKV_ERR_UNSUPPORTED;
  }
  if (table_width <= 0) { set_error("table_width must be positive"); return PKV_ERR_INVALID; }
  if (max_prefix_len < 0) { set_error("max_prefix_len %d < 0", max_prefix_len); return PKV_ERR_INVALID; }
  if (num_seqs == 0) return PKV_OK;
  if (num_groups < 1 || num_groups > num_seqs) {
    set_error("num_groups %d outside [1, num_seqs = %d]", num_groups, num_seqs);
    return PKV_ERR_INVALID;
  }
  if (!plan || !block_tables || !context_lens || !group_starts || !prefix_lens) {
    set_error("null pointer argument");
    return PKV_ERR_INVALID;
  }
  if (reinterpret_cast<uintptr_t>(plan) & 255u) {
    set_error("plan must be 256-byte aligned");
    return PKV_ERR_INVALID;
  }
  const int P = resolve_shared_partition(num_seqs, num_q_heads, num_kv_heads, block_size,
                                         num_groups, max_prefix_len, partition_size);
  if (P <= 0) {
    set_error("partition_size %d is not a positive multiple of %d", partition_size,
              partition_unit(block_size));
    return PKV_ERR_INVALID;
  }
  const int64_t items = shared_item_bound(num_seqs, num_q_heads, num_kv_heads, num_groups,
                                          max_context_len, max_prefix_len, P);
  if (items >= (int64_t{1} << 31)) {
    set_error("shared-prefix plan: too many work items");
    return PKV_ERR_UNSUPPORTED;
  }
  const int64_t need = shared_plan_bytes(num_seqs, items);
  if (plan_bytes < static_cast<size_t>(need)) {
    set_error("plan of %zu bytes is smaller than the %lld needed", plan_bytes,
              static_cast<long long>(need));
    return PKV_ERR_WORKSPACE;
  }
  const int resident = shared_resident_wgs();
  if (resident <= 0) {
    set_error("cannot query the current device");
    return PKV_ERR_HIP;
  }
  // about two items a wave
  const int64_t wgs = std::max<int64_t>(1, std::min<int64_t>(resident, cdiv64(items, 8)));
  AttnArgs a{};
  a.tables = block_tables;
  a.lens = context_lens;
  a.width = table_width;
  a.S = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.B = block_size;
  a.partition = P;
  a.max_len = max_context_len;
  a.group_starts = group_starts;
  a.prefix_lens = prefix_lens;
  a.num_groups = num_groups;
  a.max_prefix = max_prefix_len;
  a.stream_waves = static_cast<int>(wgs) * 4;
  int32_t* pl = static_cast<int32_t*>(plan);
  a.ws_seq = pl + kPlanHeaderInts;
  return launch_shared_plan(a, pl, items, stream);
}

}  // extern "C"

namespace {

int decode_shared_impl(int phases, void* out, pkv_dtype out_dtype, const void* query,
                       const void* kv_cache, const int32_t* block_tables, int table_width,
                       const int32_t* context_lens, const int32_t* group_starts,
                       const int32_t* prefix_lens, int num_groups, int num_seqs, int num_q_heads,
                       int num_kv_heads, int head_size, int block_size, int num_blocks,
                       float scale, int max_context_len, int max_prefix_len, int partition_size,
                       void* workspace, size_t workspace_bytes, pkv_dtype dtype, unsigned flags,
                       bool planned, const void* plan, size_t plan_bytes, hipStream_t stream) {
  clear_error();
  if (!shape_ok(num_seqs, num_q_heads, num_kv_heads, head_size, block_size, max_context_len, dtype))
    return PKV_ERR_INVALID;
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16) { set_error("unknown out_dtype"); return PKV_ERR_INVALID; }
  if (dtype != PKV_BF16) {
    set_error("shared-prefix decode: bf16 caches only");
    return PKV_ERR_UNSUPPORTED;
  }
  if (head_size != 64 && head_size != 128) {
    set_error("head_size %d is not built (64 or 128)", head_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64) {
    set_error("block_size %d is not built (8, 16, 32 or 64)", block_size);
    return PKV_ERR_UNSUPPORTED;
  }
  if (num_seqs > kMaxCompactSeqs) {
    set_error("shared-prefix decode: num_seqs %d above %d", num_seqs, kMaxCompactSeqs);
    return PKV_ERR_UNSUPPORTED;
  }
  if (table_width <= 0 || num_blocks <= 0) { set_error("table_width and num_blocks must be positive"); return PKV_ERR_INVALID; }
  if (!std::isfinite(scale)) { set_error("scale is not finite"); return PKV_ERR_INVALID; }
  if (flags & ~static_cast<unsigned>(PKV_ATTN_CACHED_KV)) {
    set_error("unknown flags 0x%x", flags);
    return PKV_ERR_INVALID;
  }
  if (max_prefix_len < 0) { set_error("max_prefix_len %d < 0", max_prefix_len); return PKV_ERR_INVALID; }
  if (num_seqs == 0) return PKV_OK;
  if (num_groups < 1 || num_groups > num_seqs) {
    set_error("num_groups %d outside [1, num_seqs = %d]", num_groups, num_seqs);
    return PKV_ERR_INVALID;
  }
  if (!out || !query || !kv_cache || !block_tables || !context_lens || !group_starts ||
      !prefix_lens) {
    set_error("null pointer argument");
    return PKV_ERR_INVALID;
  }
  if (!aligned16(out) || !aligned16(query) || !aligned16(kv_cache)) {
    set_error("out, query and kv_cache must be 16-byte aligned");
    return PKV_ERR_INVALID;
  }
  const int P = resolve_shared_partition(num_seqs, num_q_heads, num_kv_heads, block_size,
                                         num_groups, max_prefix_len, partition_size);
  if (P <= 0) {
    set_error("partition_size %d is not a positive multiple of %d", partition_size,
              partition_unit(block_size));
    return PKV_ERR_INVALID;
  }
  const SharedLayout lay =
      shared_layout(num_seqs, num_q_heads, head_size, max_context_len, max_prefix_len, P);
  if (!workspace || workspace_bytes < static_cast<size_t>(lay.bytes)) {
    set_error("workspace of %zu bytes is smaller than the %lld needed", workspace_bytes,
              static_cast<long long>(lay.bytes));
    return PKV_ERR_WORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) {
    set_error("workspace must be 256-byte aligned");
    return PKV_ERR_INVALID;
  }
  // work items (counted in 32-bit integers)
  const int HG = bf16_heads_per_group(num_kv_heads);
  const int64_t upper = shared_item_bound(num_seqs, num_q_heads, num_kv_heads, num_groups,
                                          max_context_len, max_prefix_len, P);
  if (upper >= (int64_t{1} << 31) || lay.parts * num_seqs * num_q_heads >= (int64_t{1} << 31)) {
    set_error("shared-prefix decode: too many work items or workspace rows");
    return PKV_ERR_UNSUPPORTED;
  }
  if (planned) {
    if (!plan) { set_error("null plan"); return PKV_ERR_INVALID; }
    if (reinterpret_cast<uintptr_t>(plan) & 255u) {
      set_error("plan must be 256-byte aligned");
      return PKV_ERR_INVALID;
    }
    const int64_t need = shared_plan_bytes(num_seqs, upper);
    if (plan_bytes < static_cast<size_t>(need)) {
      set_error("plan of %zu bytes is smaller than the %lld needed", plan_bytes,
                static_cast<long long>(need));
      return PKV_ERR_WORKSPACE;
    }
  }
  const int resident = shared_resident_wgs();
  if (resident <= 0) {
    set_error("cannot query the current device");
    return PKV_ERR_HIP;
  }
  const int nslot = 4 / HG;
  int64_t wgs = std::min<int64_t>(resident, cdiv64(upper, nslot));
  if (wgs >= 16) wgs = cdiv64(wgs, 16) * 16;  // whole blocks of 16 for the XCD pairing
  wgs = std::max<int64_t>(1, wgs);

  AttnArgs a{};
  a.out = out;
  a.query = query;
  a.kv = kv_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.width = table_width;
  a.S = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.D = head_size;
  a.B = block_size;
  a.NB = num_blocks;
  a.partition = P;
  a.max_parts = static_cast<int>(lay.parts);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = out_dtype == PKV_BF16 ? 1 : 0;
  a.nontemporal = (flags & PKV_ATTN_CACHED_KV) ? 0 : 1;
  a.k_via_lds = static_cast<int64_t>(num_kv_heads) * head_size * 2 >= 4096;
  a.max_len = max_context_len;
  a.group_starts = group_starts;
  a.prefix_lens = prefix_lens;
  a.num_groups = num_groups;
  a.max_prefix = max_prefix_len;
  a.stream_waves = static_cast<int>(wgs) * 4;
  shared_lds_plan(head_size, a.k_via_lds != 0, &a.stream_slots, &a.stream_wave_floats);
  char* ws = static_cast<char*>(workspace);
  a.ws_o = reinterpret_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(ws + lay.ml_off);
  a.ws_seq = reinterpret_cast<int*>(ws + lay.seq_off);
  if (planned) {
    a.plan = static_cast<const int32_t*>(plan);
    a.plan_capacity = upper;
  }
  if (phases & kAttend) {
    const int rc = launch_attention_bf16_shared(a, stream);
    if (rc != PKV_OK) return rc;
  }
  if (phases & kMerge) return launch_reduce_shared(a, stream);
  return PKV_OK;
}

}  // namespace

#define PKV_SHARED_ARGS                                                                          \
  out, out_dtype, query, kv_cache, block_tables, table_width, context_lens, group_starts,        \
      prefix_lens, num_groups, num_seqs, num_q_heads, num_kv_heads, head_size, block_size,       \
      num_blocks, scale, max_context_len, max_prefix_len, partition_size, workspace,             \
      workspace_bytes, dtype, flags

#define PKV_SHARED_PARAMS                                                                        \
  void *out, pkv_dtype out_dtype, const void *query, const void *kv_cache,                       \
      const int32_t *block_tables, int table_width, const int32_t *context_lens,                 \
      const int32_t *group_starts, const int32_t *prefix_lens, int num_groups, int num_seqs,     \
      int num_q_heads, int num_kv_heads, int head_size, int block_size, int num_blocks,          \
      float scale, int max_context_len, int max_prefix_len, int partition_size, void *workspace, \
      size_t workspace_bytes, pkv_dtype dtype, unsigned flags

extern "C" {

int paged_attention_decode_shared(PKV_SHARED_PARAMS, hipStream_t stream) {
  return decode_shared_impl(kAttend | kMerge, PKV_SHARED_ARGS, false, nullptr, 0, stream);
}

int paged_attention_shared_partitions(PKV_SHARED_PARAMS, hipStream_t stream) {
  return decode_shared_impl(kAttend, PKV_SHARED_ARGS, false, nullptr, 0, stream);
}

int paged_attention_shared_merge(PKV_SHARED_PARAMS, hipStream_t stream) {
  return decode_shared_impl(kMerge, PKV_SHARED_ARGS, false, nullptr, 0, stream);
}

int paged_attention_decode_shared_planned(PKV_SHARED_PARAMS, const void* plan, size_t plan_bytes,
                                          hipStream_t stream) {
  return decode_shared_impl(kAttend | kMerge, PKV_SHARED_ARGS, true, plan, plan_bytes, stream);
}

int paged_attention_shared_planned_partitions(PKV_SHARED_PARAMS, const void* plan,
                                              size_t plan_bytes, hipStream_t stream) {
  return decode_shared_impl(kAttend, PKV_SHARED_ARGS, true, plan, plan_bytes, stream);
}

int paged_attention_shared_planned_merge(PKV_SHARED_PARAMS, const void* plan, size_t plan_bytes,
                                         hipStream_t stream) {
  return decode_shared_impl(kMerge, PKV_SHARED_ARGS, true, plan, plan_bytes, stream);
}

}  // extern "C"
