// Slot mapping, the paged KV write (reshape-and-cache) and the gather through
// block tables.  All three are pure index/copy work: no arithmetic on the
// cached values, so results are bit-exact.
#include "common.hpp"

namespace pkv {
namespace {

// slot of (sequence, position): block_tables[s][p / B] * B + p % B, or -1.
__global__ void __launch_bounds__(256) slot_mapping_kernel(
    int64_t* __restrict__ out, const int32_t* __restrict__ tables, int width,
    const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions, int T, int S,
    int B, int NB) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T) return;
  const int s = seq_ids ? seq_ids[i] : i;
  const int p = positions[i];
  int64_t slot = -1;
  if (p >= 0 && s >= 0 && s < S) {
    const int lb = p / B;
    const int off = p - lb * B;
    if (lb < width) {
      const int phys = tables[static_cast<int64_t>(s) * width + lb];
      if (phys >= 0 && phys < NB) slot = static_cast<int64_t>(phys) * B + off;
    }
  }
  out[i] = slot;
}

// One token's K (or V) row for all kv heads is Hkv*D contiguous elements at
// row `slot` of the cache, so a token is `chunks` 16-byte pieces; one thread
// moves one piece of K and the same piece of V.
__global__ void __launch_bounds__(256) write_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ kv,
    const int64_t* __restrict__ slots, int64_t total, int chunks, int64_t num_slots) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t t = i / chunks;
  const int64_t c = i - t * chunks;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t dst = slot * chunks + c;
  const uint4 kk = key[i];
  const uint4 vv = value[i];
  kv[dst] = kk;
  kv[num_slots * chunks + dst] = vv;
}

// Slot derivation and write in one pass: thread (t, c) finds token t's slot
// from its table and position (positions[t] + pos_offset, as
// slot_mapping_kernel does) and moves piece c of its K and V; the thread with
// c == 0 also records the slot.  With the context lengths as positions and
// an offset of -1 it writes each sequence's last token.
__global__ void __launch_bounds__(256) write_positions_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, uint4* __restrict__ kv,
    const int32_t* __restrict__ tables, int width, const int32_t* __restrict__ seq_ids,
    const int32_t* __restrict__ positions, int pos_offset, int64_t* __restrict__ slots_out,
    int64_t total, int chunks, int S, int B, int NB) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t t = i / chunks;
  const int64_t c = i - t * chunks;
  const int s = seq_ids ? seq_ids[t] : static_cast<int>(t);
  const int p = positions[t] + pos_offset;
  int64_t slot = -1;
  if (p >= 0 && s >= 0 && s < S) {
    const int lb = p / B;
    if (lb < width) {
      const int phys = tables[static_cast<int64_t>(s) * width + lb];
      if (phys >= 0 && phys < NB) slot = static_cast<int64_t>(phys) * B + (p - lb * B);
    }
  }
  if (slots_out && c == 0) slots_out[t] = slot;
  if (slot < 0) return;
  const int64_t num_slots = static_cast<int64_t>(NB) * B;
  const int64_t dst = slot * chunks + c;
  const uint4 kk = key[i];
  const uint4 vv = value[i];
  kv[dst] = kk;
  kv[num_slots * chunks + dst] = vv;
}

__global__ void __launch_bounds__(256) gather_kernel(
    uint4* __restrict__ k_out, uint4* __restrict__ v_out, const uint4* __restrict__ kv,
    const int32_t* __restrict__ tables, int width, const int32_t* __restrict__ lens, int B,
    int NB, int max_len, int chunks, uint32_t nan_word) {
  const int s = blockIdx.y;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per_seq = static_cast<int64_t>(max_len) * chunks;
  if (i >= per_seq) return;
  const int t = static_cast<int>(i / chunks);
  const int c = static_cast<int>(i - static_cast<int64_t>(t) * chunks);
  const int L = lens[s];
  bool bad = L < 0 || L > max_len || (L + B - 1) / B > width;
  uint4 kk = make_uint4(0, 0, 0, 0);
  uint4 vv = kk;
  if (!bad && t < L) {
    const int phys = tables[static_cast<int64_t>(s) * width + t / B];
    if (phys < 0 || phys >= NB) {
      bad = true;
    } else {
      const int64_t src = (static_cast<int64_t>(phys) * B + t % B) * chunks + c;
      kk = kv[src];
      vv = kv[static_cast<int64_t>(NB) * B * chunks + src];
    }
  }
  if (bad) kk = vv = make_uint4(nan_word, nan_word, nan_word, nan_word);
  const int64_t o = static_cast<int64_t>(s) * per_seq + i;
  k_out[o] = kk;
  v_out[o] = vv;
}

}  // namespace

int launch_slot_mapping(int64_t* slot_mapping, const int32_t* tables, int width,
                        const int32_t* seq_ids, const int32_t* positions, int T, int S, int B,
                        int NB, hipStream_t stream) {
  if (T == 0) return PKV_OK;
  slot_mapping_kernel<<<dim3((T + 255) / 256), dim3(256), 0, stream>>>(
      slot_mapping, tables, width, seq_ids, positions, T, S, B, NB);
  return check_launch("slot mapping");
}

int launch_write(const void* key, const void* value, void* kv, const int64_t* slots, int T, int NB,
                 int B, int Hkv, int D, int elem_bytes, hipStream_t stream) {
  if (T == 0) return PKV_OK;
  const int chunks = Hkv * D * elem_bytes / 16;
  const int64_t total = static_cast<int64_t>(T) * chunks;
  write_kernel<<<dim3(static_cast<unsigned>(cdiv64(total, 256))), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(key), static_cast<const uint4*>(value), static_cast<uint4*>(kv),
      slots, total, chunks, static_cast<int64_t>(NB) * B);
  return check_launch("kv write");
}

int launch_write_positions(const void* key, const void* value, void* kv, const int32_t* tables,
                           int width, const int32_t* seq_ids, const int32_t* positions,
                           int pos_offset, int64_t* slots_out, int T, int S, int NB, int B,
                           int Hkv, int D, int elem_bytes, hipStream_t stream) {
  if (T == 0) return PKV_OK;
  const int chunks = Hkv * D * elem_bytes / 16;
  const int64_t total = static_cast<int64_t>(T) * chunks;
  write_positions_kernel<<<dim3(static_cast<unsigned>(cdiv64(total, 256))), dim3(256), 0, stream>>>(
      static_cast<const uint4*>(key), static_cast<const uint4*>(value), static_cast<uint4*>(kv),
      tables, width, seq_ids, positions, pos_offset, slots_out, total, chunks, S, B, NB);
  return check_launch("kv write (positions)");
}

int launch_gather(void* k_out, void* v_out, const void* kv, const int32_t* tables, int width,
                  const int32_t* lens, int S, int Hkv, int D, int B, int NB, int max_len,
                  int elem_bytes, hipStream_t stream) {
  if (S == 0 || max_len == 0) return PKV_OK;
  const int chunks = Hkv * D * elem_bytes / 16;
  const int64_t per_seq = static_cast<int64_t>(max_len) * chunks;
  const uint32_t nan_word = elem_bytes == 4 ? 0x7FC00000u : 0x7FC07FC0u;
  gather_kernel<<<dim3(static_cast<unsigned>(cdiv64(per_seq, 256)), S), dim3(256), 0, stream>>>(
      static_cast<uint4*>(k_out), static_cast<uint4*>(v_out), static_cast<const uint4*>(kv),
      tables, width, lens, B, NB, max_len, chunks, nan_word);
  return check_launch("kv gather");
}

}  // namespace pkv
