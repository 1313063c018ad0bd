// Whole-block copies between two pools of the same geometry: the
// copy-on-write copy of a shared block before a forked sample writes into it
// (studying-code.tistory.com vLLM review, "생성 단계에서의 Copy-on-Write"),
// and the swap of blocks between device memory and pinned host memory.
//
// A block is two contiguous halves (keys, values), each block_size * Hkv * D
// elements.  Workgroup (i, y) copies chunk y/2 of half y%2 of pair i with
// 16-byte loads and stores, four in flight per thread.  Bandwidth-bound:
// 2 * half bytes read and written per pair.
#include "common.hpp"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kChunkVecs = kThreads * kUnroll;  // 16-byte vectors per workgroup

__global__ void __launch_bounds__(kThreads)
copy_blocks_kernel(uint4* dst, int dst_nb, const uint4* src, int src_nb, const int32_t* src_ids,
                   const int32_t* dst_ids, int64_t half_vecs) {
  const int i = blockIdx.x;
  const int kv = blockIdx.y & 1;
  const int64_t chunk = blockIdx.y >> 1;
  const int s = src_ids[i];
  const int d = dst_ids[i];
  if (s < 0 || s >= src_nb || d < 0 || d >= dst_nb) return;
  const uint4* from = src + (static_cast<int64_t>(kv) * src_nb + s) * half_vecs;
  uint4* to = dst + (static_cast<int64_t>(kv) * dst_nb + d) * half_vecs;
  const int64_t begin = chunk * kChunkVecs + threadIdx.x;
  static_assert(kUnroll == 4, "the whole-chunk path names its four registers");
  if ((chunk + 1) * kChunkVecs <= half_vecs) {
    // a whole chunk: all loads in flight before the first store
    const uint4 v0 = from[begin], v1 = from[begin + kThreads];
    const uint4 v2 = from[begin + 2 * kThreads], v3 = from[begin + 3 * kThreads];
    to[begin] = v0;
    to[begin + kThreads] = v1;
    to[begin + 2 * kThreads] = v2;
    to[begin + 3 * kThreads] = v3;
  } else {
    // the ragged end of a half
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t e = begin + u * kThreads;
      if (e < half_vecs) to[e] = from[e];
    }
  }
}

}  // namespace

int launch_copy_blocks(void* dst, int dst_nb, const void* src, int src_nb, const int32_t* src_ids,
                       const int32_t* dst_ids, int n, int64_t half_bytes, hipStream_t stream) {
  if (n == 0) return PKV_OK;
  const int64_t half_vecs = half_bytes / 16;
  const int64_t chunks = (half_vecs + kChunkVecs - 1) / kChunkVecs;
  if (2 * chunks > 65535) {
    set_error("copy blocks: blocks of %lld bytes are too large", static_cast<long long>(half_bytes));
    return PKV_ERR_UNSUPPORTED;
  }
  copy_blocks_kernel<<<dim3(n, static_cast<unsigned>(2 * chunks)), dim3(kThreads), 0, stream>>>(
      static_cast<uint4*>(dst), dst_nb, static_cast<const uint4*>(src), src_nb, src_ids, dst_ids,
      half_vecs);
  return check_launch("copy blocks");
}

}  // namespace pkv
