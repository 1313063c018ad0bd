// Streaming-read ceiling: how fast this GPU reads a buffer once, with nothing
// else to do.  The decode kernels' HBM rates are compared with it, at the
// same number of bytes per launch.  Not part of the decode path.
//
// Each thread reads 16-byte pieces in a grid-stride loop with `per` loads in
// flight (nontemporal, as the decode kernels stream K/V), XORs them together
// and writes one word per workgroup, so the loads cannot be dropped.
#include "common.hpp"

namespace pkv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ void __launch_bounds__(256) read_ceiling_kernel(const u32x4* __restrict__ p, size_t n16,
                                                           unsigned* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  acc ^= __shfl_xor(acc, 1, 64);  // keep the sum of the whole wave live
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int pkv_read_ceiling(const void* buf, size_t bytes, int grid, int loads_in_flight,
                                unsigned* sink, hipStream_t stream) {
  clear_error();
  if (!buf || !sink || grid <= 0 || grid > (1 << 20) || !aligned16(buf) || (bytes & 15u)) {
    set_error("read ceiling: bad arguments");
    return PKV_ERR_INVALID;
  }
  const u32x4* p = static_cast<const u32x4*>(buf);
  const size_t n16 = bytes / 16;
  switch (loads_in_flight) {
    case 1: read_ceiling_kernel<1><<<grid, 256, 0, stream>>>(p, n16, sink); break;
    case 2: read_ceiling_kernel<2><<<grid, 256, 0, stream>>>(p, n16, sink); break;
    case 4: read_ceiling_kernel<4><<<grid, 256, 0, stream>>>(p, n16, sink); break;
    case 8: read_ceiling_kernel<8><<<grid, 256, 0, stream>>>(p, n16, sink); break;
    default:
      set_error("read ceiling: loads_in_flight %d is not 1, 2, 4 or 8", loads_in_flight);
      return PKV_ERR_UNSUPPORTED;
  }
  return check_launch("read ceiling");
}
