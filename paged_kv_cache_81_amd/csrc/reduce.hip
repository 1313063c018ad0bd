// Log-sum-exp merge of context partitions.
//
// For each (sequence, query head) split into n > 1 partitions with statistics
// (m_p, l_p, o_p) -- m in log2 units, o normalised, stored in the workspace
// as rows [s][p][h] -- the output is
//     M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// One wave per (sequence, head); sequences held in one partition were written
// by the attention kernel directly and are skipped here.
#include "common.hpp"

#include <cmath>

namespace pkv {
namespace {

template <int D>
__global__ void __launch_bounds__(64) reduce_kernel(AttnArgs a) {
  constexpr int PER = D / 64;
  extern __shared__ float s_w[];
  const int sh = blockIdx.x;
  const int s = sh / a.Hq;
  const int lane = threadIdx.x;
  const int L = a.lens[s];
  const int P = a.partition;
  const int n = L > 0 ? (L + P - 1) / P : 1;
  const bool bad = L < 0 || (L + a.B - 1) / a.B > a.width || n > a.max_parts;
  const int64_t out_off = static_cast<int64_t>(sh) * D + lane * PER;
  if (!bad && n <= 1) return;

  float res[PER];
  if (bad) {
#pragma unroll
    for (int e = 0; e < PER; ++e) res[e] = NAN;
  } else {
    // workspace rows are [s][p][h]: partition p of (s, h) is row (s*P + p)*Hq + h
    const int h = sh - s * a.Hq;
    const int64_t pstride = a.Hq;  // rows between consecutive partitions
    const int64_t row0 = static_cast<int64_t>(s) * a.max_parts * a.Hq + h;
    const float* ml = a.ws_ml + 2 * row0;
    const float* o = a.ws_o + row0 * D + lane * PER;
    float M = -INFINITY;
    for (int p = lane; p < n; p += 64) M = fmaxf(M, ml[2 * pstride * p]);
    M = wave_max(M);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float den = 0.f;
    for (int p = lane; p < n; p += 64) {
      const float w = ml[2 * pstride * p + 1] * __builtin_amdgcn_exp2f(ml[2 * pstride * p] - Mu);
      s_w[p] = w;
      den += w;
    }
    den = wave_sum(den);
    __syncthreads();
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    int p = 0;
    for (; p + 4 <= n; p += 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float w = s_w[p + k];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, o[(p + k) * pstride * D + e], acc[e]);
      }
    }
    for (; p < n; ++p) {
      const float w = s_w[p];
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, o[p * pstride * D + e], acc[e]);
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int e = 0; e < PER; ++e) res[e] = acc[e] * inv;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[out_off + e] = f32_to_bf16(res[e]);
    else
      static_cast<float*>(a.out)[out_off + e] = res[e];
  }
}

}  // namespace

int launch_reduce(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0 || a.max_parts <= 1) return PKV_OK;
  const dim3 grid(static_cast<unsigned>(a.S) * a.Hq);
  const size_t lds = static_cast<size_t>(a.max_parts) * sizeof(float);
  if (a.D == 64) {
    reduce_kernel<64><<<grid, dim3(64), lds, stream>>>(a);
  } else if (a.D == 128) {
    reduce_kernel<128><<<grid, dim3(64), lds, stream>>>(a);
  } else {
    set_error("partition merge: head_size %d is not built", a.D);
    return PKV_ERR_UNSUPPORTED;
  }
  return check_launch("partition merge");
}

}  // namespace pkv
