// Log-sum-exp merge of context partitions.
//
// For each (sequence, query head) whose context was split into n > 1 parts
// with statistics (m_p, l_p, o_p) -- m in log2 units, o normalised -- the
// output is
//     M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p.
// One wave per (sequence, query head); heads whose context was read in one
// part were written by the attention kernel directly and are skipped here.
#include "common.hpp"

#include <cmath>

namespace pkv {
namespace {

constexpr int kWaves = 4;

// Merge the np parts of one (sequence, head): statistics (m, l) at
// ml[2 * stride * p] and ml[2 * stride * p + 1], normalised rows at
// o[stride * D * p]; the result goes to out at out_off.  Lane (g, d4) covers
// dims 4*d4 .. 4*d4+3 of parts p = g, g + NG, ...: the rows of the first 64
// parts are loaded in one round together with their statistics (lane p holds
// part p's), whose weights then reach the row lanes by shuffles; further
// parts follow eight loads at a time.  The NG row groups are combined across
// lanes.  A poisoned part (NaN statistics) poisons the row.
template <int D>
__device__ __forceinline__ void merge_parts(const AttnArgs& a, const float* ml, const float* o,
                                            int64_t stride, int np, int64_t out_off) {
  constexpr int G4 = D / 4;    // lanes per row
  constexpr int NG = 64 / G4;  // rows per load instruction
  constexpr int U = 64 / NG;   // first-round rows per lane: parts 0 .. 63
  const int lane = threadIdx.x & 63;
  const int g = lane / G4;
  const int d4 = lane - g * G4;
  const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);

  // rows past the last part repeat it (with weight 0), so that within the
  // rounds that hold a part every lane loads
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (NG * u < np) {
      const int p = min(g + NG * u, np - 1);
      v[u] = *reinterpret_cast<const float4*>(o + stride * D * p + 4 * d4);
    } else {
      v[u] = zero;
    }
  }
  float m0 = -INFINITY, l0 = 0.f;  // statistics of part `lane`
  if (lane < np) {
    m0 = ml[2 * stride * lane];
    l0 = ml[2 * stride * lane + 1];
  }
  // running (max, sum) of the lane's parts lane, lane + 64, ..., rescaled as
  // the max grows; then the lanes are combined
  float m_l = m0, d_l = l0;
  for (int p = lane + 64; p < np; p += 64) {
    const float m = ml[2 * stride * p];
    const float l = ml[2 * stride * p + 1];
    if (m > m_l) {
      d_l = d_l * __builtin_amdgcn_exp2f(m_l - m) + l;
      m_l = m;
    } else {
      d_l += l * __builtin_amdgcn_exp2f(m - m_l);
    }
  }
  const float M = wave_max(m_l);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  const float den = wave_sum(m_l == -INFINITY ? d_l : d_l * __builtin_amdgcn_exp2f(m_l - Mu));

  const float w_lane = lane < np ? l0 * __builtin_amdgcn_exp2f(m0 - Mu) : 0.f;
  float4 acc = zero;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float w = __shfl(w_lane, g + NG * u, 64);
    acc.x = fmaf(w, v[u].x, acc.x);
    acc.y = fmaf(w, v[u].y, acc.y);
    acc.z = fmaf(w, v[u].z, acc.z);
    acc.w = fmaf(w, v[u].w, acc.w);
  }
  constexpr int U2 = 8;
  for (int p0 = 64 + g; p0 < np; p0 += NG * U2) {
    float4 r[U2];
    float w[U2];
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      const int p = min(p0 + NG * u, np - 1);
      r[u] = *reinterpret_cast<const float4*>(o + stride * D * p + 4 * d4);
      w[u] = p0 + NG * u < np
                 ? ml[2 * stride * p + 1] * __builtin_amdgcn_exp2f(ml[2 * stride * p] - Mu)
                 : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      acc.x = fmaf(w[u], r[u].x, acc.x);
      acc.y = fmaf(w[u], r[u].y, acc.y);
      acc.z = fmaf(w[u], r[u].z, acc.z);
      acc.w = fmaf(w[u], r[u].w, acc.w);
    }
  }
#pragma unroll
  for (int m = G4; m < 64; m <<= 1) {
    acc.x += __shfl_xor(acc.x, m, 64);
    acc.y += __shfl_xor(acc.y, m, 64);
    acc.z += __shfl_xor(acc.z, m, 64);
    acc.w += __shfl_xor(acc.w, m, 64);
  }
  if (g == 0) {
    const float inv = 1.f / den;
    const float4 r = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    const int64_t off = out_off + 4 * d4;
    if (a.out_bf16) {
      const uint32_t lo = f32_to_bf16(r.x) | (static_cast<uint32_t>(f32_to_bf16(r.y)) << 16);
      const uint32_t hi = f32_to_bf16(r.z) | (static_cast<uint32_t>(f32_to_bf16(r.w)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = r;
    }
  }
}

// Fixed partitions: partition p of (s, h) is workspace row (s*P + p)*Hq + h.
template <int D>
__global__ void __launch_bounds__(64 * kWaves) reduce_kernel(AttnArgs a) {
  const int wv = threadIdx.x >> 6;
  const int64_t sh = static_cast<int64_t>(blockIdx.x) * kWaves + wv;
  if (sh >= static_cast<int64_t>(a.S) * a.Hq) return;
  const int s = static_cast<int>(sh / a.Hq);
  const int h = static_cast<int>(sh - static_cast<int64_t>(s) * a.Hq);
  const int lane = threadIdx.x & 63;
  const int L = a.lens[s];
  const int P = a.partition;
  const int n = L > 0 ? (L + P - 1) / P : 1;
  const bool bad = L < 0 || (L + a.B - 1) / a.B > a.width || n > a.max_parts;
  if (!bad && n <= 1) return;
  if (bad) {
    for (int d = lane; d < D; d += 64) {
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[sh * D + d] = f32_to_bf16(NAN);
      else
        static_cast<float*>(a.out)[sh * D + d] = NAN;
    }
    return;
  }
  const int64_t row0 = static_cast<int64_t>(s) * a.max_parts * a.Hq + h;
  merge_parts<D>(a, a.ws_ml + 2 * row0, a.ws_o + row0 * D, a.Hq, n, sh * D);
}

// Stream schedule: unit r = (sequence s, group of HG kv heads, query-head
// chunk) covers stream steps [g0, g0 + n).  The pieces holding its first and
// last steps are w0 and w1 (stream_wave_of).  If they are the same piece the
// unit was finished there; else each piece w0 .. w1 read a non-empty part of
// it and left a partial result in workspace slot w + r, rows [kv head in
// the group][query head].
template <int D>
__global__ void __launch_bounds__(64 * kWaves) reduce_stream_kernel(AttnArgs a) {
  const int wv = threadIdx.x >> 6;
  const int64_t sh = static_cast<int64_t>(blockIdx.x) * kWaves + wv;
  if (sh >= static_cast<int64_t>(a.S) * a.Hq) return;
  const int s = static_cast<int>(sh / a.Hq);
  const int h = static_cast<int>(sh - static_cast<int64_t>(s) * a.Hq);
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  const int HG = bf16_heads_per_group(a.Hkv);
  const int Y = (a.Hkv / HG) * chunks;
  const int nhs = min(16, G);
  const int kvh = h / G;
  const int jh = h - kvh * G;  // query head inside the kv head's group
  const int chunk = jh >> 4;
  const int hh = jh & 15;
  const int hg = kvh / HG;
  const int hi = kvh - hg * HG;
  const int y = hg * chunks + chunk;
  const int64_t r = static_cast<int64_t>(s) * Y + y;

  const int64_t T = a.ws_pref[a.S];
  const int64_t W = a.stream_waves / HG;  // pieces of the attention launch
  const int n = (a.ws_pref[s + 1] - a.ws_pref[s]) / Y;
  const int64_t g0 = a.ws_pref[s] + static_cast<int64_t>(y) * n;
  const int64_t w0 = stream_wave_of(g0, T, W);
  const int64_t w1 = stream_wave_of(g0 + n - 1, T, W);
  if (w0 == w1) return;
  const int64_t row0 = ((w0 + r) * HG + hi) * nhs + hh;
  merge_parts<D>(a, a.ws_ml + 2 * row0, a.ws_o + row0 * D, static_cast<int64_t>(HG) * nhs,
                 static_cast<int>(w1 - w0 + 1), sh * D);
}

// Shared-prefix schedule: sequence s has ws_seq[s] parts (-1: NaN output,
// 0: an empty context, zero output); part p of (s, h) is workspace row
// p*S*Hq + s*Hq + h, so each part of a sequence is Hq*D contiguous floats.
// ws_seq[3S + s] is set when s's own table entries for its group's prefix
// differ from those the prefix was read through: NaN.  Workgroup b takes
// sequence b / per (per = 256-piece runs of its Hq*D/4 float4 pieces) and
// thread t piece e = (b % per) * 256 + t, dims 4e .. 4e + 3 of its rows,
// parts in order: one piece a thread keeps each thread's chain of dependent
// loads short (the sequence's record, the parts' (m, l), their outputs), and
// every load instruction reads 4 KB of one part.  A part with NaN statistics
// poisons its row.
__global__ void __launch_bounds__(256) reduce_shared_kernel(AttnArgs a, int per) {
  const int s = blockIdx.x / per;
  const int e = (blockIdx.x - s * per) * 256 + threadIdx.x;
  const int64_t SH = static_cast<int64_t>(a.S) * a.Hq;
  const int np = a.ws_seq[s];
  const bool bad = np < 0 || a.ws_seq[3 * a.S + s] != 0;
  const int nvec = a.Hq * a.D / 4;
  const int64_t row0 = static_cast<int64_t>(s) * a.Hq;
  if (e < nvec) {
    const int h = 4 * e / a.D;
    const int64_t row = row0 + h;
    float4 r;
    if (bad || np <= 0) {
      const float v = bad ? NAN : 0.f;
      r = make_float4(v, v, v, v);
    } else {
      float M = -INFINITY;
      bool poison = false;
      for (int p = 0; p < np; ++p) {
        const float m = a.ws_ml[2 * (p * SH + row)];
        const float l = a.ws_ml[2 * (p * SH + row) + 1];
        poison = poison || m != m || l != l;
        M = fmaxf(M, m);
      }
      const float Mu = M == -INFINITY ? 0.f : M;
      float den = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int p = 0; p < np; ++p) {
        const float w = a.ws_ml[2 * (p * SH + row) + 1] *
                        __builtin_amdgcn_exp2f(a.ws_ml[2 * (p * SH + row)] - Mu);
        const float4 o = *reinterpret_cast<const float4*>(a.ws_o + (p * SH + row0) * a.D + 4 * e);
        den += w;
        acc.x = fmaf(w, o.x, acc.x);
        acc.y = fmaf(w, o.y, acc.y);
        acc.z = fmaf(w, o.z, acc.z);
        acc.w = fmaf(w, o.w, acc.w);
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
      r = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      if (poison) r = make_float4(NAN, NAN, NAN, NAN);
    }
    const int64_t off = row0 * a.D + 4 * static_cast<int64_t>(e);
    if (a.out_bf16) {
      const uint32_t lo = f32_to_bf16(r.x) | (static_cast<uint32_t>(f32_to_bf16(r.y)) << 16);
      const uint32_t hi = f32_to_bf16(r.z) | (static_cast<uint32_t>(f32_to_bf16(r.w)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = r;
    }
  }
}

}  // namespace

int launch_reduce_shared(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0) return PKV_OK;
  const int per = (a.Hq * a.D / 4 + 255) / 256;
  reduce_shared_kernel<<<dim3(static_cast<unsigned>(a.S) * per), dim3(256), 0, stream>>>(a, per);
  return check_launch("partition merge (shared prefix)");
}

int launch_reduce(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0 || (!a.stream && a.max_parts <= 1)) return PKV_OK;
  const int64_t waves = static_cast<int64_t>(a.S) * a.Hq;
  const dim3 grid(static_cast<unsigned>((waves + kWaves - 1) / kWaves));
  if (a.D != 64 && a.D != 128) {
    set_error("partition merge: head_size %d is not built", a.D);
    return PKV_ERR_UNSUPPORTED;
  }
  if (a.stream) {
    if (a.D == 64) reduce_stream_kernel<64><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
    else reduce_stream_kernel<128><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
  } else {
    if (a.D == 64) reduce_kernel<64><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
    else reduce_kernel<128><<<grid, dim3(64 * kWaves), 0, stream>>>(a);
  }
  return check_launch("partition merge");
}

}  // namespace pkv
