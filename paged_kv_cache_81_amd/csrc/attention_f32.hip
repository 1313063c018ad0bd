// Paged decode attention for fp32 caches (vector ALU path).
//
// One wave per (partition of <= 512 tokens, kv head, group of <= 16 query
// heads, sequence).  Phase 1: lane t scores token t of the partition against
// every query head of the group (q rows staged in LDS).  Phase 2: per-head max
// and exponentials in the log2 domain.  Phase 3: lanes own dims, walk the
// partition's tokens and accumulate the weighted values of all heads, so each
// V row is read once.  fp32 throughout.
#include "common.hpp"

#include <cmath>

namespace pkv {
namespace {

constexpr int kMaxPart = 512;
constexpr int kMaxHeads = 16;

// NH: query heads one wave serves (the group's heads, rounded up to a power
// of two; the padding rows of q are zero), fixed at compile time so that no
// per-head branch separates the loads from the arithmetic.
template <int D, int NH>
__global__ void __launch_bounds__(64) attention_f32_kernel(AttnArgs a) {
  constexpr int PER = D / 64;  // output dims per lane
  __shared__ float s_q[NH][D];
  __shared__ float s_p[NH][kMaxPart];
  // element offset of each token's row in the K (and V) half of the pool, -1
  // for a token on a block outside the pool: phase 3 then addresses a value
  // row with one add, and its loads go out back to back
  __shared__ int64_t s_off[kMaxPart];

  const int lane = threadIdx.x;
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + kMaxHeads - 1) / kMaxHeads;
  const int part = blockIdx.x;
  const int kvh = blockIdx.y / chunks;
  const int chunk = blockIdx.y - kvh * chunks;
  const int s = blockIdx.z;
  const int B = a.B;

  const int P = a.partition;
  const int t_begin = part * P;
  const int nh = min(NH, G - chunk * kMaxHeads);
  const int h0 = kvh * G + chunk * kMaxHeads;
  const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.width;
  // The length, the table entry of the lane's first token and the query rows
  // in one round of loads, so the key loads wait for one round trip, not
  // two: the entry is read before the length is known (any entry below the
  // table's width is the table's memory) and dropped if past it.
  const int L = a.lens[s];
  const int tb = (t_begin + lane) / B;
  const int phys_spec = lane < P && tb < a.width ? trow[tb] : 0;
  const float* q = static_cast<const float*>(a.query);
  for (int i = lane; i < NH * D; i += 64)
    s_q[i / D][i % D] = i < nh * D ? q[(static_cast<int64_t>(s) * a.Hq + h0) * D + i] : 0.f;
  // the kv head's row of the sequence's new key and value (if given), in the
  // same round: lane l < D/4 holds dims 4l .. 4l + 3
  float4 k_new = make_float4(0.f, 0.f, 0.f, 0.f), v_new = k_new;
  if (a.k_new != nullptr && lane < D / 4) {
    const int64_t nrow = (static_cast<int64_t>(s) * a.Hkv + kvh) * D + 4 * lane;
    k_new = *reinterpret_cast<const float4*>(static_cast<const float*>(a.k_new) + nrow);
    v_new = *reinterpret_cast<const float4*>(static_cast<const float*>(a.v_new) + nrow);
  }

  const int nparts = L > 0 ? (L + P - 1) / P : 1;
  const bool bad_seq = L < 0 || (L + B - 1) / B > a.width || nparts > a.max_parts;
  if (part > 0 && (bad_seq || part >= nparts)) return;
  const int t_end = bad_seq ? t_begin : min(L, t_begin + P);
  const int n = max(0, t_end - t_begin);
  const int64_t row = static_cast<int64_t>(a.Hkv) * D;
  const float* kbase = static_cast<const float*>(a.kv) + static_cast<int64_t>(kvh) * D;
  const float* vbase = kbase + static_cast<int64_t>(a.NB) * B * row;
  bool bad = bad_seq;
  const int phys_first = lane < n ? phys_spec : 0;

  // With new tokens given, token L - 1 of the sequence is stored into the
  // cache by every work item that reads it (each query-head chunk of the kv
  // head stores the same bytes; an invalid sequence's token is stored by its
  // partition 0, as the write kernel would), before the loads below read it
  // back: a wavefront's own stores precede its later loads of the same
  // address, and the release/acquire pair keeps the compiler from moving
  // those loads above the stores.  The slot rule and its -1 cases are the
  // write kernel's.  The token's block comes from the entries loaded above
  // when it lies among the partition's first 64 tokens.
  if (a.k_new != nullptr && L > 0 && part == (bad_seq ? 0 : nparts - 1)) {
    const int tl = L - 1;
    if (tl / B < a.width) {
      const int k = tl - t_begin;
      const int phys = k >= 0 && k < 64 && k < P ? __shfl(phys_spec, k, 64) : trow[tl / B];
      if (phys >= 0 && phys < a.NB && lane < D / 4) {
        float* kd = const_cast<float*>(kbase) + (static_cast<int64_t>(phys) * B + tl % B) * row +
                    4 * lane;
        *reinterpret_cast<float4*>(kd) = k_new;
        *reinterpret_cast<float4*>(kd + static_cast<int64_t>(a.NB) * B * row) = v_new;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();

  // phase 1: scores
  for (int i = lane; i < n; i += 64) {
    const int t = t_begin + i;
    const int phys = i == lane ? phys_first : trow[t / B];
    const bool in_pool = phys >= 0 && phys < a.NB;
    const int64_t off = (static_cast<int64_t>(phys) * B + t % B) * row;
    s_off[i] = in_pool ? off : -1;
    float dot[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) dot[h] = 0.f;
    if (!in_pool) {
      bad = true;
    } else {
      const float4* kr = reinterpret_cast<const float4*>(kbase + off);
      for (int c = 0; c < D / 4; ++c) {
        const float4 kk = kr[c];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          dot[h] = fmaf(kk.x, s_q[h][4 * c + 0], dot[h]);
          dot[h] = fmaf(kk.y, s_q[h][4 * c + 1], dot[h]);
          dot[h] = fmaf(kk.z, s_q[h][4 * c + 2], dot[h]);
          dot[h] = fmaf(kk.w, s_q[h][4 * c + 3], dot[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) s_p[h][i] = dot[h] * a.scale_log2;
  }
  __syncthreads();

  // 64 tokens per batch of value loads when one head's accumulators are all
  // a lane holds, 32 for a few heads, 16 when many heads' accumulators fill
  // the registers.  Every load of a batch is issued (a token past the end, or
  // on a block outside the pool -- flagged in phase 1 -- reads the pool's
  // first row and its value is then zeroed), so no branch separates them;
  // the first batch is issued before phase 2, whose arithmetic then covers
  // its latency.
  constexpr int kBatch = NH * PER == 1 ? 64 : (NH * PER >= 16 ? 16 : 32);
  float v[kBatch][PER];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int i = i0 + k;
      const int64_t off = i < n ? s_off[i] : -1;
      const bool ok = off >= 0;
      const float* vr = vbase + (ok ? off : 0) + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) v[k][e] = vr[e];
#pragma unroll
      for (int e = 0; e < PER; ++e) v[k][e] = ok ? v[k][e] : 0.f;
    }
  };
  load_batch(0);  // unconditional: a branch here would make the compiler wait for it at once

  // phase 2: per-head max and exponentials (log2 domain)
  float m[NH], l[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) mx = fmaxf(mx, s_p[h][i]);
    mx = wave_max(mx);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    float sum = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float p = __builtin_amdgcn_exp2f(s_p[h][i] - mu);
      s_p[h][i] = p;
      sum += p;
    }
    m[h] = mx;
    l[h] = wave_sum(sum);
  }
  __syncthreads();

  // phase 3: weighted values; lane owns dims lane*PER .. +PER
  float acc[NH][PER];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[h][e] = 0.f;
  for (int i0 = 0; i0 < n; i0 += kBatch) {
    if (i0 > 0) load_batch(i0);
    // tokens past the end have zero values (and weights never read past n)
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const float p = i0 + k < n ? s_p[h][i0 + k] : 0.f;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[h][e] = fmaf(p, v[k][e], acc[h][e]);
      }
    }
  }

  // any lane that saw a bad block poisons the whole work item
  bad = __any(bad);
  // without a workspace (one partition per sequence) results always go to out
  const bool single = nparts == 1 || a.max_parts == 1;
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    if (h >= nh) continue;
    const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
    const int hq = h0 + h;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float o = bad ? NAN : acc[h][e] * inv;
      const int d = lane * PER + e;
      if (single) {
        const int64_t off = (static_cast<int64_t>(s) * a.Hq + hq) * D + d;
        if (a.out_bf16)
          static_cast<uint16_t*>(a.out)[off] = f32_to_bf16(o);
        else
          static_cast<float*>(a.out)[off] = o;
      } else {
        const int64_t sp = (static_cast<int64_t>(s) * a.max_parts + part) * a.Hq + hq;
        a.ws_o[sp * D + d] = o;
        if (d == 0) {
          a.ws_ml[2 * sp] = bad ? NAN : m[h];
          a.ws_ml[2 * sp + 1] = bad ? NAN : l[h];
        }
      }
    }
  }
}

}  // namespace

int launch_attention_f32(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0) return PKV_OK;
  if (a.partition > kMaxPart) {
    set_error("paged attention (fp32): partition of %d tokens exceeds %d", a.partition, kMaxPart);
    return PKV_ERR_UNSUPPORTED;
  }
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + kMaxHeads - 1) / kMaxHeads;
  dim3 grid(a.max_parts, a.Hkv * chunks, a.S);
  if (a.D != 64 && a.D != 128) {
    set_error("paged attention (fp32): head_size %d is not built", a.D);
    return PKV_ERR_UNSUPPORTED;
  }
  const int nh = G < kMaxHeads ? G : kMaxHeads;
  const int NH = nh <= 1 ? 1 : nh <= 2 ? 2 : nh <= 4 ? 4 : nh <= 8 ? 8 : 16;
  auto go = [&](auto kern) { kern<<<grid, dim3(64), 0, stream>>>(a); };
  if (a.D == 64) {
    switch (NH) {
      case 1: go(attention_f32_kernel<64, 1>); break;
      case 2: go(attention_f32_kernel<64, 2>); break;
      case 4: go(attention_f32_kernel<64, 4>); break;
      case 8: go(attention_f32_kernel<64, 8>); break;
      default: go(attention_f32_kernel<64, 16>); break;
    }
  } else {
    switch (NH) {
      case 1: go(attention_f32_kernel<128, 1>); break;
      case 2: go(attention_f32_kernel<128, 2>); break;
      case 4: go(attention_f32_kernel<128, 4>); break;
      case 8: go(attention_f32_kernel<128, 8>); break;
      default: go(attention_f32_kernel<128, 16>); break;
    }
  }
  return check_launch("paged attention (fp32)");
}

}  // namespace pkv
