// Paged decode attention for bf16 caches on gfx950 matrix cores.
//
// Work item: one workgroup (4 waves) per (partition of P tokens, kv head,
// group of <= 16 query heads, sequence).  The query heads that share a kv head
// are handled together, so every K/V block is read once per kv head.
//
// A wave step covers 32 tokens as two 16-token tiles.  Lane l is (j, g) with
// j = l % 16 and g = l / 16.
//
//  * Scores, S[token][head] = K . Q^T, use v_mfma_f32_16x16x32_bf16 with the
//    K tile as the A operand (row j = token, 8 dims per lane) and the query
//    heads as the B operand (column j = head).  The accumulator gives lane
//    (j, g) the scores of head j for tokens 4g..4g+3 of the tile.
//  * Softmax runs online, per head, in the log2 domain: one cross-lane max per
//    step (xor 16, xor 32), everything else lane-local.
//  * Values are contracted as O^T = V^T . P^T so that head j stays in column
//    j: the P operand (B) is exactly the weights lane (j, g) already holds, for
//    its 8 tokens {4g..4g+3} of each tile.  Output dims are permuted: row i of
//    output block n is dim NV*i + n (NV = D/16), so lane (j, g) needs dims
//    NV*j .. NV*j+NV-1 of each of its 8 tokens -- a contiguous piece of every V
//    row (16 lanes cover a full row: fully coalesced loads) -- followed by an
//    8 x NV transpose of bf16 pairs in registers (v_perm_b32).
//  * P is split into bf16 hi + lo parts, so P.V keeps ~16 mantissa bits of
//    the fp32 weights; accumulation is fp32.
//  * The 4 waves' (m, l, O) are merged through LDS; the workgroup writes the
//    normalised output (single partition) or its partition statistics.
#include "common.hpp"

#include <cmath>

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStep = 32;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int NW>
struct Words {
  uint32_t w[NW];
};

template <int NW>
__device__ __forceinline__ Words<NW> load_words(const uint16_t* p) {
  Words<NW> r;
  if constexpr (NW == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else {
    static_assert(NW == 2, "unsupported");
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    r.w[0] = v.x; r.w[1] = v.y;
  }
  return r;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int B>
__global__ void __launch_bounds__(kThreads) attention_bf16_kernel(AttnArgs a) {
  constexpr int QC = D / 32;  // score MFMAs per tile (32 dims each)
  constexpr int NV = D / 16;  // output blocks of 16 rows; dims per lane per V token
  constexpr int NW = NV / 2;  // 32-bit words per lane per V token
  constexpr int LDS_ROW = D + 4;

  __shared__ float s_o[kWaves][16][LDS_ROW];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ int s_bad;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g = lane >> 4;

  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  const int part = blockIdx.x;
  const int kvh = blockIdx.y / chunks;
  const int chunk = blockIdx.y - kvh * chunks;
  const int s = blockIdx.z;

  const int L = a.lens[s];
  const int P = a.partition;
  const int nparts = L > 0 ? (L + P - 1) / P : 1;
  const bool bad_seq = L < 0 || (L + B - 1) / B > a.width || nparts > a.max_parts;
  if (part > 0 && (bad_seq || part >= nparts)) return;

  const int nh = min(16, G - chunk * 16);
  const int h0 = kvh * G + chunk * 16;

  if (threadIdx.x == 0) s_bad = bad_seq ? 1 : 0;

  // query fragments: q[s][h0 + j][32c + 8g .. +8]
  bf16x8 qf[QC];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.query) +
                         (static_cast<int64_t>(s) * a.Hq + h0 + j) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < QC; ++c)
      qf[c] = (j < nh) ? load_bf16x8(qp + 32 * c) : bf16x8{};
  }

  const int t_begin = part * P;
  const int t_end = bad_seq ? t_begin : min(L, t_begin + P);
  const int nsteps = (t_end - t_begin + kStep - 1) / kStep;

  const int64_t row = static_cast<int64_t>(a.Hkv) * D;  // elements between slots
  const uint16_t* kbase = static_cast<const uint16_t*>(a.kv) + static_cast<int64_t>(kvh) * D;
  const uint16_t* vbase = kbase + static_cast<int64_t>(a.NB) * B * row;
  const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.width;
  const int koff = j * static_cast<int>(row) + 8 * g;
  int voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) voff[r] = (4 * g + r) * static_cast<int>(row) + NV * j;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad_blk = false;

  for (int st = wave; st < nsteps; st += kWaves) {
    const int ts = t_begin + st * kStep;

    // block of each 16-token tile (uniform across the wave)
    int64_t tile_base[2];
    bool tile_ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tt = ts + 16 * u;
      tile_ok[u] = tt < t_end;
      tile_base[u] = 0;
      if (tile_ok[u]) {
        const int phys = trow[tt / B];
        if (phys < 0 || phys >= a.NB) {
          bad_blk = true;
          tile_ok[u] = false;
        } else {
          tile_base[u] = (static_cast<int64_t>(phys) * B + (tt % B)) * row;
        }
      }
    }

    // K tiles (A operand): token j of the tile, dims 32c + 8g .. +8
    bf16x8 kf[2][QC];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int c = 0; c < QC; ++c)
        kf[u][c] = tile_ok[u] ? load_bf16x8(kbase + tile_base[u] + koff + 32 * c) : bf16x8{};

    // V pieces: token 4g + r of tile u, dims NV*j .. NV*j + NV - 1; zero past the end
    Words<NW> vr[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = tile_ok[u] && (ts + 16 * u + 4 * g + r < t_end);
        if (ok) {
          vr[u][r] = load_words<NW>(vbase + tile_base[u] + voff[r]);
        } else {
#pragma unroll
          for (int w = 0; w < NW; ++w) vr[u][r].w[w] = 0u;
        }
      }

    // scores
    float x[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < QC; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u][c], qf[c], sc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = tile_ok[u] && (ts + 16 * u + 4 * g + r < t_end);
        x[u][r] = ok ? sc[r] * a.scale_log2 : -INFINITY;
      }
    }

    // online softmax (log2 domain), per head j
    float mx = x[0][0];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[u][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;

    bf16x8 phi, plo;
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = fast_exp2(x[u][r] - m_use);
        psum += pv;
        const __bf16 hb = static_cast<__bf16>(pv);
        phi[4 * u + r] = hb;
        plo[4 * u + r] = static_cast<__bf16>(pv - static_cast<float>(hb));
      }
    l_run = l_run * alpha + psum;

    // V^T operand for output block n: the 8 tokens' value of dim NV*j + n
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
      u32x4 va;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e0 = 2 * q, e1 = 2 * q + 1;  // token slots (u = e/4, r = e%4)
        va[q] = __builtin_amdgcn_perm(vr[e1 >> 2][e1 & 3].w[n >> 1], vr[e0 >> 2][e0 & 3].w[n >> 1], sel);
      }
      const bf16x8 vb = __builtin_bit_cast(bf16x8, va);
      f32x4 o = acc[n] * alpha;
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, phi, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, plo, o, 0, 0, 0);
      acc[n] = o;
    }
  }

  // per-head sum over the four lane groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  __syncthreads();  // s_bad initialised
  if (bad_blk) s_bad = 1;
  if (g == 0) {
    s_m[wave][j] = m_run;
    s_l[wave][j] = l_run;
  }
  // lane (j, g) holds head j, dims NV*(4g + r) + n
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int n = 0; n < NV; ++n) s_o[wave][j][NV * (4 * g + r) + n] = acc[n][r];
  __syncthreads();

  const bool bad = s_bad != 0;
  // without a workspace (one partition per sequence) results always go to out
  const bool single = nparts == 1 || a.max_parts == 1;
  constexpr int D4 = D / 4;
  for (int idx = threadIdx.x; idx < nh * D4; idx += kThreads) {
    const int hh = idx / D4;
    const int d = (idx - hh * D4) * 4;
    float M = s_m[0][hh];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][hh]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float lsum = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(s_m[w][hh] - Mu);
      lsum += sc * s_l[w][hh];
      o.x += sc * s_o[w][hh][d + 0];
      o.y += sc * s_o[w][hh][d + 1];
      o.z += sc * s_o[w][hh][d + 2];
      o.w += sc * s_o[w][hh][d + 3];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    o.x *= inv; o.y *= inv; o.z *= inv; o.w *= inv;
    if (bad) {
      o = make_float4(NAN, NAN, NAN, NAN);
      M = NAN;
      lsum = NAN;
    }
    const int h = h0 + hh;
    if (single) {
      const int64_t off = (static_cast<int64_t>(s) * a.Hq + h) * D + d;
      if (a.out_bf16) {
        uint16_t* op = static_cast<uint16_t*>(a.out) + off;
        const uint32_t lo = f32_to_bf16(o.x) | (static_cast<uint32_t>(f32_to_bf16(o.y)) << 16);
        const uint32_t hi = f32_to_bf16(o.z) | (static_cast<uint32_t>(f32_to_bf16(o.w)) << 16);
        *reinterpret_cast<u32x2*>(op) = u32x2{lo, hi};
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = o;
      }
    } else {
      const int64_t sp = (static_cast<int64_t>(s) * a.Hq + h) * a.max_parts + part;
      *reinterpret_cast<float4*>(a.ws_o + sp * D + d) = o;
      if (d == 0) {
        a.ws_ml[2 * sp] = M;
        a.ws_ml[2 * sp + 1] = lsum;
      }
    }
  }
}

template <int D, int B>
int launch(const AttnArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) / 16;
  dim3 grid(a.max_parts, a.Hkv * chunks, a.S);
  attention_bf16_kernel<D, B><<<grid, dim3(kThreads), 0, stream>>>(a);
  return check_launch("paged attention (bf16)");
}

}  // namespace

int launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0) return PKV_OK;
  switch (a.D * 1000 + a.B) {
    case 64016: return launch<64, 16>(a, stream);
    case 64032: return launch<64, 32>(a, stream);
    case 64064: return launch<64, 64>(a, stream);
    case 128016: return launch<128, 16>(a, stream);
    case 128032: return launch<128, 32>(a, stream);
    case 128064: return launch<128, 64>(a, stream);
    default:
      set_error("paged attention (bf16): head_size %d with block_size %d is not built", a.D, a.B);
      return PKV_ERR_UNSUPPORTED;
  }
}

}  // namespace pkv
