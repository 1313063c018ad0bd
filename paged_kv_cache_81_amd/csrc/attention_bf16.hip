// Paged decode attention for bf16 caches on gfx950 matrix cores.
//
// Work item: one workgroup of 4 waves per (run of partitions of P tokens,
// group of HG consecutive kv heads, group of <= 16 query heads per kv head,
// sequence).  Wave w works on kv head (w % HG) of the group and on its own
// contiguous run of partitions (4/HG runs per workgroup), finishing each
// partition's softmax statistics as it crosses into the next.  All query heads sharing a kv head are handled by its
// wave, so every K/V block is read once per kv head; the HG waves of a group
// walk the same tokens together, so each cached row is read as HG*D*2
// contiguous bytes (>= 1 KB for HG = 4, D = 128) rather than one head's piece.
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
//  * Block-table entries are loaded once per wave (one per lane) and read back
//    as scalars; each wave keeps two steps of K/V in registers, so the next
//    step's loads are in flight while the current one computes.
//  * Each wave writes its results from registers: the normalised output when
//    the sequence is one partition, else per partition the statistics
//    (max score, exponent sum, normalised partial output) for the merge kernel.
#include "common.hpp"

#include <algorithm>
#include <cmath>
#include <mutex>

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

// Cached K/V is streamed once per kv head: read it with nontemporal loads,
// which keep it from displacing other lines in L2 and the memory-side cache
// and sustain a higher HBM read rate than ordinary loads.
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int NW, bool NT>
__device__ __forceinline__ Words<NW> load_words(const uint16_t* p) {
  Words<NW> r;
  if constexpr (NW == 4) {
    const u32x4 v = ld<NT>(reinterpret_cast<const u32x4*>(p));
    r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  } else {
    static_assert(NW == 2, "unsupported");
    const u32x2 v = ld<NT>(reinterpret_cast<const u32x2*>(p));
    r.w[0] = v.x; r.w[1] = v.y;
  }
  return r;
}

template <bool NT>
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, ld<NT>(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D, int B, int HG, bool NT, bool KL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
attention_bf16_kernel(AttnArgs a) {
  constexpr int QC = D / 32;  // score MFMAs per tile (32 dims each)
  constexpr int NV = D / 16;  // output blocks of 16 rows; dims per lane per V token
  constexpr int NW = NV / 2;  // 32-bit words per lane per V token
  constexpr int NSLOT = kWaves / HG;  // waves per kv head, each on its own partitions
  constexpr int NCH = D / 8;          // 16-byte chunks per K row
  auto kskew = [](int t) { return (t * NCH / 16) % NCH; };

  // Finished partitions stay in LDS until the wave has read its last K/V:
  // a global store issued between the loads would make the following waits
  // for those loads also wait for the store to be acknowledged.  Per wave:
  // pps partitions x nhs heads of SROW floats, then their (m, l) pairs.
  constexpr int SROW = D + 4;  // padded head row (floats)
  extern __shared__ float s_dyn[];

  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = wv % HG;    // kv head inside the group
  const int slot = wv / HG;  // which run of partitions

  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  const int Y = (a.Hkv / HG) * chunks;  // (kv-head group, query-head chunk) pairs
  const int P = a.partition;

  // Work items are (sequence, pair y, run of partitions).  Dense grid: x =
  // run, y = pair, z = sequence, so all work of a sequence is dispatched
  // together; workgroups past a sequence's last partition exit at once.
  // Compact list (split contexts of a ragged batch, where most of the dense
  // grid would be such empty workgroups): the items of all sequences are
  // numbered consecutively -- sequence, then pair, then run -- and workgroup b
  // takes items b, b + gridDim.x, ...
  // compact list: first item of each sequence; dense grid: the lengths
  __shared__ int s_seq[kMaxCompactSeqs + 1];
  __shared__ int s_wsum[kWaves];
  int total = 1;
  if (a.compact) {
    auto runs_of = [&](int L) {
      const int np = L > 0 ? (L + P - 1) / P : 1;
      const bool bad = L < 0 || (L + B - 1) / B > a.width || np > a.max_parts;
      return bad ? 1 : (np + a.parts_per_wg - 1) / a.parts_per_wg;
    };
    const int i0 = 2 * threadIdx.x;
    const int c0 = i0 < a.S ? Y * runs_of(a.lens[i0]) : 0;
    const int c1 = i0 + 1 < a.S ? Y * runs_of(a.lens[i0 + 1]) : 0;
    int v = c0 + c1;  // inclusive scan over the wave's lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(v, d, 64);
      if (lane >= d) v += t;
    }
    if (lane == 63) s_wsum[wv] = v;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      before += w < wv ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
    const int excl = before + v - c0 - c1;
    if (i0 < a.S) s_seq[i0] = excl;
    if (i0 + 1 < a.S) s_seq[i0 + 1] = excl + c0;
    if (threadIdx.x == 0) s_seq[a.S] = total;
    __syncthreads();
  }

  // Longest sequences first (dense grid): workgroups are dispatched in
  // blockIdx order, so the workgroups of z take the z-th longest sequence
  // (ties by index).  Long sequences then start first and short ones fill
  // the tail.
  int s_dense = blockIdx.z;
  if (!a.compact && a.longest_first) {
    __shared__ int s_pick;
    for (int i = threadIdx.x; i < a.S; i += kThreads) s_seq[i] = a.lens[i];
    __syncthreads();
    for (int c = threadIdx.x; c < a.S; c += kThreads) {
      const int lc = s_seq[c];
      int rank = 0;
      for (int t = 0; t < a.S; ++t) {
        const int lt = s_seq[t];
        rank += (lt > lc || (lt == lc && t < c)) ? 1 : 0;
      }
      if (rank == static_cast<int>(blockIdx.z)) s_pick = c;
    }
    __syncthreads();
    s_dense = s_pick;
  }

  // one work item: sequence s, pair yy, partition run xr
  auto item = [&](const int s, const int yy, const int xr) {
    const int hg = yy / chunks;
    const int chunk = yy - hg * chunks;
    const int kvh = hg * HG + hi;
    const int nh = min(16, G - chunk * 16);
    const int h0 = kvh * G + chunk * 16;

    const int L = a.lens[s];
    const int nparts = L > 0 ? (L + P - 1) / P : 1;
    const bool bad_seq = L < 0 || (L + B - 1) / B > a.width || nparts > a.max_parts;
    // without a workspace (one partition per sequence) results always go to out
    const bool single = nparts == 1 || a.max_parts == 1;
    // this workgroup covers partitions [p_first, p_first + parts_per_wg); the
    // wave covers a contiguous run of pps of them, i.e. one token range
    const int pps = a.parts_per_wg / NSLOT;
    const int p_first = xr * a.parts_per_wg + slot * pps;
    if (p_first >= nparts) return;  // (partition 0 always exists)

    // LDS of this wave: the current step's K tile (32 tokens x D bf16), then
    // rows [i][hh][SROW] of its i-th finished partition, then their (m, l)
    const int nhs = min(16, G);  // head rows per partition slot
    float* wave_lds = s_dyn + static_cast<int64_t>(wv) * bf16_lds_wave_floats(pps, G, D, KL);
    char* k_lds = reinterpret_cast<char*>(wave_lds);
    float* stage = wave_lds + (KL ? bf16_lds_k_floats(D) : 0);
    float* stage_ml = stage + pps * nhs * SROW;  // 16-byte aligned: SROW % 4 == 0

    // Write partition p_first + i of heads h0 .. h0+nh-1 from the wave's LDS:
    // the normalised output (single partition) into out, else the partial
    // output and (m, l) into the workspace, whose layout [s][p][h][D] keeps a
    // wave's heads adjacent.  Each store instruction covers 64 consecutive
    // 16-byte pieces.
    auto store_rows = [&](int i) {
      const int p = p_first + i;
      const float* src = stage + i * nhs * SROW;
      constexpr int D4 = D / 4;
      const int64_t row0 = single ? static_cast<int64_t>(s) * a.Hq + h0
                                  : (static_cast<int64_t>(s) * a.max_parts + p) * a.Hq + h0;
      for (int e = lane; e < nh * D4; e += 64) {
        const int hh = e / D4;
        const int d = (e - hh * D4) * 4;
        const float4 o = *reinterpret_cast<const float4*>(src + hh * SROW + d);
        const int64_t off = row0 * D + static_cast<int64_t>(e) * 4;
        if (single && a.out_bf16) {
          const uint32_t lo = f32_to_bf16(o.x) | (static_cast<uint32_t>(f32_to_bf16(o.y)) << 16);
          const uint32_t hi2 = f32_to_bf16(o.z) | (static_cast<uint32_t>(f32_to_bf16(o.w)) << 16);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + off) = u32x2{lo, hi2};
        } else {
          *reinterpret_cast<float4*>((single ? static_cast<float*>(a.out) : a.ws_o) + off) = o;
        }
      }
      if (!single && lane < nh)
        *reinterpret_cast<float2*>(a.ws_ml + 2 * (row0 + lane)) =
            *reinterpret_cast<const float2*>(stage_ml + 2 * (i * nhs + lane));
    };

    if (bad_seq) {
      // the merge kernel poisons split sequences itself
      if (single) {
        for (int i = lane; i < nh * SROW; i += 64) stage[i] = NAN;
        __builtin_amdgcn_wave_barrier();
        store_rows(0);
      }
      return;
    }

    // query fragments: q[s][h0 + j][32c + 8g .. +8]
    bf16x8 qf[QC];
    {
      const uint16_t* qp = static_cast<const uint16_t*>(a.query) +
                           (static_cast<int64_t>(s) * a.Hq + h0 + j) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < QC; ++c)
        qf[c] = (j < nh) ? load_bf16x8<false>(qp + 32 * c) : bf16x8{};
    }

    const int tw_begin = p_first * P;
    const int tw_end = min(L, (p_first + pps) * P);
    const int my_steps = (tw_end - tw_begin + kStep - 1) / kStep;  // 0 only when L == 0

    const int64_t row = static_cast<int64_t>(a.Hkv) * D;  // elements between slots
    const uint16_t* kbase = static_cast<const uint16_t*>(a.kv) + static_cast<int64_t>(kvh) * D;
    const uint16_t* vbase = kbase + static_cast<int64_t>(a.NB) * B * row;
    const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.width;
    // Per-lane byte offsets inside a 16-token tile (unsigned 32-bit, so a load is
    // scalar base + vector offset).  Keys and values are read alike: one load
    // instruction covers 4 rows of D*2 contiguous bytes (lane (j, g): row
    // 4g + r, bytes 2*NV*j ..), the shape that streams at full rate; a load
    // giving each lane its MFMA row directly (16 rows of 64 bytes) streams ~30%
    // slower.  Keys are then rearranged through LDS for the score MFMA.
    uint32_t voff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) voff[r] = ((4 * g + r) * static_cast<uint32_t>(row) + NV * j) * 2u;
    const uint32_t koff = (j * static_cast<uint32_t>(row) + 8 * g) * 2u;

    // Block-table window: lane l holds the physical block of tile (l & 1) of
    // step q0 + (l >> 1), so 32 steps need one load; per step the entries are
    // read back as scalars.
    auto load_window = [&](int q0) -> int {
      const int tt = tw_begin + (q0 + (lane >> 1)) * kStep + 16 * (lane & 1);
      return tt < tw_end ? trow[tt / B] : -1;
    };
    int win_q0 = 0;
    int win = load_window(0);
    asm volatile("" ::"v"(win));

    // K arrives either row-wise like V and is rearranged through LDS (KL), or
    // straight in MFMA layout (token j, dims 32c + 8g: 16 rows of 64 bytes per
    // load instruction)
    struct Step {
      Words<NW> k[2][4];  // KL: token 4g + r of tile u, dims NV*j ..
      bf16x8 kd[2][QC];   // !KL: token j of tile u, dims 32c + 8g ..
      Words<NW> v[2][4];
      bool bad;  // a table entry of this step is out of range
    };
    bool bad_blk = false;  // ... of some step of the current partition

    // issue the loads of step q (tokens tw_begin + 32q ..).  The same 16 loads
    // are issued on every path, so the compiler can wait for exactly one
    // buffer's loads: a tile past the end of the run, or whose table entry is
    // out of range, reads block 0 instead (always in the pool); its scores are
    // masked and its values zeroed in compute(), or its partition poisoned.
    auto issue = [&](Step& d, int q) {
      if (q - win_q0 >= 32) {
        win_q0 = q;
        win = load_window(q);
        // wait for the entries here: a load still pending where the paths join
        // would make every step wait for all outstanding K/V loads
        asm volatile("" ::"v"(win));
      }
      const int ts = tw_begin + q * kStep;
      d.bad = false;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tt = ts + 16 * u;
        const int phys = __builtin_amdgcn_readlane(win, 2 * (q - win_q0) + u);
        const bool in_range = phys >= 0 && phys < a.NB;
        d.bad = d.bad || (tt < tw_end && !in_range);
        const int blk = (tt < tw_end && in_range) ? phys : 0;
        const int64_t base = (static_cast<int64_t>(blk) * B + (tt % B)) * row;
        const char* kp = reinterpret_cast<const char*>(kbase + base);
        const char* vp = reinterpret_cast<const char*>(vbase + base);
        if constexpr (KL) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            d.k[u][r] = load_words<NW, NT>(reinterpret_cast<const uint16_t*>(kp + voff[r]));
        } else {
#pragma unroll
          for (int c = 0; c < QC; ++c)
            d.kd[u][c] = load_bf16x8<NT>(reinterpret_cast<const uint16_t*>(kp + koff + 64 * c));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          d.v[u][r] = load_words<NW, NT>(reinterpret_cast<const uint16_t*>(vp + voff[r]));
      }
    };

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4 acc[NV];
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // keep partition p's result in LDS and start the next partition afresh.
    // lane (j, g) holds head j, dims NV*(4g + r) + n
    auto finalize = [&](int p) {
      float lsum = l_run + __shfl_xor(l_run, 16, 64);
      lsum += __shfl_xor(lsum, 32, 64);
      const bool bad = bad_blk;
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const int i = p - p_first;
      if (j < nh) {
        float* dst = stage + (i * nhs + j) * SROW;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int n0 = 0; n0 < NV; n0 += 4) {
            float4 o = make_float4(acc[n0][r] * inv, acc[n0 + 1][r] * inv, acc[n0 + 2][r] * inv,
                                   acc[n0 + 3][r] * inv);
            if (bad) o = make_float4(NAN, NAN, NAN, NAN);
            *reinterpret_cast<float4*>(dst + NV * (4 * g + r) + n0) = o;
          }
        if (g == 0)
          *reinterpret_cast<float2*>(stage_ml + 2 * (i * nhs + j)) =
              make_float2(bad ? NAN : m_run, bad ? NAN : lsum);
      }
      m_run = -INFINITY;
      l_run = 0.f;
#pragma unroll
      for (int n = 0; n < NV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      bad_blk = false;
    };

    auto compute = [&](Step& d, int q) {
      const int ts = tw_begin + q * kStep;
      if (q > 0 && ts % P == 0) finalize(ts / P - 1);  // a new partition starts here
      bad_blk = bad_blk || d.bad;
      const int lim = tw_end - ts;  // valid tokens in this step (>= 1)

      // K tile through LDS: token t of the step is a row of 2D bytes; its
      // 16-byte chunk ch sits at chunk position (ch + skew(t)) mod NCH, so both
      // the row-wise writes and the MFMA-layout reads (token j, chunk 4c + g)
      // hit distinct banks within each 16-lane pass
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (!KL) break;
          const int t = 16 * u + 4 * g + r;
          const int pb = NW * 4;                 // bytes of this lane's piece
          const int ch = (j * pb) >> 4;          // its 16-byte chunk
          const int pos = t * (2 * D) + 16 * ((ch + kskew(t)) % NCH) + ((j * pb) & 15);
          if constexpr (NW == 4) {
            *reinterpret_cast<u32x4*>(k_lds + pos) = u32x4{d.k[u][r].w[0], d.k[u][r].w[1], d.k[u][r].w[2], d.k[u][r].w[3]};
          } else {
            *reinterpret_cast<u32x2*>(k_lds + pos) = u32x2{d.k[u][r].w[0], d.k[u][r].w[1]};
          }
        }

      // scores
      float x[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < QC; ++c) {
          bf16x8 kf;
          if constexpr (KL) {
            const int t = 16 * u + j;
            const int pos = t * (2 * D) + 16 * ((4 * c + g + kskew(t)) % NCH);
            kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(k_lds + pos));
          } else {
            kf = d.kd[u][c];
          }
          sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[c], sc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) x[u][r] = sc[r] * a.scale_log2;
      }
      if (lim < kStep) {  // the sequence ends inside this step: mask scores, zero values
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * u + 4 * g + r >= lim) {
              x[u][r] = -INFINITY;
#pragma unroll
              for (int w = 0; w < NW; ++w) d.v[u][r].w[w] = 0u;
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
        for (int e = 0; e < 4; ++e) {
          const int e0 = 2 * e, e1 = 2 * e + 1;  // token slots (u = e/4, r = e%4)
          va[e] = __builtin_amdgcn_perm(d.v[e1 >> 2][e1 & 3].w[n >> 1], d.v[e0 >> 2][e0 & 3].w[n >> 1], sel);
        }
        const bf16x8 vb = __builtin_bit_cast(bf16x8, va);
        f32x4 o = acc[n] * alpha;
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, phi, o, 0, 0, 0);
        o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, plo, o, 0, 0, 0);
        acc[n] = o;
      }
    };

    // two register buffers: the next step's loads are in flight while the
    // current step computes (also across partition boundaries)
    Step bufA, bufB;
    if (my_steps > 0) issue(bufA, 0);
    for (int q = 0; q < my_steps; q += 2) {
      if (q + 1 < my_steps) issue(bufB, q + 1);
      compute(bufA, q);
      if (q + 1 >= my_steps) break;
      if (q + 2 < my_steps) issue(bufA, q + 2);
      compute(bufB, q + 1);
    }
    // the last partition (or, for an empty sequence, its zero output)
    const int p_last = my_steps > 0 ? (tw_begin + (my_steps - 1) * kStep) / P : p_first;
    finalize(p_last);
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i <= p_last - p_first; ++i) store_rows(i);
  };  // item

  if (!a.compact) {
    item(s_dense, blockIdx.y, blockIdx.x);
    return;
  }
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    // the sequence whose items contain it: the last s with s_seq[s] <= it
    int lo = 0, hi2 = a.S - 1;
    while (lo < hi2) {
      const int mid = (lo + hi2 + 1) >> 1;
      if (s_seq[mid] <= it) lo = mid; else hi2 = mid - 1;
    }
    const int nruns = (s_seq[lo + 1] - s_seq[lo]) / Y;
    const int local = it - s_seq[lo];
    const int yy = local / nruns;
    item(lo, yy, local - yy * nruns);
    // the wave's LDS is reused by the next item: finish reading it first
    __builtin_amdgcn_wave_barrier();
  }
}

// Workgroups of this kernel that one CU holds with `lds` bytes of dynamic LDS.
template <typename K>
int resident_per_cu(K kern, size_t lds) {
  static std::mutex mu;
  static size_t cached_lds = 0;
  static int cached = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached == 0 || cached_lds != lds) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kern), kThreads,
                                                     lds) != hipSuccess || n <= 0)
      n = 1;
    cached = n;
    cached_lds = lds;
  }
  return cached;
}

template <int D, int B, int HG, bool NT, bool KL>
int launch_one(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
  auto kern = attention_bf16_kernel<D, B, HG, NT, KL>;
  static bool attr_set = false;  // allow dynamic LDS up to the per-workgroup maximum
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bf16_lds_limit())) != hipSuccess) {
      set_error("paged attention (bf16): cannot raise the LDS limit");
      return PKV_ERR_HIP;
    }
    attr_set = true;
  }
  if (a.compact) {
    // one round of resident workgroups walks the item list (never more
    // workgroups than the dense grid has)
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      set_error("paged attention (bf16): cannot query the device");
      return PKV_ERR_HIP;
    }
    const int64_t dense = static_cast<int64_t>(grid.x) * grid.y * grid.z;
    grid = dim3(static_cast<unsigned>(std::min<int64_t>(dense, static_cast<int64_t>(cus) *
                                                                   resident_per_cu(kern, lds))));
  }
  kern<<<grid, dim3(kThreads), lds, stream>>>(a);
  return check_launch("paged attention (bf16)");
}

template <int D, int B, int HG>
int launch_hg(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
  const bool nt = a.nontemporal != 0, kl = a.k_via_lds != 0;
  if (nt) return kl ? launch_one<D, B, HG, true, true>(a, grid, lds, stream)
                    : launch_one<D, B, HG, true, false>(a, grid, lds, stream);
  return kl ? launch_one<D, B, HG, false, true>(a, grid, lds, stream)
            : launch_one<D, B, HG, false, false>(a, grid, lds, stream);
}

template <int D, int B>
int launch(const AttnArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) / 16;
  const int HG = bf16_heads_per_group(a.Hkv);
  dim3 grid((a.max_parts + a.parts_per_wg - 1) / a.parts_per_wg, (a.Hkv / HG) * chunks, a.S);
  const size_t lds = bf16_lds_bytes(a.parts_per_wg / (4 / HG), G, D, a.k_via_lds != 0);
  if (lds > bf16_lds_limit()) {
    set_error("paged attention (bf16): %zu bytes of LDS needed", lds);
    return PKV_ERR_UNSUPPORTED;
  }
  if (HG == 4) return launch_hg<D, B, 4>(a, grid, lds, stream);
  if (HG == 2) return launch_hg<D, B, 2>(a, grid, lds, stream);
  return launch_hg<D, B, 1>(a, grid, lds, stream);
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
