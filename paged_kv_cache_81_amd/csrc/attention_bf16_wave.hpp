// One wave's machinery for paged decode attention over bf16 caches (gfx950):
// loading 32-token steps of K/V through a block table, scores on matrix
// cores, online softmax, P.V, and finishing a run of tokens into LDS.  Both
// bf16 kernels (fixed partitions, and the balanced stream schedule) drive it.
//
// A wave works on one kv head and up to 16 of the query heads sharing it, so
// every K/V row piece is read once per kv head.  A step covers 32 tokens as
// two 16-token tiles.  Lane l is (j, g) with j = l % 16 and g = l / 16.
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
//  * Block-table entries are loaded once per 32 steps (one per lane) and read
//    back as scalars; two steps of K/V are kept in registers, the next one
//    issued before the current one is folded in (see run()).
#pragma once

#include "common.hpp"

#include <cmath>

namespace pkv {
namespace wave {

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
__device__ __forceinline__ Words<NW> load_words(const char* p) {
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
__device__ __forceinline__ bf16x8 load_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8, ld<NT>(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Block-table entries per 32-token step: one per 16-token tile, or one per
// block when blocks are smaller than a tile (B = 8: a tile spans two).
template <int B>
__host__ __device__ constexpr int window_entries_per_step() { return B < 16 ? kStep / B : 2; }

// Block-table window of the token run [t0, t1) read through table row trow:
// lane l holds the physical block of piece l % EPS (a 16-token tile, or a
// block of 8 tokens) of step q0 + l / EPS, -1 past the run, so 64 / EPS
// steps take one load.
template <int B>
__device__ __forceinline__ int table_window(const int32_t* trow, int t0, int t1, int q0, int lane) {
  constexpr int EPS = window_entries_per_step<B>();
  const int tt = t0 + (q0 + lane / EPS) * kStep + (kStep / EPS) * (lane % EPS);
  return tt < t1 ? trow[tt / B] : -1;
}

// Floats of LDS one wave's K tile takes (32 tokens x D bf16).
__host__ __device__ constexpr int k_tile_floats(int D) { return 16 * D; }

template <int D, int B, bool NT, bool KL>
struct Wave {
  static constexpr int QC = D / 32;  // score MFMAs per tile (32 dims each)
  static constexpr int NV = D / 16;  // output blocks of 16 rows; dims per lane per V token
  static constexpr int NW = NV / 2;  // 32-bit words per lane per V token
  static constexpr int NCH = D / 8;  // 16-byte chunks per K row
  static constexpr int SROW = D + 4;  // LDS floats per finished head row (padded)
  static constexpr int EPS = window_entries_per_step<B>();
  static constexpr int WIN = 64 / EPS;  // steps one table window covers
  static_assert(B >= 8 && 64 % EPS == 0, "unsupported block size");

  // K arrives either row-wise like V and is rearranged through LDS (KL), or
  // straight in MFMA layout (token j, dims 32c + 8g: 16 rows of 64 bytes per
  // load instruction)
  struct Step {
    Words<NW> k[2][4];  // KL: token 4g + r of tile u, dims NV*j ..
    bf16x8 kd[2][QC];   // !KL: token j of tile u, dims 32c + 8g ..
    Words<NW> v[2][4];
    bool bad;  // a table entry of this step is out of range
  };

  int lane, j, g;
  int NB;
  float scale_log2;
  char* k_lds;  // this wave's K tile (KL)
  // per-lane byte offsets inside a 16-token tile (unsigned 32-bit, so a load
  // is scalar base + vector offset)
  uint32_t voff[4];
  uint32_t koff;
  int64_t row;  // elements between consecutive slots (Hkv * D)

  // the token run being read: [t_begin, t_end) of one sequence and kv head
  const char* kbase;
  const char* vbase;
  const int32_t* trow;
  int t_begin, t_end;
  int win, win_q0;  // block-table window of steps [win_q0, win_q0 + WIN) (see load_window)
  int win_next;     // ... and of the 32 steps after it
  bf16x8 qf[QC];

  // running softmax state of the current partition
  float m_run, l_run;
  f32x4 acc[NV];
  bool bad_blk;  // a table entry of some step of the partition is out of range

  __device__ __forceinline__ void init(const AttnArgs& a, char* k_tile) {
    lane = threadIdx.x & 63;
    j = lane & 15;
    g = lane >> 4;
    NB = a.NB;
    scale_log2 = a.scale_log2;
    k_lds = k_tile;
    row = static_cast<int64_t>(a.Hkv) * D;
    // Keys and values are read alike when keys go through LDS: one load
    // instruction covers 4 rows of D*2 contiguous bytes (lane (j, g): row
    // 4g + r, bytes 2*NV*j ..).
#pragma unroll
    for (int r = 0; r < 4; ++r) voff[r] = ((4 * g + r) % B * static_cast<uint32_t>(row) + NV * j) * 2u;
    koff = (j % B * static_cast<uint32_t>(row) + 8 * g) * 2u;
    reset();
  }

  __device__ __forceinline__ void reset() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int n = 0; n < NV; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    bad_blk = false;
  }

  // Block-table window of steps q0 .. q0 + WIN - 1 of the run (see
  // table_window); per step the entries are read back as scalars.
  __device__ __forceinline__ int load_window(int q0) const {
    return table_window<B>(trow, t_begin, t_end, q0, lane);
  }

  // Start reading tokens [t0, t1) of sequence s for kv head kvh and query
  // heads h0 .. h0 + nh - 1: query fragments q[s][h0 + j][32c + 8g .. +8]
  // and the first table window.
  __device__ __forceinline__ void begin(const AttnArgs& a, int s, int kvh, int h0, int nh, int t0,
                                        int t1) {
    begin_rows(a, j < nh ? static_cast<int64_t>(s) * a.Hq + h0 + j : -1, s, kvh, t0, t1);
  }

  // The same with any query rows: column j of the score tile is query row
  // qrow (of the [S * Hq] rows; qrow < 0: no query, a zero column) of the
  // lane's j, and the tokens are read through table row s.
  __device__ __forceinline__ void begin_rows(const AttnArgs& a, int64_t qrow, int s, int kvh, int t0,
                                             int t1) {
    start_rows(a, qrow, s, kvh, t0, t1);
    win = load_window(0);
    asm volatile("" ::"v"(win));
    win_next = load_window(WIN);
  }

  // The same with the run's first table window given (win0: this lane's
  // entry of it, as load_window(0) would return), e.g. from a plan.
  __device__ __forceinline__ void begin_rows(const AttnArgs& a, int64_t qrow, int s, int kvh, int t0,
                                             int t1, int win0) {
    start_rows(a, qrow, s, kvh, t0, t1);
    win = win0;
    win_next = load_window(WIN);
  }

  // query fragments and the run's addresses
  __device__ __forceinline__ void start_rows(const AttnArgs& a, int64_t qrow, int s, int kvh, int t0,
                                             int t1) {
    const uint16_t* qp = static_cast<const uint16_t*>(a.query) + (qrow < 0 ? 0 : qrow) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < QC; ++c) qf[c] = (qrow >= 0) ? load_bf16x8<false>(qp + 32 * c) : bf16x8{};
    const uint16_t* kb = static_cast<const uint16_t*>(a.kv) + static_cast<int64_t>(kvh) * D;
    kbase = reinterpret_cast<const char*>(kb);
    vbase = reinterpret_cast<const char*>(kb + static_cast<int64_t>(NB) * B * row);
    trow = a.tables + static_cast<int64_t>(s) * a.width;
    t_begin = t0;
    t_end = t1;
    win_q0 = 0;
  }

  // Issue the loads of step q (tokens t_begin + 32q ..), steps in order.
  // The same K/V loads are issued on every path, so the compiler can wait
  // for exactly one buffer's loads: a tile past the end of the run, or whose
  // table entry is out of range, reads block 0 instead (always in the pool);
  // its scores are masked and its values zeroed in compute(), or its
  // partition poisoned.  Table windows are loaded one window ahead: when the
  // steps reach the prefetched window it becomes current and the next one
  // is requested (ahead of this step's K/V, so waiting for it later costs
  // nothing extra).
  __device__ __forceinline__ void issue(Step& d, int q) {
    if (q - win_q0 >= WIN) {
      win = win_next;
      win_q0 += WIN;
      win_next = load_window(win_q0 + WIN);
    }
    const int ts = t_begin + q * kStep;
    d.bad = false;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tt = ts + 16 * u;
      if constexpr (B >= 16) {
        const int phys = __builtin_amdgcn_readlane(win, 2 * (q - win_q0) + u);
        const bool in_range = phys >= 0 && phys < NB;
        d.bad = d.bad || (tt < t_end && !in_range);
        const int blk = (tt < t_end && in_range) ? phys : 0;
        const int64_t base = ((static_cast<int64_t>(blk) * B + (tt % B)) * row) * 2;
        const char* kp = kbase + base;
        const char* vp = vbase + base;
        if constexpr (KL) {
#pragma unroll
          for (int r = 0; r < 4; ++r) d.k[u][r] = load_words<NW, NT>(kp + voff[r]);
        } else {
#pragma unroll
          for (int c = 0; c < QC; ++c) d.kd[u][c] = load_bf16x8<NT>(kp + koff + 64 * c);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) d.v[u][r] = load_words<NW, NT>(vp + voff[r]);
      } else {
        // blocks of 8: the tile spans two, tokens 0-7 in the first and 8-15
        // in the second; each lane's rows (4g + r for V and row-wise K, j
        // for K in MFMA layout) sit in one of them
        static_assert(B == 8, "blocks below 16 tokens: only 8 is built");
        int64_t base[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int phys = __builtin_amdgcn_readlane(win, EPS * (q - win_q0) + 2 * u + p);
          const bool live = tt + B * p < t_end;
          const bool in_range = phys >= 0 && phys < NB;
          d.bad = d.bad || (live && !in_range);
          base[p] = static_cast<int64_t>((live && in_range) ? phys : 0) * B * row * 2;
        }
        const int64_t vrow = g >= 2 ? base[1] : base[0];
        const char* kp = kbase + vrow;
        const char* vp = vbase + vrow;
        if constexpr (KL) {
#pragma unroll
          for (int r = 0; r < 4; ++r) d.k[u][r] = load_words<NW, NT>(kp + voff[r]);
        } else {
          const char* kj = kbase + (j >= 8 ? base[1] : base[0]);
#pragma unroll
          for (int c = 0; c < QC; ++c) d.kd[u][c] = load_bf16x8<NT>(kj + koff + 64 * c);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) d.v[u][r] = load_words<NW, NT>(vp + voff[r]);
      }
    }
  }

  static __device__ __forceinline__ int kskew(int t) { return (t * NCH / 16) % NCH; }

  // Fold step q (loaded into d) into the running partition.  MASK: the run
  // may end inside this step.
  template <bool MASK>
  __device__ __forceinline__ void compute(Step& d, int q) {
    const int ts = t_begin + q * kStep;
    bad_blk = bad_blk || d.bad;
    const int lim = t_end - ts;  // valid tokens in this step (>= 1)

    // K tile through LDS: token t of the step is a row of 2D bytes; its
    // 16-byte chunk ch sits at chunk position (ch + skew(t)) mod NCH, so both
    // the row-wise writes and the MFMA-layout reads (token j, chunk 4c + g)
    // hit distinct banks within each 16-lane pass
    if constexpr (KL) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * u + 4 * g + r;
          const int pb = NW * 4;         // bytes of this lane's piece
          const int ch = (j * pb) >> 4;  // its 16-byte chunk
          const int pos = t * (2 * D) + 16 * ((ch + kskew(t)) % NCH) + ((j * pb) & 15);
          if constexpr (NW == 4) {
            *reinterpret_cast<u32x4*>(k_lds + pos) =
                u32x4{d.k[u][r].w[0], d.k[u][r].w[1], d.k[u][r].w[2], d.k[u][r].w[3]};
          } else {
            *reinterpret_cast<u32x2*>(k_lds + pos) = u32x2{d.k[u][r].w[0], d.k[u][r].w[1]};
          }
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
      for (int r = 0; r < 4; ++r) x[u][r] = sc[r] * scale_log2;
    }
    if (MASK && lim < kStep) {  // the run ends inside this step: mask scores, zero values
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
        va[e] = __builtin_amdgcn_perm(d.v[e1 >> 2][e1 & 3].w[n >> 1],
                                      d.v[e0 >> 2][e0 & 3].w[n >> 1], sel);
      }
      const bf16x8 vb = __builtin_bit_cast(bf16x8, va);
      f32x4 o = acc[n] * alpha;
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, phi, o, 0, 0, 0);
      o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, plo, o, 0, 0, 0);
      acc[n] = o;
    }
  }

  // Steps 0 .. nsteps-1 of the run through two register buffers: step q+1
  // is issued before step q is folded in.  As compiled, the wait before
  // step q covers step q+1's loads too (the last pass skips the issue, so
  // where the paths meet the compiler cannot tell which loads are still
  // pending), so a wave keeps one step in flight and does not overlap its
  // own loads with its arithmetic; the 8-12 waves of a CU cover each other.
  // Measured against this on one box (OPT-13B-shaped / Qwen2-shaped /
  // long-context attention): true overlap (every issue unconditional, so
  // the wait covers only step q) was 6.5% / 4.7% / 0.5% slower -- more
  // loads in flight per CU deepen the HBM queues, as a plain streaming read
  // also shows; awaiting each step before issuing the next and overlapping
  // its arithmetic, 3% slower on the OPT-13B shape; one register buffer,
  // and the same order as here with explicit waits, 5% slower on it.  The
  // fixed-partition kernel uses this loop; the stream and shared-prefix
  // kernels use run_single below.
  // at_step(q) runs before step q is folded in (partition boundaries).
  template <typename F>
  __device__ __forceinline__ void run(int nsteps, F&& at_step) {
    Step bufA, bufB;
    if (nsteps > 0) issue(bufA, 0);
    for (int q = 0; q < nsteps; q += 2) {
      if (q + 1 < nsteps) issue(bufB, q + 1);
      at_step(q);
      compute<true>(bufA, q);
      if (q + 1 >= nsteps) break;
      if (q + 2 < nsteps) issue(bufA, q + 2);
      at_step(q + 1);
      compute<true>(bufB, q + 1);
    }
  }

  // The same with one step in flight: issue step q, then fold it in.  Half
  // the bytes a wave has in flight at once and half the K/V registers (at
  // head size 128, 153-165 VGPRs against 253).  Measured against run() on
  // one box, each run after 20 s idle: OPT-13B-shaped stream 220.9-221.0 vs
  // 222.2-222.9 us, long-context 328.5-328.6 vs 328.7-329.0 us, Qwen2-shaped
  // 26.4-26.9 us both; the shared-prefix decode (eight waves a CU) 62.3-62.8
  // vs 62.8-64.8 us.
  template <typename F>
  __device__ __forceinline__ void run_single(int nsteps, F&& at_step) {
    Step buf;
    for (int q = 0; q < nsteps; ++q) {
      issue(buf, q);
      at_step(q);
      compute<true>(buf, q);
    }
  }

  // Write the partition's normalised output rows [hh][SROW] (head hh of the
  // wave's query heads) and (m, l) pairs into LDS and start afresh.  Lane
  // (j, g) holds head j, dims NV*(4g + r) + n.  A poisoned partition gives NaN.
  __device__ __forceinline__ void finish(float* rows, float* ml, int nh) {
    float lsum = l_run + __shfl_xor(l_run, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    const bool bad = bad_blk;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (j < nh) {
      float* dst = rows + j * SROW;
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
        *reinterpret_cast<float2*>(ml + 2 * j) =
            make_float2(bad ? NAN : m_run, bad ? NAN : lsum);
    }
    reset();
  }
};

// Copy nh finished head rows from LDS to global memory: into out (rows
// [row0, row0 + nh) of [S*Hq][D], fp32 or rounded to bf16) when to_out, else
// into the workspace (partial output rows of ws_o, (m, l) pairs of ws_ml).
// Each store instruction covers 64 consecutive 16-byte pieces.
template <int D>
__device__ __forceinline__ void store_rows(const AttnArgs& a, const float* rows, const float* ml,
                                           int nh, int64_t row0, bool to_out, int lane) {
  constexpr int D4 = D / 4;
  constexpr int SROW = D + 4;
  for (int e = lane; e < nh * D4; e += 64) {
    const int hh = e / D4;
    const int d = (e - hh * D4) * 4;
    const float4 o = *reinterpret_cast<const float4*>(rows + hh * SROW + d);
    const int64_t off = row0 * D + static_cast<int64_t>(e) * 4;
    if (to_out && a.out_bf16) {
      const uint32_t lo = f32_to_bf16(o.x) | (static_cast<uint32_t>(f32_to_bf16(o.y)) << 16);
      const uint32_t hi = f32_to_bf16(o.z) | (static_cast<uint32_t>(f32_to_bf16(o.w)) << 16);
      *reinterpret_cast<wave::u32x2*>(static_cast<uint16_t*>(a.out) + off) = wave::u32x2{lo, hi};
    } else {
      *reinterpret_cast<float4*>((to_out ? static_cast<float*>(a.out) : a.ws_o) + off) = o;
    }
  }
  if (!to_out && lane < nh)
    *reinterpret_cast<float2*>(a.ws_ml + 2 * (row0 + lane)) =
        *reinterpret_cast<const float2*>(ml + 2 * lane);
}

}  // namespace wave
}  // namespace pkv
