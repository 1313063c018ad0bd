// Paged prefill attention (gfx950): causal attention of chunks of query
// tokens over their sequences' paged K/V -- a whole prompt, or one chunk of
// it whose earlier tokens are already cached (chunked prefill, prefix-cache
// hits).  Sequence s's chunk is query rows [qstart[s], qstart[s+1]); row i
// of it sits at position lens[s] - chunk_len + i and attends keys 0 .. its
// position of its own sequence, read through the block table.
//
// bf16 caches: a workgroup (8 waves) takes a tile of 256 query vectors of
// one kv head (rows x its query heads); wave w takes vectors 32w .. 32w + 31
// as the 32 columns of 32 x 32 matrix-core tiles.  Workgroups take the
// tiles longest first (ranked in LDS by the keys they read) with the kv
// heads of a tile innermost, so the work of every XCD is the same and the
// launch ends on short tiles.  Keys are walked in steps of 64: the
// workgroup loads a step's K and V rows (through the table) into one of two
// LDS buffers while the waves compute on the other, so each K/V row is read
// from memory once per workgroup and 256 query vectors use it.  Per 32 keys
// a wave runs the scores S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (K rows
// from LDS as the A operand, its query vectors as B), the causal mask, an
// online softmax per vector in the log2 domain whose reference max moves
// only in jumps (few accumulator rescales), and O^T += V^T . P^T with P
// split into bf16 hi + lo parts and the V^T operand read from the row-major
// V tile by gfx950's transposing LDS read.  Rows are finished through LDS so
// every global store covers whole rows.  (Against 16 x 16 x 32 tiles: the
// same speed at head size 128, 10% faster at 64, where the kernel then fits
// in 128 registers and two workgroups share a CU.)
//
// fp32 caches: one wave per (query row, head), keys in batches of 64 with an
// online softmax (vector ALU; a reference-precision path).
#include "attention_bf16_wave.hpp"

#include <cmath>

namespace pkv {
namespace {

// Waves per workgroup: 8 (one workgroup per CU; at head size 128 two waves
// per SIMD, at 64 up to three).  A wave takes 32 query vectors, a workgroup
// a tile of 32 x waves: each K/V step staged in LDS serves 256 vectors, and
// the per-tile costs (ranking, first loads, output) come once per 256.
// Measured against 4 waves: 6% faster at head size 128, 2-3% at 64.
#ifndef PKV_PREFILL_WAVES_128
#define PKV_PREFILL_WAVES_128 8
#endif
#ifndef PKV_PREFILL_WAVES_64
#define PKV_PREFILL_WAVES_64 8
#endif
template <int D>
constexpr int kPWaves = D == 128 ? PKV_PREFILL_WAVES_128 : PKV_PREFILL_WAVES_64;
constexpr int kPKeys = 64;   // keys per LDS step
// tile costs (64-key steps) the launch orders its work by, counted exactly below this
constexpr int kRankBins = 1024;
// how far (log2 units) a row's max may pass its reference before a rescale
constexpr float kLazyLog2 = 8.f;

template <int D, int NW>
struct PGeom {
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROWS = 32 * NW;  // query vectors per tile
  static constexpr int NCH = D / 8;   // 16-byte chunks per row
  static constexpr int KROW = 2 * D;  // LDS bytes per K row (chunks skewed)
  // LDS bytes per V row, padded so the 8 rows x 32 bytes of a transposed
  // read's half-wave fall on distinct banks
  static constexpr int VROW = 2 * D + 64;
  static constexpr int KBYTES = kPKeys * KROW;
  static constexpr int BUF = KBYTES + kPKeys * VROW;
  static constexpr int CPT = kPKeys * NCH / THREADS;  // chunks per thread per tensor
  static constexpr int SROW = D + 4;  // floats per finished row in LDS
  static constexpr int LDS = 2 * BUF > ROWS * SROW * 4 ? 2 * BUF : ROWS * SROW * 4;
};

// max(v[l], v[l ^ 32]) without LDS: the permlane swap exchanges the two
// halves of the wave between its two operands, so swapping v with itself
// leaves one half's values in the first result and the other half's in the
// second.
__device__ __forceinline__ float max_xor32(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ds_read_b64_tr_b16 at an LDS byte address given as a generic pointer into
// the dynamic LDS array
__device__ __forceinline__ bf16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const_cast<char*>(p)));
}

// chunk ch of K row t sits at chunk position (ch + kskew(t)) mod NCH, so both
// the row-wise stores and the MFMA-layout reads (16 rows, one chunk each)
// spread over the banks
template <int NCH>
__device__ __forceinline__ int kskew(int t) { return (t * NCH / 16) % NCH; }

// A sequence's chunk as the launch sees it.  Per kv head the chunk holds
// qlen x G query vectors (row i, head kvh G + k is vector G i + k), taken in
// tiles of consecutive vectors: ntiles of them (none when the rows lie
// outside the output; at most the grid's qtiles).  A bad sequence's tiles
// write NaN rows only.
struct SeqShape {
  int q0, qlen, L, ntiles;
  bool bad;
};

template <int B, int ROWS>
__device__ __forceinline__ SeqShape seq_shape(const PrefillArgs& a, int s, int G) {
  SeqShape r;
  r.q0 = a.qstart[s];
  r.qlen = a.qstart[s + 1] - r.q0;
  r.L = a.lens[s];
  r.ntiles = 0;
  r.bad = false;
  if (r.q0 < 0 || r.qlen < 0 || r.q0 + r.qlen > a.T) return r;  // rows outside the output
  r.bad = r.L < 0 || (r.L + B - 1) / B > a.width || r.qlen > r.L || r.qlen > a.max_q;
  r.ntiles = min((r.qlen * G + ROWS - 1) / ROWS, a.qtiles);
  return r;
}

// v / G for 0 <= v < 2^31: a double-precision estimate, then one step of
// correction either way
__device__ __forceinline__ int div_g(int v, int G, double rG) {
  int q = static_cast<int>(static_cast<double>(v) * rG);
  const int r = v - q * G;
  q += r >= G ? 1 : 0;
  q -= r < 0 ? 1 : 0;
  return q;
}

// Keys [0, kend) tile x reads: up to the position of its last vector's row
template <int ROWS>
__device__ __forceinline__ int tile_kend(int qlen, int L, bool bad, int x, int G, double rG) {
  if (bad) return 0;
  const int last_row = div_g(min(qlen * G, (x + 1) * ROWS) - 1, G, rG);
  return max(0, min(L, L - qlen + last_row + 1));
}

// What tile x costs: the 64-key steps it reads (capped)
template <int ROWS>
__device__ __forceinline__ int tile_key(int qlen, int L, bool bad, int x, int G, double rG) {
  return min((tile_kend<ROWS>(qlen, L, bad, x, G, rG) + kPKeys - 1) / kPKeys, kRankBins - 1);
}

// Exclusive prefix sum of v over the workgroup; *total gets the sum.  Uses
// wsum[NW]; the caller separates two calls by a barrier.
template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(x, d, 64);
    if (lane >= d) x += t;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = wsum[w];
    before += w < wv ? t : 0;
    all += t;
  }
  *total = all;
  return before + x - v;
}

// The tile of rank r when the launch's tiles are ordered by tile_key,
// largest first (equal keys: by sequence, then tile).  A counting sort in
// LDS over the flattened list of tiles (sequence by sequence), each thread
// taking a contiguous run of it: the histogram of keys, the bin that holds
// rank r, then that bin's tiles in order.  sm holds nints ints (the
// histogram, a few scalars, and each sequence's first tile, chunk length
// and context length -- so batches of up to (nints - kRankBins - 25) / 3
// sequences).  Every thread of the workgroup calls it (it synchronises,
// and ends with a barrier, so the caller may reuse sm); false, for all of
// them, when r is past the last tile.
template <int B, int NW>
__device__ bool tile_of_rank(const PrefillArgs& a, int G, double rG, int r, int* sm, int nints,
                             int* s_out, int* x_out) {
  constexpr int THREADS = 64 * NW, ROWS = 32 * NW;
  static_assert(kRankBins % THREADS == 0 && NW <= 16, "bins split evenly over the threads");
  int* hist = sm;
  int* wsum = sm + kRankBins;  // [16]
  int* res = wsum + 16;        // [8]
  int* first = res + 8;        // [S + 1]: flattened index of each sequence's first tile
  int* qlen_of = first + a.S + 1;
  int* len_of = qlen_of + a.S;  // context length, -1 for a bad sequence
  const int tid = threadIdx.x;
  if (3 * a.S + 1 + kRankBins + 24 > nints) {  // host checks the batch fits
    return false;
  }
  // sequences: a contiguous run per thread
  const int per_s = (a.S + THREADS - 1) / THREADS;
  const int s0 = min(a.S, tid * per_s), s1 = min(a.S, s0 + per_s);
  int mine = 0;
  for (int s = s0; s < s1; ++s) {
    const SeqShape q = seq_shape<B, ROWS>(a, s, G);
    qlen_of[s] = q.qlen;
    len_of[s] = q.bad ? -1 : q.L;
    first[s] = q.ntiles;  // count for now
    mine += q.ntiles;
  }
  for (int i = tid; i < kRankBins; i += THREADS) hist[i] = 0;
  int ntot;
  int run0 = block_exclusive_scan<NW>(mine, wsum, &ntot);
  for (int s = s0; s < s1; ++s) {
    const int n = first[s];
    first[s] = run0;
    run0 += n;
  }
  if (tid == 0) first[a.S] = ntot;
  __syncthreads();
  // flattened tiles: a contiguous run per thread; (sequence, tile) of its first
  const int per_t = (ntot + THREADS - 1) / THREADS;
  const int i0 = min(ntot, tid * per_t), i1 = min(ntot, i0 + per_t);
  int sq = 0;
  {
    int lo = 0, hi = a.S;  // last sequence with first[s] <= i0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (first[mid] <= i0) lo = mid; else hi = mid;
    }
    sq = lo;
  }
  auto walk = [&](auto&& f) {  // f(key, sequence, tile) over this thread's run
    int s = sq;
    for (int i = i0; i < i1; ++i) {
      while (first[s + 1] <= i) ++s;
      const int x = i - first[s];
      const int L = len_of[s];
      f(tile_key<ROWS>(qlen_of[s], L, L < 0, x, G, rG), s, x);
    }
  };
  walk([&](int key, int, int) { atomicAdd(&hist[key], 1); });
  __syncthreads();
  // thread t holds the bins of keys kRankBins - 1 - PER t - k, k < PER
  constexpr int PER = kRankBins / THREADS;
  int c[PER], mb = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    c[k] = hist[kRankBins - 1 - (PER * tid + k)];
    mb += c[k];
  }
  int all;
  const int before = block_exclusive_scan<NW>(mb, wsum, &all);
  if (r >= all) return false;
  if (r >= before && r < before + mb) {
    int cum = before;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (r >= cum && r < cum + c[k]) {
        res[0] = kRankBins - 1 - (PER * tid + k);
        res[1] = r - cum;
      }
      cum += c[k];
    }
  }
  __syncthreads();
  const int key = res[0], j = res[1];
  // the j-th tile with that key, in flattened order
  int n = 0;
  walk([&](int k, int, int) { n += k == key; });
  int all2;
  int cum = block_exclusive_scan<NW>(n, wsum, &all2);
  if (j >= cum && j < cum + n) {
    walk([&](int k, int s, int x) {
      if (k != key) return;
      if (cum == j) {
        res[2] = s;
        res[3] = x;
      }
      ++cum;
    });
  }
  __syncthreads();
  *s_out = res[2];
  *x_out = res[3];
  __syncthreads();
  return true;
}

template <int D, int B>
__global__ void __launch_bounds__(64 * kPWaves<D>) __attribute__((amdgpu_waves_per_eu(2)))
prefill_bf16_kernel(PrefillArgs a) {
  constexpr int NW = kPWaves<D>;
  using Gm = PGeom<D, NW>;
  constexpr int kPThreads = Gm::THREADS, kPRows = Gm::ROWS;
  constexpr int NCH = Gm::NCH, CPT = Gm::CPT;
  extern __shared__ __align__(16) char lds[];
  const int tid = threadIdx.x;
  const int wv = tid >> 6, lane = tid & 63, j = lane & 15, g = lane >> 4;

  // Work item: (tile of rank r, kv head), kv heads innermost.  Tiles are
  // ranked longest first, so the launch ends on short items, and the kv
  // heads of a tile spread over the XCDs (workgroup b runs on XCD b % 8),
  // which keeps the XCDs' shares of the work equal whatever the batch's
  // length mix.  A tile's columns are query vectors of one kv head: its
  // G query heads at consecutive rows, so the K/V staged for it serve G
  // heads, and short chunks still fill the tile.
  const int bid = blockIdx.x;
  const int G = a.Hq / a.Hkv, kvh = bid % a.Hkv;
  int s, x;
  const double rG = 1.0 / G;
  if (!tile_of_rank<B, NW>(a, G, rG, bid / a.Hkv, reinterpret_cast<int*>(lds), Gm::LDS / 4, &s, &x))
    return;
  const SeqShape sq = seq_shape<B, kPRows>(a, s, G);
  const int q0 = sq.q0, qlen = sq.qlen, L = sq.L;
  const bool bad_seq = sq.bad;
  const int nvec = qlen * G;
  const int v0 = x * kPRows;                       // the tile's first vector
  const int tile_vecs = min(kPRows, nvec - v0);
  const int P0 = L - qlen;                         // position of the chunk's first row
  const int kend = tile_kend<kPRows>(qlen, L, bad_seq, x, G, rG);  // keys [0, kend)
  const int nsteps = (kend + kPKeys - 1) / kPKeys;

  // this wave's vectors: tile vectors 32 wv .. 32 wv + 31
  const int wr0 = 32 * wv;
  const int wave_vecs = max(0, min(32, tile_vecs - wr0));
  const int wmin = P0 + div_g(v0 + wr0, G, rG);    // position of the wave's first row
  const int wmax = wave_vecs > 0 ? P0 + div_g(v0 + wr0 + wave_vecs - 1, G, rG) : -1;  // ... and of its last
  // 32x32 tiles: column c32 = lane % 32 is tile vector 32 wv + c32; lanes
  // l and l + 32 hold the two halves (h2) of its k range
  const int h2 = lane >> 5, c32 = lane & 31;
  constexpr int QK = D / 16;  // score MFMAs (k = 16) per 32 x 32 tile
  constexpr int NB = D / 32;  // output blocks of 32 dims
  int pos1;
  bf16x8 qf[QK];
  const uint16_t* qb = static_cast<const uint16_t*>(a.query);
  {
    const int lv = wr0 + c32;
    const bool live = lv < tile_vecs;
    const int vv = v0 + lv, row = div_g(vv, G, rG), head = kvh * G + (vv - row * G);
    pos1 = live ? P0 + row : kend - 1;
    const uint16_t* qp = qb + (static_cast<int64_t>(q0 + row) * a.Hq + head) * D + 8 * h2;
#pragma unroll
    for (int c = 0; c < QK; ++c) qf[c] = live ? wave::load_bf16x8<false>(qp + 16 * c) : bf16x8{};
  }

  const int64_t rowst = static_cast<int64_t>(a.Hkv) * D;  // elements between slots
  const uint16_t* kbase = static_cast<const uint16_t*>(a.kv) + static_cast<int64_t>(kvh) * D;
  const uint16_t* vbase = kbase + static_cast<int64_t>(a.NB) * B * rowst;
  const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.width;
  bool bad = false;

  // global -> registers (step q) and registers -> LDS.  Thread chunk
  // e = tid + 256 i is row t0 + i * RSTEP of the step, 16-byte chunk ch; B
  // divides the 64-key step, so the row's offset inside its block is fixed
  // per thread.  The table entries a step's loads need are read one step
  // earlier, so the K/V loads never wait for them.  Rows at or past kend
  // read block 0 (always in the pool) and are zeroed in LDS instead (their
  // K/V may be unwritten); an out-of-range table entry is clamped into the
  // pool and poisons the result.
  constexpr int RSTEP = kPThreads / NCH;
  const int t0 = tid / NCH, ch = tid % NCH;
  const char* kbytes = reinterpret_cast<const char*>(kbase);
  const int64_t vdelta = reinterpret_cast<const char*>(vbase) - kbytes;
  const int64_t blockbytes = static_cast<int64_t>(B) * rowst * 2;
  wave::u32x4 pk[CPT], pv[CPT];
  int tab[CPT];
  auto load_table = [&](int q) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int key = q * kPKeys + t0 + RSTEP * i;
      tab[i] = key < kend ? trow[key / B] : 0;
    }
  };
  auto issue = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t phys = min(static_cast<uint32_t>(tab[i]), static_cast<uint32_t>(a.NB - 1));
      bad = bad || phys != static_cast<uint32_t>(tab[i]);
      const uint32_t inoff = (((t0 + RSTEP * i) % B) * static_cast<uint32_t>(rowst) + 8 * ch) * 2;
      const char* kp = kbytes + (static_cast<int64_t>(phys) * blockbytes + inoff);
      pk[i] = *reinterpret_cast<const wave::u32x4*>(kp);
      pv[i] = *reinterpret_cast<const wave::u32x4*>(kp + vdelta);
    }
  };
  auto stage = [&](char* buf, int valid_rows) {
    if (valid_rows < kPKeys) {  // the sequence's keys end inside this step
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        if (t0 + RSTEP * i >= valid_rows) {
          pk[i] = wave::u32x4{0u, 0u, 0u, 0u};
          pv[i] = wave::u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int t = t0 + RSTEP * i;
      *reinterpret_cast<wave::u32x4*>(buf + t * Gm::KROW + 16 * ((ch + kskew<NCH>(t)) % NCH)) = pk[i];
      *reinterpret_cast<wave::u32x4*>(buf + Gm::KBYTES + t * Gm::VROW + 16 * ch) = pv[i];
    }
  };

  // LDS byte offset of this lane's K piece c in a step's first 32 rows (the
  // skew repeats every 16 rows, so the second 32 are these plus 32 rows)
  int kofs[QK];
#pragma unroll
  for (int c = 0; c < QK; ++c) kofs[c] = c32 * Gm::KROW + 16 * ((2 * c + h2 + kskew<NCH>(c32)) % NCH);
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x16{};

  // fold 32 keys (rows 32 hs .. 32 hs + 31 of the LDS step at buf, first key
  // kb) into the wave's 32 vectors with v_mfma_f32_32x32x16_bf16.  Score
  // register e of lane l is key 8(e/4) + 4 h2 + e%4 of the 32; P operand m
  // (k = 16) takes registers 8m .. 8m + 7, i.e. keys 16m + 4 h2 + 0..3 and
  // 16m + 8 + 4 h2 + 0..3, and the V^T operand reads the same keys.
  auto substep = [&](const char* buf, int kb, int hs) {
    // one accumulation chain: the matrix core takes each product's result as
    // the next one's accumulator without waiting (two chains, even and odd k
    // blocks, added afterwards: 415-416 against 413-414 us on the OPT-13B
    // shape, 16 more adds per 32 keys)
    f32x16 sc = {};
    {
      const char* kb0 = buf + 32 * hs * Gm::KROW;
#pragma unroll
      for (int c = 0; c < QK; ++c) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const wave::u32x4*>(kb0 + kofs[c]));
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sc, 0, 0, 0);
      }
    }
    const float sl2 = a.scale_log2;
    float xs[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) xs[e] = sc[e];
    if (kb + 31 > wmin) {  // some key may be past some row of the wave
      int k = kb + 4 * h2;
      asm volatile("" : "+v"(k));  // keep the compares inside the branch
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (k + 8 * (e >> 2) + (e & 3) > pos1) xs[e] = -INFINITY;
    }
    float mx = xs[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, xs[e]);
    mx = max_xor32(mx);
    const float mxs = mx * sl2;
    float alpha = 1.f;
    if (mxs > m_run + kLazyLog2) {
      if (m_run != -INFINITY) alpha = wave::fast_exp2(m_run - mxs);
      m_run = mxs;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
    bf16x8 phi[2], plo[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = wave::fast_exp2(fmaf(xs[8 * m + e], sl2, -m_use));
        const float p1 = wave::fast_exp2(fmaf(xs[8 * m + e + 1], sl2, -m_use));
        psum += p0 + p1;
        const bf16x2 hh = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
        const uint32_t hw = __builtin_bit_cast(uint32_t, hh);
        const bf16x2 ll = __builtin_convertvector(
            f32x2{p0 - __uint_as_float(hw << 16), p1 - __uint_as_float(hw & 0xFFFF0000u)}, bf16x2);
        phi[m][e] = hh.x;
        phi[m][e + 1] = hh.y;
        plo[m][e] = ll.x;
        plo[m][e + 1] = ll.y;
      }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
      float al = alpha;
      asm volatile("" : "+v"(al));  // keep the multiplies inside the branch
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] *= al;
    }
    // V^T operand of output block n (dims 32n .. 32n + 31) for P operand m:
    // the 16-lane group (h2, half) reads the 4-row x 16-column blocks at
    // keys 16m + 4 h2 (+ 8) and dims 32n + 16 half, lane j getting column j
    const char* vt = buf + Gm::KBYTES + (32 * hs + 4 * h2 + ((lane & 15) >> 2)) * Gm::VROW +
                     32 * ((lane >> 4) & 1) + 8 * (lane & 3);
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x4 w0 = lds_read_tr16(vt + 16 * m * Gm::VROW + 64 * n);
        const bf16x4 w1 = lds_read_tr16(vt + (16 * m + 8) * Gm::VROW + 64 * n);
        const bf16x8 vb = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, phi[m], acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, plo[m], acc[n], 0, 0, 0);
      }
  };

  if (nsteps > 0) {
    load_table(0);
    issue();
    if (nsteps > 1) load_table(1);
    stage(lds, kend);
  }
  // The query fragments arrive before the loop: otherwise the compiler,
  // allowing for their loads still being in flight on the first pass, makes
  // every step's first score wait for the oldest K/V loads of the next step.
#pragma unroll
  for (int c = 0; c < QK; ++c) asm volatile("" : "+v"(qf[c]));
  __syncthreads();
  for (int q = 0; q < nsteps; ++q) {
    const char* cur = lds + (q & 1) * Gm::BUF;
    // The next step's loads are issued on every pass, the last included (its
    // table entries are stale but in the pool, and nothing stages them): a
    // path skipping them left the table loads possibly pending where the
    // paths meet, and the compiler then waited for every outstanding load --
    // these K/V loads too -- before the next table loads, so they never
    // overlapped the computation.
    issue();
    if (q + 2 < nsteps) load_table(q + 2);
    const int k0 = q * kPKeys;
    // keys past every row of the wave need no work; a step reaching past
    // the wave's first row needs the causal mask
    if (k0 <= wmax) substep(cur, k0, 0);
    if (k0 + 32 <= wmax) substep(cur, k0 + 32, 1);
    if (q + 1 < nsteps) stage(lds + ((q + 1) & 1) * Gm::BUF, kend - (q + 1) * kPKeys);
    __syncthreads();
  }
  bad = __syncthreads_or(bad) || bad_seq;

  // finish: normalise, stage rows [kPRows][SROW] in LDS (no wave reads K/V any
  // more), then store whole rows
  float* rows = reinterpret_cast<float*>(lds);
  {
    const float lsum = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* dst = rows + (wr0 + c32) * Gm::SROW;
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // dims 32n + 8i + 4 h2 .. + 3
        float4 o = make_float4(acc[n][4 * i] * inv, acc[n][4 * i + 1] * inv,
                               acc[n][4 * i + 2] * inv, acc[n][4 * i + 3] * inv);
        if (bad) o = make_float4(NAN, NAN, NAN, NAN);
        *reinterpret_cast<float4*>(dst + 32 * n + 8 * i + 4 * h2) = o;
      }
  }
  __syncthreads();
  constexpr int D4 = D / 4;
  for (int e = lane; e < 32 * D4; e += 64) {
    const int lv = wr0 + e / D4;
    if (lv >= tile_vecs) break;
    const int d = (e % D4) * 4;
    const float4 o = *reinterpret_cast<const float4*>(rows + lv * Gm::SROW + d);
    const int vv = v0 + lv, row = div_g(vv, G, rG), head = kvh * G + (vv - row * G);
    const int64_t off = (static_cast<int64_t>(q0 + row) * a.Hq + head) * D + d;
    if (a.out_bf16) {
      const uint32_t lo = f32_to_bf16(o.x) | (static_cast<uint32_t>(f32_to_bf16(o.y)) << 16);
      const uint32_t hi = f32_to_bf16(o.z) | (static_cast<uint32_t>(f32_to_bf16(o.w)) << 16);
      *reinterpret_cast<wave::u32x2*>(static_cast<uint16_t*>(a.out) + off) = wave::u32x2{lo, hi};
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = o;
    }
  }
  // A chunk longer than max_query_len has vectors past the grid's tiles:
  // the last tile writes them too (NaN, as for every row of a bad
  // sequence), so no row of the chunk keeps what the output held before.
  if (bad_seq && x == a.qtiles - 1 && nvec > a.qtiles * kPRows) {
    const int vbeg = a.qtiles * kPRows;
    const int64_t n4 = static_cast<int64_t>(nvec - vbeg) * D4;
    for (int64_t e = tid; e < n4; e += kPThreads) {
      const int vv = vbeg + static_cast<int>(e / D4);
      const int d = static_cast<int>(e % D4) * 4;
      const int row = div_g(vv, G, rG), head = kvh * G + (vv - row * G);
      const int64_t off = (static_cast<int64_t>(q0 + row) * a.Hq + head) * D + d;
      if (a.out_bf16) {
        const uint32_t nn = f32_to_bf16(NAN) | (static_cast<uint32_t>(f32_to_bf16(NAN)) << 16);
        *reinterpret_cast<wave::u32x2*>(static_cast<uint16_t*>(a.out) + off) = wave::u32x2{nn, nn};
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) =
            make_float4(NAN, NAN, NAN, NAN);
      }
    }
  }
}

// fp32: one wave per (query row, query head)
template <int D>
__global__ void __launch_bounds__(64) prefill_f32_kernel(PrefillArgs a) {
  constexpr int PER = D / 64;
  __shared__ float s_q[D];
  __shared__ float s_p[64];
  // element offset of each key's row in the K (and V) half of the pool, -1
  // for a key past the row's causal end or on a block outside the pool
  __shared__ int64_t s_off[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x, h = blockIdx.y;
  // the sequence whose chunk holds this row: largest s with qstart[s] <= row
  int lo = 0, hi = a.S;  // qstart[lo] <= row < qstart[hi] if the row is covered
  if (a.S == 0 || row < a.qstart[0] || row >= a.qstart[a.S]) return;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (a.qstart[mid] <= row) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int q0 = a.qstart[s], qlen = a.qstart[s + 1] - q0;
  const int L = a.lens[s];
  const int B = a.B;
  const bool bad_seq = L < 0 || (L + B - 1) / B > a.width || qlen > L || qlen > a.max_q;
  const int n = bad_seq ? 0 : max(0, min(L, L - qlen + (row - q0) + 1));  // keys 0 .. position
  const int kvh = h / (a.Hq / a.Hkv);
  const float* q = static_cast<const float*>(a.query) + (static_cast<int64_t>(row) * a.Hq + h) * D;
  for (int d = lane; d < D; d += 64) s_q[d] = q[d];
  __syncthreads();

  const int64_t rowst = static_cast<int64_t>(a.Hkv) * D;
  const float* kbase = static_cast<const float*>(a.kv) + static_cast<int64_t>(kvh) * D;
  const float* vbase = kbase + static_cast<int64_t>(a.NB) * B * rowst;
  const int32_t* trow = a.tables + static_cast<int64_t>(s) * a.width;
  bool bad = bad_seq;
  float m = -INFINITY, l = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int t = t0 + lane;
    float sc = -INFINITY;
    int phys = -1;
    if (t < n) {
      phys = trow[t / B];
      if (phys < 0 || phys >= a.NB) {
        bad = true;
        phys = -1;
      } else {
        const float4* kr = reinterpret_cast<const float4*>(kbase + (static_cast<int64_t>(phys) * B + t % B) * rowst);
        float dot = 0.f;
        for (int c = 0; c < D / 4; ++c) {
          const float4 kk = kr[c];
          dot = fmaf(kk.x, s_q[4 * c], dot);
          dot = fmaf(kk.y, s_q[4 * c + 1], dot);
          dot = fmaf(kk.z, s_q[4 * c + 2], dot);
          dot = fmaf(kk.w, s_q[4 * c + 3], dot);
        }
        sc = dot * a.scale_log2;
      }
    }
    const float m_new = fmaxf(m, wave_max(sc));
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    const float p = __builtin_amdgcn_exp2f(sc - m_use);  // 0 for a key without a score
    l = l * alpha + wave_sum(p);
    m = m_new;
    s_p[lane] = p;
    s_off[lane] = phys >= 0 ? (static_cast<int64_t>(phys) * B + t % B) * rowst : -1;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= alpha;
    // values KB keys at a time, every load issued (a key without a row reads
    // the pool's first row, zeroed), so no branch separates them
    constexpr int KB = 16;
    const int cnt = min(64, n - t0);
    for (int k0 = 0; k0 < cnt; k0 += KB) {
      float v[KB][PER];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int64_t off = s_off[k0 + k];
        const float* vr = vbase + (off >= 0 ? off : 0) + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) v[k][e] = vr[e];
#pragma unroll
        for (int e = 0; e < PER; ++e) v[k][e] = off >= 0 ? v[k][e] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const float pk = s_p[k0 + k];
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(pk, v[k][e], acc[e]);
      }
    }
    __syncthreads();
  }
  bad = __any(bad);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float o = bad ? NAN : acc[e] * inv;
    const int64_t off = (static_cast<int64_t>(row) * a.Hq + h) * D + lane * PER + e;
    if (a.out_bf16) static_cast<uint16_t*>(a.out)[off] = f32_to_bf16(o);
    else static_cast<float*>(a.out)[off] = o;
  }
}

template <int D, int B>
int launch_bf16_db(const PrefillArgs& a, hipStream_t stream) {
  auto kern = prefill_bf16_kernel<D, B>;
  using Gm = PGeom<D, kPWaves<D>>;
  const int lds = Gm::LDS;
  if (const int rc = raise_lds_limit(reinterpret_cast<const void*>(kern), lds)) return rc;
  kern<<<dim3(static_cast<unsigned>(a.total)), dim3(Gm::THREADS), lds, stream>>>(a);
  return check_launch("paged prefill (bf16)");
}

template <int D>
int launch_bf16_d(const PrefillArgs& a, hipStream_t stream) {
  switch (a.B) {
    case 8: return launch_bf16_db<D, 8>(a, stream);
    case 16: return launch_bf16_db<D, 16>(a, stream);
    case 32: return launch_bf16_db<D, 32>(a, stream);
    case 64: return launch_bf16_db<D, 64>(a, stream);
  }
  set_error("paged prefill (bf16): block_size %d is not built (8, 16, 32, 64)", a.B);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace

int prefill_max_seqs(int D) {
  const int nints = (D == 64 ? PGeom<64, kPWaves<64>>::LDS : PGeom<128, kPWaves<128>>::LDS) / 4;
  return (nints - kRankBins - 24 - 1) / 3;
}

int prefill_tile_vectors(int D) { return 32 * (D == 64 ? kPWaves<64> : kPWaves<128>); }

int launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  if (a.total == 0) return PKV_OK;
  if (a.D == 64) return launch_bf16_d<64>(a, stream);
  if (a.D == 128) return launch_bf16_d<128>(a, stream);
  set_error("paged prefill (bf16): head_size %d is not built (64, 128)", a.D);
  return PKV_ERR_UNSUPPORTED;
}

int launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  if (a.T == 0 || a.S == 0) return PKV_OK;
  const dim3 grid(static_cast<unsigned>(a.T), static_cast<unsigned>(a.Hq));
  if (a.D == 64) {
    prefill_f32_kernel<64><<<grid, dim3(64), 0, stream>>>(a);
  } else if (a.D == 128) {
    prefill_f32_kernel<128><<<grid, dim3(64), 0, stream>>>(a);
  } else {
    set_error("paged prefill (fp32): head_size %d is not built (64, 128)", a.D);
    return PKV_ERR_UNSUPPORTED;
  }
  return check_launch("paged prefill (fp32)");
}

}  // namespace pkv
