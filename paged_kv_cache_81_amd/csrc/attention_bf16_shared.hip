// Paged decode attention for bf16 caches on gfx950 when groups of sequences
// share their first blocks: the parallel samples of one prompt, whose tables
// all hold the prompt's physical blocks (each with a reference count above
// one) followed by blocks of their own.
//
// The attention is unchanged -- every sequence attends to all of its tokens --
// but a group's shared prefix is read once instead of once per member:
//  * a prefix item reads one partition of the group's shared tokens for one
//    kv head and scores it against the query heads of all the members at
//    once: the members' heads are the columns of the score tile (column c is
//    member c / G, head c % G of that kv head), up to 16 per wave;
//  * a suffix item reads one partition of a single sequence's tokens after
//    the prefix, as the ordinary decode does.
// Every item leaves a partial result (normalised rows and (m, l)) in the
// workspace; the log-sum-exp merge then combines each sequence's parts.
//
// Work items are numbered group by group (prefix items first, then suffix
// items sequence by sequence); a persistent grid of resident workgroups walks
// them, HG waves (adjacent kv heads, reading each token as HG*D*2 contiguous
// bytes) per item, round by round, every other round in reverse.  The column blocks of one prefix partition are numbered
// next to each other and placed on the same XCD, so the second reads the
// shared rows from that XCD's L2.
#include "attention_bf16_wave.hpp"

#include <algorithm>

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
using wave::kStep;

// What every workgroup derives from the lengths and the groups.
struct Plan {
  int pscan[kMaxSharedGroups + 1];  // prefix items before group g
  int sscan[kMaxCompactSeqs + 1];   // suffix items before sequence s
  int glp[kMaxSharedGroups];        // prefix length of group g
  int lp[kMaxCompactSeqs];          // prefix length of s's group, -1 if s gives NaN
  int len[kMaxCompactSeqs];
  int wsum[kWaves];
  int bad;
  int16_t gs[kMaxSharedGroups + 1];  // group starts (checked to lie in [0, S])
  int16_t lead[kMaxCompactSeqs];     // first sequence of s's group
};

static_assert(sizeof(Plan) <= kSharedPlanInts * sizeof(int), "plan larger than budgeted");

// Exclusive scan of c(i), i < n <= 2 * kThreads, into out[0 .. n] (out[n]
// is the total).  c(i) may read out[i] (a scan in place): every c(i) is
// read before anything is written.
template <typename F>
__device__ __forceinline__ void block_scan(int n, int* out, int* wsum, F c) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int i0 = 2 * threadIdx.x;
  const int c0 = i0 < n ? c(i0) : 0;
  const int c1 = i0 + 1 < n ? c(i0 + 1) : 0;
  int v = c0 + c1;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    before += w < wv ? wsum[w] : 0;
    total += wsum[w];
  }
  const int excl = before + v - c0 - c1;
  __syncthreads();  // every c(i) has been read
  if (i0 < n) out[i0] = excl;
  if (i0 + 1 < n) out[i0 + 1] = excl + c0;
  if (threadIdx.x == 0) out[n] = total;
  __syncthreads();
}

// Last index i in [0, n) with v[i] <= x (v non-decreasing, v[0] <= x).
__device__ __forceinline__ int last_le(const int* v, int n, int x) {
  int lo = 0, up = n - 1;
  while (lo < up) {
    const int mid = (lo + up + 1) >> 1;
    if (v[mid] <= x) lo = mid; else up = mid - 1;
  }
  return lo;
}

template <int B>
__device__ __forceinline__ bool seq_ok(const AttnArgs& a, int L) {
  return L >= 0 && L <= a.max_len && (L + B - 1) / B <= a.width;
}

// The item list.  A group is valid when its starts run from 0 to S without
// decreasing and its prefix length is a multiple of the partition unit, fits
// the table and max_prefix and is no longer than any valid member; members
// of an invalid group, and invalid sequences, give NaN.  Workgroup 0 also
// records each sequence's parts, group leader and prefix for the merge.
template <int B>
__device__ void make_plan(const AttnArgs& a, Plan& p, int HGN, int chunks, int G) {
  constexpr int kUnit = B > 32 ? B : 32;  // partitions start on whole steps and blocks
  const int ng = a.num_groups, S = a.S, P = a.partition;
  if (threadIdx.x == 0) p.bad = 0;
  __syncthreads();
  for (int i = threadIdx.x; i <= ng; i += kThreads) {
    const int v = a.group_starts[i];
    if (v < 0 || v > S) p.bad = 1;
    p.gs[i] = static_cast<int16_t>(v);
  }
  for (int i = threadIdx.x; i < S; i += kThreads) p.len[i] = a.lens[i];
  __syncthreads();
  for (int i = threadIdx.x; i < ng; i += kThreads)
    if (p.gs[i] > p.gs[i + 1]) p.bad = 1;
  if (threadIdx.x == 0 && (p.gs[0] != 0 || p.gs[ng] != S)) p.bad = 1;
  __syncthreads();
  const bool all_bad = p.bad != 0;
  const bool rec = blockIdx.x == 0;

  // per group: its prefix items (into pscan, scanned below) and its members' prefix
  for (int g = threadIdx.x; g < ng; g += kThreads) {
    int count = 0;
    p.glp[g] = 0;
    if (!all_bad) {
      const int s0 = p.gs[g], s1 = p.gs[g + 1];
      const int lp = a.prefix_lens[g];
      p.glp[g] = lp;
      bool ok = lp >= 0 && lp <= a.max_prefix && lp % kUnit == 0 && (lp + B - 1) / B <= a.width;
      for (int s = s0; s < s1 && ok; ++s)
        if (seq_ok<B>(a, p.len[s]) && p.len[s] < lp) ok = false;
      for (int s = s0; s < s1; ++s) {
        const int L = p.len[s];
        const bool good = ok && seq_ok<B>(a, L);
        p.lp[s] = good ? lp : -1;
        p.lead[s] = s0;
        if (rec) {
          a.ws_seq[s] = good ? (lp + P - 1) / P + (L - lp + P - 1) / P : -1;
          a.ws_seq[S + s] = s0;
          a.ws_seq[2 * S + s] = good ? lp : 0;
        }
      }
      const int M = s1 - s0;
      if (ok && lp > 0 && M > 0) count = HGN * ((M * G + 15) / 16) * ((lp + P - 1) / P);
    }
    p.pscan[g] = count;
  }
  if (all_bad)
    for (int s = threadIdx.x; s < S; s += kThreads) {
      p.lp[s] = -1;
      p.lead[s] = s;
      if (rec) {
        a.ws_seq[s] = -1;
        a.ws_seq[S + s] = s;
        a.ws_seq[2 * S + s] = 0;
      }
    }
  __syncthreads();
  block_scan(ng, p.pscan, p.wsum, [&](int g) { return p.pscan[g]; });
  block_scan(S, p.sscan, p.wsum, [&](int s) {
    const int lp = p.lp[s];
    return lp < 0 ? 0 : HGN * chunks * ((p.len[s] - lp + P - 1) / P);
  });
}

template <int D, int B, int HG, bool NT, bool KL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
attention_bf16_shared_kernel(AttnArgs a) {
  using Wv = wave::Wave<D, B, NT, KL>;
  constexpr int SROW = Wv::SROW;
  constexpr int D4 = D / 4;
  constexpr int NSLOT = kWaves / HG;  // items a workgroup works on at once
  extern __shared__ float s_dyn[];
  __shared__ Plan p;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = wv % HG;    // kv head inside the group
  const int slot = wv / HG;  // which item of the workgroup
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  const int HGN = a.Hkv / HG;
  const int P = a.partition;
  const int ng = a.num_groups;
  make_plan<B>(a, p, HGN, chunks, G);
  const int t_pre = p.pscan[ng];
  const int total = t_pre + p.sscan[a.S];

  // Sequences s = blockIdx.x, + gridDim.x, ...: do s's own table entries for
  // its group's prefix match its leader's (whose table the prefix items
  // read)?  A mismatch makes the merge give NaN for s.
  if (wv == 0)
    for (int s = blockIdx.x; s < a.S; s += gridDim.x) {
      const int lp = p.lp[s], lead = p.lead[s];
      bool diff = false;
      if (lp > 0 && lead != s) {
        const int32_t* mine = a.tables + static_cast<int64_t>(s) * a.width;
        const int32_t* theirs = a.tables + static_cast<int64_t>(lead) * a.width;
        for (int i = lane; i < (lp + B - 1) / B; i += 64) diff = diff || mine[i] != theirs[i];
      }
      const bool any = __ballot(diff) != 0;
      if (lane == 0) a.ws_seq[3 * a.S + s] = any ? 1 : 0;
    }

  // Workgroup b runs on XCD b mod 8; with one item per workgroup, pair
  // workgroups b and b + 8 (same XCD) on consecutive items -- the column
  // blocks of one prefix partition.
  const int nwg = gridDim.x;
  int b = blockIdx.x;
  if (NSLOT == 1 && nwg % 16 == 0) b = (b / 16) * 16 + 2 * (b % 8) + (b / 8) % 2;

  // LDS of this wave: its K tile, then stream_slots finished results of 16
  // rows [hh][SROW], their (m, l) pairs, and where each goes
  const int K = a.stream_slots;
  float* wave_lds = s_dyn + static_cast<int64_t>(wv) * a.stream_wave_floats;
  float* rows = wave_lds + (KL ? wave::k_tile_floats(D) : 0);
  float* mls = rows + K * 16 * SROW;
  int* meta = reinterpret_cast<int*>(mls + 2 * K * 16);
  int used = 0;
  // row of the workspace holding column hh of a result: base + hh for a
  // suffix item; for a prefix item (col0 >= 0), column col0 + hh is member
  // (col0 + hh) / G and head (col0 + hh) % G of the kv head at base
  auto dest = [&](const int* m, int hh) -> int64_t {
    const int64_t base = (static_cast<int64_t>(m[0]) * a.S + m[1]) * a.Hq + m[2];
    if (m[3] < 0) return base + hh;
    const int c = m[3] + hh;
    const int mem = c / G;
    return base + static_cast<int64_t>(mem) * a.Hq + (c - mem * G);
  };
  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i < used; ++i) {
      const int* m = meta + kSharedMeta * i;
      const int nh = m[4];
      const float* r = rows + i * 16 * SROW;
      for (int e = lane; e < nh * D4; e += 64) {
        const int hh = e / D4;
        const int d = (e - hh * D4) * 4;
        *reinterpret_cast<float4*>(a.ws_o + dest(m, hh) * D + d) =
            *reinterpret_cast<const float4*>(r + hh * SROW + d);
      }
      if (lane < nh)
        *reinterpret_cast<float2*>(a.ws_ml + 2 * dest(m, lane)) =
            *reinterpret_cast<const float2*>(mls + 2 * (i * 16 + lane));
    }
    __builtin_amdgcn_wave_barrier();
    used = 0;
  };

  Wv w;
  w.init(a, reinterpret_cast<char*>(wave_lds));
  // Items are dealt out in rounds of one per item slot of the grid; odd
  // rounds are dealt in reverse, so the slots that drew the long prefix items
  // (which come first) draw the short items at the end of the next round.
  const int stride = nwg * NSLOT;
  for (int it0 = b * NSLOT + slot, round = 0; it0 < total + stride; it0 += stride, ++round) {
    const int it = (round & 1) ? (2 * round + 1) * stride - 1 - it0 : it0;
    if (it >= total) continue;
    int part, seq, kvh, hbase, t0, t1, nh, col0, tab;
    int64_t qrow;
    if (it < t_pre) {
      // prefix item: group g, kv-head group hgi, partition pp, column block cb
      const int g = last_le(p.pscan, ng, it);
      const int s0 = p.gs[g];
      const int M = p.gs[g + 1] - s0;
      const int lp = p.glp[g];
      const int CB = (M * G + 15) / 16;
      const int NP = (lp + P - 1) / P;
      const int local = it - p.pscan[g];
      const int cb = local % CB;
      const int r = local / CB;
      const int pp = r % NP;
      kvh = (r / NP) * HG + hi;
      hbase = kvh * G;
      col0 = 16 * cb;
      nh = min(16, M * G - col0);
      const int c = col0 + (lane & 15);
      const int mem = c / G;
      qrow = (lane & 15) < nh ? static_cast<int64_t>(s0 + mem) * a.Hq + kvh * G + (c - mem * G) : -1;
      tab = s0;
      seq = s0;
      part = pp;
      t0 = pp * P;
      t1 = min(lp, t0 + P);
    } else {
      // suffix item: sequence s, (kv-head group, query-head chunk) y, partition q
      const int x = it - t_pre;
      const int s = last_le(p.sscan, a.S, x);
      const int lp = p.lp[s];
      const int L = p.len[s];
      const int NQ = (L - lp + P - 1) / P;
      const int local = x - p.sscan[s];
      const int q = local % NQ;
      const int y = local / NQ;
      const int chunk = y % chunks;
      kvh = (y / chunks) * HG + hi;
      col0 = -1;
      nh = min(16, G - 16 * chunk);
      hbase = kvh * G + 16 * chunk;
      qrow = (lane & 15) < nh ? static_cast<int64_t>(s) * a.Hq + hbase + (lane & 15) : -1;
      tab = s;
      seq = s;
      part = (lp + P - 1) / P + q;
      t0 = lp + q * P;
      t1 = min(L, t0 + P);
    }

    if (used == K) flush();
    const int i = used++;
    w.begin_rows(a, qrow, tab, kvh, t0, t1);
    w.run((t1 - t0 + kStep - 1) / kStep, [](int) {});
    w.finish(rows + i * 16 * SROW, mls + 2 * i * 16, nh);
    if (lane == 0) {
      int* m = meta + kSharedMeta * i;
      m[0] = part;
      m[1] = seq;
      m[2] = hbase;
      m[3] = col0;
      m[4] = nh;
    }
  }
  flush();
}

template <int D, int B, int HG, bool NT, bool KL>
int launch_one(const AttnArgs& a, hipStream_t stream) {
  auto kern = attention_bf16_shared_kernel<D, B, HG, NT, KL>;
  if (const int rc = raise_lds_limit(reinterpret_cast<const void*>(kern))) return rc;
  const size_t lds = static_cast<size_t>(kWaves) * a.stream_wave_floats * sizeof(float);
  kern<<<dim3(a.stream_waves / kWaves), dim3(kThreads), lds, stream>>>(a);
  return check_launch("paged attention (bf16, shared prefix)");
}

template <int D, int B, int HG>
int launch_hg(const AttnArgs& a, hipStream_t stream) {
  const bool nt = a.nontemporal != 0, kl = a.k_via_lds != 0;
  if (nt) return kl ? launch_one<D, B, HG, true, true>(a, stream)
                    : launch_one<D, B, HG, true, false>(a, stream);
  return kl ? launch_one<D, B, HG, false, true>(a, stream)
            : launch_one<D, B, HG, false, false>(a, stream);
}

template <int D, int B>
int launch(const AttnArgs& a, hipStream_t stream) {
  const int HG = bf16_heads_per_group(a.Hkv);
  if (HG == 4) return launch_hg<D, B, 4>(a, stream);
  if (HG == 2) return launch_hg<D, B, 2>(a, stream);
  return launch_hg<D, B, 1>(a, stream);
}

}  // namespace

int launch_attention_bf16_shared(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0) return PKV_OK;
  if (static_cast<size_t>(kWaves) * a.stream_wave_floats * sizeof(float) > bf16_lds_limit()) {
    set_error("paged attention (bf16, shared prefix): too much LDS");
    return PKV_ERR_UNSUPPORTED;
  }
  switch (a.D * 1000 + a.B) {
    case 64008: return launch<64, 8>(a, stream);
    case 64016: return launch<64, 16>(a, stream);
    case 64032: return launch<64, 32>(a, stream);
    case 64064: return launch<64, 64>(a, stream);
    case 128008: return launch<128, 8>(a, stream);
    case 128016: return launch<128, 16>(a, stream);
    case 128032: return launch<128, 32>(a, stream);
    case 128064: return launch<128, 64>(a, stream);
    default: break;
  }
  set_error("paged attention (bf16, shared prefix): head_size %d with block_size %d is not built",
            a.D, a.B);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
