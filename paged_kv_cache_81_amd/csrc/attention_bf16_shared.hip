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
// Work items are numbered group by group for the prefix items, then sequence
// by sequence for the suffix items, longest suffix first; a persistent grid
// of resident workgroups walks them, HG waves (adjacent kv heads, reading
// each token as HG*D*2 contiguous bytes) per item, round by round, every
// other round in reverse, so the slots that drew the longest suffix items
// draw the shortest next.  Each wave keeps one 32-token step in flight.  The
// column blocks of one prefix partition are numbered next to each other and
// placed on the same XCD, so the second reads the shared rows from that
// XCD's L2.
//
// The item list depends only on the tables, lengths and groups, which every
// layer of a decode step shares.  So it can also be made once per step by a
// plan launch, which writes each item's description and first block-table
// window to a plan buffer; the attention launches given that plan skip the
// list's derivation and start each item's K/V loads one load after it is
// dealt.
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
  int bad;
  int16_t gs[kMaxSharedGroups + 1];  // group starts (checked to lie in [0, S])
  int16_t order[kMaxCompactSeqs];    // sequences by their own steps, longest first
};

static_assert(sizeof(Plan) <= kSharedPlanInts * sizeof(int), "plan larger than budgeted");

// Inclusive prefix sum over the wave's 64 lanes with DPP moves: shifts by 1,
// 2, 4, 8 lanes inside each row of 16, then the last lane of row 0 added to
// row 1 and of row 2 to row 3 (row_bcast:15), then lane 31 to rows 2 and 3
// (row_bcast:31).  A lane with no source lane adds 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// Exclusive scans over the workgroup of NV per-thread values at once (in
// thread order): v[n] becomes the sum of v[n] over the threads before this
// one, total[n] the sum over all.  wsum: NV * kWaves ints of LDS, free until
// the next barrier after the call.
template <int NV>
__device__ __forceinline__ void block_excl_scan(int (&v)[NV], int (&total)[NV], int* wsum) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int inc[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) inc[n] = wave_incl_scan(v[n]);
  if (lane == 63)
#pragma unroll
    for (int n = 0; n < NV; ++n) wsum[n * kWaves + wv] = inc[n];
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NV; ++n) {
    int before = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int x = wsum[n * kWaves + w];
      before += w < wv ? x : 0;
      sum += x;
    }
    v[n] = before + inc[n] - v[n];
    total[n] = sum;
  }
}

// Last index i in [0, n) with v[i] <= x (v non-decreasing, v[0] <= x).
template <typename T>
__device__ __forceinline__ int last_le(const T* v, int n, int x) {
  int lo = 0, up = n - 1;
  while (lo < up) {
    const int mid = (lo + up + 1) >> 1;
    if (v[mid] <= x) lo = mid; else up = mid - 1;
  }
  return lo;
}

// v / d for 0 <= v < 2^31, d >= 1 (rd = 1.0 / d): a double-precision
// estimate, then one step of correction either way
__device__ __forceinline__ int div_by(int v, int d, double rd) {
  int q = static_cast<int>(static_cast<double>(v) * rd);
  const int r = v - q * d;
  q += r >= d ? 1 : 0;
  q -= r < 0 ? 1 : 0;
  return q;
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
// Suffix items are listed by sequence, longest suffix first: a stable
// counting sort on the steps of each sequence's own tokens (capped), so every
// workgroup derives the same list.  Few barriers and dependent LDS reads: the
// plan is all a workgroup does before its first loads.
constexpr int kSortBins = 64;
constexpr int kSortChunks = kMaxCompactSeqs / 64;  // 64 sequences a chunk, one wave each
// scratch LDS: chunk histograms, group flags, item counts in sorted order,
// bin offsets, scan partials
constexpr int kPlanScratchInts =
    kSortChunks * kSortBins + kMaxSharedGroups + kMaxCompactSeqs + kSortBins + 2 * kWaves;

template <int B>
__device__ void make_plan(const AttnArgs& a, Plan& p, int HGN, int chunks, int G, int* scratch) {
  static_assert(kMaxCompactSeqs == 2 * kThreads && kMaxSharedGroups == 2 * kThreads &&
                kSortBins <= 2 * kThreads, "plan layout: two sequences and groups a thread");
  constexpr int kUnit = B > 32 ? B : 32;  // partitions start on whole steps and blocks
  const int ng = a.num_groups, S = a.S, P = a.partition;
  const double rP = 1.0 / P;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  int* hist = scratch;                         // [chunk][bin]: sequences of the chunk in the bin
  int* gbad = hist + kSortChunks * kSortBins;  // [group]: a valid member is shorter than the prefix
  int* cnt = gbad + kMaxSharedGroups;          // [rank]: suffix items of the rank's sequence
  int* boff = cnt + kMaxCompactSeqs;           // [bin]: sequences in earlier bins
  int* wsum = boff + kSortBins;

  // 1. inputs, in one round of loads; clear the flags and histograms
  bool bad = false;
  if (tid == 0) p.bad = 0;
  for (int i = tid; i < kSortChunks * kSortBins; i += kThreads) hist[i] = 0;
  for (int i = tid; i < ng; i += kThreads) gbad[i] = 0;
  for (int i = tid; i <= ng; i += kThreads) {
    const int v = a.group_starts[i];
    const int next = i < ng ? a.group_starts[i + 1] : S;
    bad = bad || v < 0 || v > S || v > next || (i == 0 && v != 0) || (i == ng && v != S);
    p.gs[i] = static_cast<int16_t>(v);
  }
  for (int i = tid; i < ng; i += kThreads) p.glp[i] = a.prefix_lens[i];
  for (int i = tid; i < S; i += kThreads) p.len[i] = a.lens[i];
  __syncthreads();

  // 2. each sequence s = tid + 256 j: its group (meaningless, but in range,
  // when the starts are bad) and whether it makes the group invalid
  if (bad) p.bad = 1;
  int grp[2], glen[2], len[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = tid + j * kThreads;
    grp[j] = 0;
    glen[j] = -1;
    len[j] = 0;
    if (s < S) {
      grp[j] = last_le(p.gs, ng, s);
      glen[j] = p.glp[grp[j]];
      len[j] = p.len[s];
      if (seq_ok<B>(a, len[j]) && len[j] < glen[j]) gbad[grp[j]] = 1;
    }
  }
  __syncthreads();

  // 3. prefixes, item counts, sort keys; groups g = 2 tid + e
  const bool all_bad = p.bad != 0;
  const bool rec = blockIdx.x == 0;
  auto group_ok = [&](int g, int lp) {
    return !all_bad && gbad[g] == 0 && lp >= 0 && lp <= a.max_prefix && lp % kUnit == 0 &&
           (lp + B - 1) / B <= a.width;
  };
  const uint64_t below = (uint64_t{1} << lane) - 1;
  int items[2], bin[2], pos[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = tid + j * kThreads;
    const int L = len[j];
    const int lp = s < S && group_ok(grp[j], glen[j]) && seq_ok<B>(a, L) ? glen[j] : -1;
    if (s < S) {
      p.lp[s] = lp;
      if (rec) {
        a.ws_seq[s] = lp >= 0 ? div_by(lp + P - 1, P, rP) + div_by(L - lp + P - 1, P, rP) : -1;
        a.ws_seq[S + s] = all_bad ? s : p.gs[grp[j]];
        a.ws_seq[2 * S + s] = lp >= 0 ? lp : 0;
      }
    }
    items[j] = lp < 0 ? 0 : HGN * chunks * div_by(L - lp + P - 1, P, rP);
    const int key = lp < 0 ? 0 : min((L - lp + kStep - 1) / kStep, kSortBins - 1);
    // sequence s lies in chunk s / 64, lane s % 64; the lanes of its bin come
    // from a ballot per bit of the bin
    bin[j] = kSortBins - 1 - key;
    uint64_t same = __ballot(s < S);
#pragma unroll
    for (int bit = 1; bit < kSortBins; bit <<= 1) {
      const uint64_t m = __ballot((bin[j] & bit) != 0);
      same &= (bin[j] & bit) ? m : ~m;
    }
    pos[j] = __popcll(same & below);
    if (s < S && pos[j] == 0) hist[(s >> 6) * kSortBins + bin[j]] = __popcll(same);
  }
  int sc[2] = {0, 0};  // scanned: prefix items of groups 2 tid, 2 tid + 1; sequences in bins 2 tid, 2 tid + 1
  int pre[2] = {0, 0};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int g = 2 * tid + e;
    if (g < ng) {
      const int s0 = p.gs[g], M = p.gs[g + 1] - s0, lp = p.glp[g];
      if (group_ok(g, lp) && lp > 0 && M > 0)
        pre[e] = HGN * ((M * G + 15) / 16) * div_by(lp + P - 1, P, rP);
    }
  }
  __syncthreads();

  // 4. scans of the groups' prefix items and of the bins' sizes
  int bsz[2] = {0, 0};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int k = 2 * tid + e;
    if (k < kSortBins)
#pragma unroll
      for (int c = 0; c < kSortChunks; ++c) bsz[e] += hist[c * kSortBins + k];
  }
  int v2[2] = {pre[0] + pre[1], bsz[0] + bsz[1]}, tot2[2];
  block_excl_scan<2>(v2, tot2, wsum);
  if (2 * tid < ng) p.pscan[2 * tid] = v2[0];
  if (2 * tid + 1 < ng) p.pscan[2 * tid + 1] = v2[0] + pre[0];
  if (tid == 0) p.pscan[ng] = tot2[0];
  if (2 * tid < kSortBins) boff[2 * tid] = v2[1];
  if (2 * tid + 1 < kSortBins) boff[2 * tid + 1] = v2[1] + bsz[0];
  __syncthreads();

  // 5. rank of each sequence: earlier bins, then earlier chunks of its bin,
  // then lower lanes of its chunk
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = tid + j * kThreads;
    if (s < S) {
      int r = boff[bin[j]] + pos[j];
      for (int c = 0; c < (s >> 6); ++c) r += hist[c * kSortBins + bin[j]];
      p.order[r] = static_cast<int16_t>(s);
      cnt[r] = items[j];
    }
  }
  __syncthreads();

  // 6. suffix items before each rank
  const int c0 = 2 * tid < S ? cnt[2 * tid] : 0;
  const int c1 = 2 * tid + 1 < S ? cnt[2 * tid + 1] : 0;
  int v1[1] = {c0 + c1}, tot1[1];
  block_excl_scan<1>(v1, tot1, wsum);
  if (2 * tid < S) p.sscan[2 * tid] = v1[0];
  if (2 * tid + 1 < S) p.sscan[2 * tid + 1] = v1[0] + c0;
  if (tid == 0) p.sscan[S] = tot1[0];
  __syncthreads();
}

// One work item, for all HG kv heads of its group (each wave of the item
// adds its own head to kvg).
struct Item {
  int part;   // partition number of the results in its sequences' workspace rows
  int seq;    // prefix item: the group's first sequence (its table is read); suffix item: the sequence
  int kvg;    // first kv head of the item's group of HG
  int col0;   // prefix item: first score column (member col0 / G, head col0 % G); suffix item: -1
  int nh;     // score columns (query heads) of the item
  int t0, t1; // tokens read
  int chunk;  // suffix item: the query heads 16 chunk .. of each kv head
};
static_assert(sizeof(Item) == kPlanItemFields * sizeof(int), "plan item record layout");

// Item it of the list the plan p describes (t_pre prefix items first).
__device__ __forceinline__ Item decode_item(const AttnArgs& a, const Plan& p, int it, int t_pre,
                                            int HG, int G, int chunks) {
  const int P = a.partition;
  Item m;
  if (it < t_pre) {
    // prefix item: group g, kv-head group, partition pp, column block cb
    const int g = last_le(p.pscan, a.num_groups, it);
    const int s0 = p.gs[g];
    const int M = p.gs[g + 1] - s0;
    const int lp = p.glp[g];
    const int CB = (M * G + 15) / 16;
    const int NP = (lp + P - 1) / P;
    const int local = it - p.pscan[g];
    const int cb = local % CB;
    const int r = local / CB;
    const int pp = r % NP;
    m.part = pp;
    m.seq = s0;
    m.kvg = (r / NP) * HG;
    m.col0 = 16 * cb;
    m.nh = min(16, M * G - m.col0);
    m.t0 = pp * P;
    m.t1 = min(lp, m.t0 + P);
    m.chunk = 0;
  } else {
    // suffix item: sequence s, (kv-head group, query-head chunk) y, partition q
    const int x = it - t_pre;
    const int k = last_le(p.sscan, a.S, x);
    const int s = p.order[k];
    const int lp = p.lp[s];
    const int L = p.len[s];
    const int NQ = (L - lp + P - 1) / P;
    const int local = x - p.sscan[k];
    const int q = local % NQ;
    const int y = local / NQ;
    m.chunk = y % chunks;
    m.part = (lp + P - 1) / P + q;
    m.seq = s;
    m.kvg = (y / chunks) * HG;
    m.col0 = -1;
    m.nh = min(16, G - 16 * m.chunk);
    m.t0 = lp + q * P;
    m.t1 = min(L, m.t0 + P);
  }
  return m;
}

// Sequences s = blockIdx.x, + nwg, ... (wave 0 of each workgroup): do s's
// own table entries for its group's prefix match its leader's (whose table
// the prefix items read)?  A mismatch makes the merge give NaN for s.
template <int B>
__device__ __forceinline__ void check_prefix_tables(const AttnArgs& a, const Plan& p, int nwg,
                                                    int lane) {
  for (int s = blockIdx.x; s < a.S; s += nwg) {
    const int lp = p.lp[s];
    // s's group (valid groups have non-decreasing starts): its leader
    const int lead = lp > 0 ? p.gs[last_le(p.gs, a.num_groups, s)] : s;
    bool diff = false;
    if (lp > 0 && lead != s) {
      const int32_t* mine = a.tables + static_cast<int64_t>(s) * a.width;
      const int32_t* theirs = a.tables + static_cast<int64_t>(lead) * a.width;
      for (int i = lane; i < (lp + B - 1) / B; i += 64) diff = diff || mine[i] != theirs[i];
    }
    const bool any = __ballot(diff) != 0;
    if (lane == 0) a.ws_seq[3 * a.S + s] = any ? 1 : 0;
  }
}

// The plan launch: every workgroup makes the plan (as the attention
// workgroups do without one), workgroup 0 records the header and the
// sequences' records for the merge (a.ws_seq points into the plan), each
// workgroup checks its share of the sequences' prefix tables and records its
// share of the items, one a wave at a time.  nwg = a.stream_waves / 4.
template <int B>
__global__ void __launch_bounds__(kThreads)
shared_plan_kernel(AttnArgs a, int32_t* plan, int64_t capacity) {
  __shared__ Plan p;
  __shared__ int scratch[kPlanScratchInts];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  const int HG = bf16_heads_per_group(a.Hkv);
  const int nwg = a.stream_waves / kWaves;
  make_plan<B>(a, p, a.Hkv / HG, chunks, G, scratch);
  const int t_pre = p.pscan[a.num_groups];
  const int total = t_pre + p.sscan[a.S];
  const bool fits = total <= capacity;
  if (blockIdx.x == 0 && threadIdx.x < kPlFields) {
    const int f = threadIdx.x;
    const int v = f == kPlMagic ? kPlanMagic : f == kPlS ? a.S : f == kPlHq ? a.Hq :
                  f == kPlHkv ? a.Hkv : f == kPlB ? a.B : f == kPlWidth ? a.width :
                  f == kPlMaxLen ? a.max_len : f == kPlMaxPrefix ? a.max_prefix :
                  f == kPlGroups ? a.num_groups : f == kPlPartition ? a.partition :
                  f == kPlStatus ? (fits ? 0 : 1) : f == kPlPrefixItems ? t_pre : total;
    plan[f] = v;
  }
  if (wv == 0) check_prefix_tables<B>(a, p, nwg, lane);
  if (!fits) return;
  int32_t* items = plan + plan_items_off(a.S);
  for (int it = blockIdx.x * kWaves + wv; it < total; it += nwg * kWaves) {
    const Item m = decode_item(a, p, it, t_pre, HG, G, chunks);
    int32_t* r = items + static_cast<int64_t>(it) * kPlanItemInts;
    if (lane < kPlanItemFields)
      r[lane] = lane == 0 ? m.part : lane == 1 ? m.seq : lane == 2 ? m.kvg : lane == 3 ? m.col0 :
                lane == 4 ? m.nh : lane == 5 ? m.t0 : lane == 6 ? m.t1 : m.chunk;
    r[kPlanItemFields + lane] =
        wave::table_window<B>(a.tables + static_cast<int64_t>(m.seq) * a.width, m.t0, m.t1, 0, lane);
  }
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
  // the plan's scratch lies in the dynamic LDS (at least one result slot a wave)
  static_assert(kPlanScratchInts <= kWaves * 16 * (D + 4), "plan scratch exceeds dynamic LDS");

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = wv % HG;    // kv head inside the group
  const int slot = wv / HG;  // which item of the workgroup
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  const int HGN = a.Hkv / HG;
  const int ng = a.num_groups;
  // the grid's size from the arguments (read with the others at the start),
  // not from the dispatch's hidden arguments
  const int nwg = a.stream_waves / kWaves;
  // Workgroup b runs on XCD b mod 8; with one item per workgroup, pair
  // workgroups b and b + 8 (same XCD) on consecutive items -- the column
  // blocks of one prefix partition.
  int b = blockIdx.x;
  if (NSLOT == 1 && nwg % 16 == 0) b = (b / 16) * 16 + 2 * (b % 8) + (b / 8) % 2;
  const int it_first = b * NSLOT + slot;  // this wave's item of the first round

  // With a plan: its item counts (none if it was made for other arguments:
  // the merge then gives NaN), and its item records.  Without: make it.
  const bool planned = a.plan != nullptr;
  const int32_t* items = planned ? a.plan + plan_items_off(a.S) : nullptr;
  // the record of the first round's item (see the item loop), loaded with
  // the header: any record below the capacity lies in the plan buffer
  int first_f = 0, first_win = 0;
  if (planned && it_first < a.plan_capacity) {
    const int32_t* r = items + static_cast<int64_t>(it_first) * kPlanItemInts;
    first_f = r[lane % kPlanItemFields];
    first_win = r[kPlanItemFields + lane];
  }
  int t_pre, total;
  if (planned) {
    const int n_pre = a.plan[kPlPrefixItems];
    const int n_all = a.plan[kPlItems];
    const bool ok = plan_matches(a);
    t_pre = __builtin_amdgcn_readfirstlane(ok ? n_pre : 0);
    total = __builtin_amdgcn_readfirstlane(ok ? n_all : 0);
    // the sequences' records for the merge, from the plan into the
    // workspace (a record written this late is still in the caches when the
    // merge reads it); parts -1 (NaN rows) when the plan does not match
    if (wv == 0) {
      const int32_t* rec = a.plan + kPlanHeaderInts;
      for (int s = blockIdx.x * 64 + lane; s < a.S; s += nwg * 64)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int v = rec[f * a.S + s];
          a.ws_seq[f * a.S + s] = ok ? v : (f == 0 ? -1 : 0);
        }
    }
  } else {
    make_plan<B>(a, p, HGN, chunks, G, reinterpret_cast<int*>(s_dyn));
    t_pre = p.pscan[ng];
    total = t_pre + p.sscan[a.S];
    if (wv == 0) check_prefix_tables<B>(a, p, nwg, lane);
  }

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
  for (int it0 = it_first, round = 0; it0 < total + stride; it0 += stride, ++round) {
    const int it = (round & 1) ? (2 * round + 1) * stride - 1 - it0 : it0;
    if (it >= total) continue;
    Item m;
    int win0 = 0;
    if (planned) {
      // the record in two loads issued together: lane l takes field l % 8
      // of the description and entry l of the table window (the first
      // round's, it == it_first, are loaded already)
      int f = first_f;
      win0 = first_win;
      if (round > 0) {
        const int32_t* r = items + static_cast<int64_t>(it) * kPlanItemInts;
        f = r[lane % kPlanItemFields];
        win0 = r[kPlanItemFields + lane];
      }
      m.part = __builtin_amdgcn_readlane(f, 0);
      m.seq = __builtin_amdgcn_readlane(f, 1);
      m.kvg = __builtin_amdgcn_readlane(f, 2);
      m.col0 = __builtin_amdgcn_readlane(f, 3);
      m.nh = __builtin_amdgcn_readlane(f, 4);
      m.t0 = __builtin_amdgcn_readlane(f, 5);
      m.t1 = __builtin_amdgcn_readlane(f, 6);
      m.chunk = __builtin_amdgcn_readlane(f, 7);
    } else {
      m = decode_item(a, p, it, t_pre, HG, G, chunks);
    }
    // this wave's kv head, its first query head, and the query row of score
    // column lane % 16 (-1: none)
    const int kvh = m.kvg + hi;
    const int jc = lane & 15;
    int hbase;
    int64_t qrow = -1;
    if (m.col0 >= 0) {
      hbase = kvh * G;
      const int c = m.col0 + jc;
      const int mem = c / G;
      if (jc < m.nh) qrow = static_cast<int64_t>(m.seq + mem) * a.Hq + hbase + (c - mem * G);
    } else {
      hbase = kvh * G + 16 * m.chunk;
      if (jc < m.nh) qrow = static_cast<int64_t>(m.seq) * a.Hq + hbase + jc;
    }

    if (used == K) flush();
    const int i = used++;
    if (planned) w.begin_rows(a, qrow, m.seq, kvh, m.t0, m.t1, win0);
    else w.begin_rows(a, qrow, m.seq, kvh, m.t0, m.t1);
    w.run_single((m.t1 - m.t0 + kStep - 1) / kStep, [](int) {});
    w.finish(rows + i * 16 * SROW, mls + 2 * i * 16, m.nh);
    if (lane == 0) {
      int* md = meta + kSharedMeta * i;
      md[0] = m.part;
      md[1] = m.seq;
      md[2] = hbase;
      md[3] = m.col0;
      md[4] = m.nh;
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

int launch_shared_plan(const AttnArgs& a, int32_t* plan, int64_t capacity, hipStream_t stream) {
  if (a.S == 0) return PKV_OK;
  const dim3 grid(a.stream_waves / kWaves), block(kThreads);
  switch (a.B) {
    case 8: shared_plan_kernel<8><<<grid, block, 0, stream>>>(a, plan, capacity); break;
    case 16: shared_plan_kernel<16><<<grid, block, 0, stream>>>(a, plan, capacity); break;
    case 32: shared_plan_kernel<32><<<grid, block, 0, stream>>>(a, plan, capacity); break;
    case 64: shared_plan_kernel<64><<<grid, block, 0, stream>>>(a, plan, capacity); break;
    default:
      set_error("shared-prefix plan: block_size %d is not built", a.B);
      return PKV_ERR_UNSUPPORTED;
  }
  return check_launch("shared-prefix plan");
}

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
