// Paged decode attention for bf16 caches on gfx950 matrix cores: the two
// ways of dividing the work among waves.  The per-wave arithmetic (table
// walk, MFMA scores, online softmax, P.V) is in attention_bf16_wave.hpp.
//
// Stream schedule (automatic partitioning, batches of up to 1024 sequences).
// The work is the list of (sequence s, group of HG kv heads, query-head chunk)
// pairs, each a run of cdiv(L_s, 32) steps, laid end to end in pair order.  A
// persistent grid of one round of resident workgroups cuts this stream into
// equal contiguous pieces, 4/HG per workgroup, each read by HG waves (one kv
// head each, walking the same tokens), so every wave -- and every CU -- reads
// the same number of K/V bytes whatever the mix of context lengths.  A pair
// lying inside one piece is finished there and written to out; a pair cut
// into several pieces leaves one partial result per piece in consecutive
// workspace slots, combined afterwards by the log-sum-exp merge.
//
// Fixed partitions (an explicit partition size, or larger batches): a
// workgroup of 4 waves covers HG consecutive kv heads x 4/HG runs of
// partitions.  The HG waves of a group walk the same tokens together, so
// each cached row is read as HG*D*2 contiguous bytes.  Workgroups are a dense
// grid (x = partition run, y = kv-head group and query-head chunk, z =
// sequence), or, when most of that grid would be empty (ragged batches split
// into several runs), a compact list of the real work items.
#include "attention_bf16_wave.hpp"

#include <algorithm>
#include <mutex>

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;  // accelerator complexes (each with its own L2) of an MI355X
using wave::kStep;

// ---------------------------------------------------------------- fixed partitions

template <int D, int B, int HG, bool NT, bool KL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
attention_bf16_kernel(AttnArgs a) {
  using Wv = wave::Wave<D, B, NT, KL>;
  constexpr int SROW = Wv::SROW;
  constexpr int NSLOT = kWaves / HG;  // waves per kv head, each on its own partitions
  // Finished partitions stay in LDS until the wave has read its last K/V:
  // a global store issued between the loads would make the following waits
  // for those loads also wait for the store to be acknowledged.
  extern __shared__ float s_dyn[];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = wv % HG;    // kv head inside the group
  const int slot = wv / HG;  // which run of partitions

  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  const int Y = (a.Hkv / HG) * chunks;  // (kv-head group, query-head chunk) pairs
  const int P = a.partition;

  // Compact list: the items of all sequences are numbered consecutively --
  // sequence, then pair, then run -- and workgroup b takes items b,
  // b + gridDim.x, ...  Dense grid with ranking: the lengths.
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

  const int pps = a.parts_per_wg / NSLOT;  // partitions per wave run
  const int nhs = min(16, G);              // head rows per partition slot
  // LDS of this wave: its K tile, then rows [i][hh][SROW] of its i-th
  // finished partition, then their (m, l) pairs
  float* wave_lds = s_dyn + static_cast<int64_t>(wv) * bf16_lds_wave_floats(pps, G, D, KL);
  float* stage = wave_lds + (KL ? wave::k_tile_floats(D) : 0);
  float* stage_ml = stage + pps * nhs * SROW;  // 16-byte aligned: SROW % 4 == 0

  Wv w;
  w.init(a, reinterpret_cast<char*>(wave_lds));

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
    const int p_first = xr * a.parts_per_wg + slot * pps;
    if (p_first >= nparts) return;  // (partition 0 always exists)

    // partition p_first + i: the normalised output (single partition) into
    // out, else the partial output and (m, l) into the workspace, whose
    // layout [s][p][h][D] keeps a wave's heads adjacent
    auto store = [&](int i) {
      const int64_t row0 = single ? static_cast<int64_t>(s) * a.Hq + h0
                                  : (static_cast<int64_t>(s) * a.max_parts + p_first + i) * a.Hq + h0;
      wave::store_rows<D>(a, stage + i * nhs * SROW, stage_ml + 2 * i * nhs, nh, row0, single, lane);
    };

    if (bad_seq) {
      // the merge kernel poisons split sequences itself
      if (single) {
        for (int i = lane; i < nh * SROW; i += 64) stage[i] = NAN;
        __builtin_amdgcn_wave_barrier();
        store(0);
      }
      return;
    }

    const int t0 = p_first * P;
    const int t1 = min(L, (p_first + pps) * P);
    const int nsteps = (t1 - t0 + kStep - 1) / kStep;  // 0 only when L == 0
    w.begin(a, s, kvh, h0, nh, t0, t1);
    w.run(nsteps, [&](int q) {
      const int ts = t0 + q * kStep;
      if (q > 0 && ts % P == 0) {  // a new partition starts here
        const int i = ts / P - 1 - p_first;
        w.finish(stage + i * nhs * SROW, stage_ml + 2 * i * nhs, nh);
      }
    });
    // the last partition (or, for an empty sequence, its zero output)
    const int i_last = nsteps > 0 ? (t0 + (nsteps - 1) * kStep) / P - p_first : 0;
    w.finish(stage + i_last * nhs * SROW, stage_ml + 2 * i_last * nhs, nh);
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i <= i_last; ++i) store(i);
  };

  if (!a.compact) {
    item(s_dense, blockIdx.y, blockIdx.x);
    return;
  }
  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    // the sequence whose items contain it: the last s with s_seq[s] <= it
    int lo = 0, up = a.S - 1;
    while (lo < up) {
      const int mid = (lo + up + 1) >> 1;
      if (s_seq[mid] <= it) lo = mid; else up = mid - 1;
    }
    const int nruns = (s_seq[lo + 1] - s_seq[lo]) / Y;
    const int local = it - s_seq[lo];
    const int yy = local / nruns;
    item(lo, yy, local - yy * nruns);
    // the wave's LDS is reused by the next item: finish reading it first
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------- stream schedule

// (resident workgroups per CU as stream_wgs_per_cu assumes: 3 for head size
// 64, 2 for 128)
template <int D, int B, int HG, bool NT, bool KL>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2)))
attention_bf16_stream_kernel(AttnArgs a) {
  using Wv = wave::Wave<D, B, NT, KL>;
  constexpr int SROW = Wv::SROW;
  constexpr int NSLOT = kWaves / HG;               // pieces per workgroup
  constexpr int PER = kMaxStreamSeqs / kThreads;  // sequences per thread in the scan
  extern __shared__ float s_dyn[];
  __shared__ int s_pref[kMaxStreamSeqs + 1];  // first stream step of each sequence
  __shared__ int s_wsum[kWaves];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = wv % HG;    // kv head inside the group
  const int slot = wv / HG;  // which piece of the workgroup
  const int G = a.Hq / a.Hkv;
  const int chunks = (G + 15) >> 4;
  // stream pairs per sequence: (group of HG kv heads, query-head chunk)
  const int Y = (a.Hkv / HG) * chunks;
  const int nhs = min(16, G);

  // Steps of sequence s per pair: cdiv(L, 32), and one step for an empty
  // sequence (zero output) or an invalid one (NaN output).  Exclusive scan of
  // Y times that over the batch.
  {
    int c[PER];
    int tot = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = threadIdx.x * PER + k;
      int n = 0;
      if (i < a.S) {
        const int L = a.lens[i];
        const bool bad = L < 0 || L > a.max_len || (L + B - 1) / B > a.width;
        n = (bad || L == 0) ? 1 : (L + kStep - 1) / kStep;
      }
      c[k] = Y * n;
      tot += c[k];
    }
    int v = tot;  // inclusive scan over the wave's lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(v, d, 64);
      if (lane >= d) v += t;
    }
    if (lane == 63) s_wsum[wv] = v;
    __syncthreads();
    int e = v - tot, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      e += w < wv ? s_wsum[w] : 0;
      total += s_wsum[w];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = threadIdx.x * PER + k;
      if (i < a.S) s_pref[i] = e;
      e += c[k];
    }
    if (threadIdx.x == 0) s_pref[a.S] = total;
    __syncthreads();
  }

  // the merge kernel locates the pieces of each unit from the same prefix
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.S; i += kThreads) a.ws_pref[i] = s_pref[i];

  // This piece of the stream: steps [x, x_end), read by the HG waves of the
  // workgroup with the same slot, one kv head each.  Workgroup b runs on XCD
  // b mod 8, so pieces are numbered XCD by XCD: each XCD reads one contiguous
  // eighth of the stream, and sequences adjacent in the batch (such as forks
  // sharing a prompt's blocks) share its L2.
  const int nwg = gridDim.x;
  const int wg = (nwg % kXcds == 0) ? (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds
                                    : static_cast<int>(blockIdx.x);
  const int piece = wg * NSLOT + slot;
  const int npieces = nwg * NSLOT;
  int x = stream_piece_start(piece, s_pref[a.S], npieces);
  const int x_end = stream_piece_start(piece + 1, s_pref[a.S], npieces);

  // LDS of this wave: its K tile, then a.stream_slots result slots of nhs
  // rows [hh][SROW], their (m, l) pairs, and per slot where it goes
  // (destination row, heads, whole unit?)
  const int K = a.stream_slots;
  float* wave_lds = s_dyn + static_cast<int64_t>(wv) * a.stream_wave_floats;
  float* rows = wave_lds + (KL ? wave::k_tile_floats(D) : 0);
  float* mls = rows + K * nhs * SROW;
  int* meta = reinterpret_cast<int*>(mls + 2 * K * nhs);
  int used = 0;
  // whole units go to out, pieces of cut units to the workspace
  auto flush = [&]() {
    __builtin_amdgcn_wave_barrier();
    for (int i = 0; i < used; ++i) {
      const int* m = meta + kStreamMeta * i;
      wave::store_rows<D>(a, rows + i * nhs * SROW, mls + 2 * i * nhs, m[1], m[0], m[2] != 0, lane);
    }
    __builtin_amdgcn_wave_barrier();
    used = 0;
  };
  Wv w;
  w.init(a, reinterpret_cast<char*>(wave_lds));
  while (x < x_end) {
    // the sequence holding step x: the last s with s_pref[s] <= x
    int lo = 0, up = a.S - 1;
    while (lo < up) {
      const int mid = (lo + up + 1) >> 1;
      if (s_pref[mid] <= x) lo = mid; else up = mid - 1;
    }
    const int s = lo;
    const int n = (s_pref[s + 1] - s_pref[s]) / Y;  // steps of each pair of s
    const int local = x - s_pref[s];
    const int y = local / n;
    const int st0 = local - y * n;
    const int st1 = min(n, st0 + (x_end - x));
    const bool whole = st0 == 0 && st1 == n;  // the pair lies inside this piece
    const int hg = y / chunks;
    const int chunk = y - hg * chunks;
    const int kvh = hg * HG + hi;
    const int nh = min(16, G - chunk * 16);
    const int h0 = kvh * G + chunk * 16;

    if (used == K) flush();
    const int i = used++;
    float* srow = rows + i * nhs * SROW;
    float* sml = mls + 2 * i * nhs;
    const int L = a.lens[s];
    if (L < 0 || L > a.max_len || (L + B - 1) / B > a.width) {
      // an invalid sequence is one step, so always whole: NaN output
      for (int e = lane; e < nh * SROW; e += 64) srow[e] = NAN;
    } else {
      const int t0 = st0 * kStep;
      const int t1 = min(L, st1 * kStep);
      w.begin(a, s, kvh, h0, nh, t0, t1);
      w.run((t1 - t0 + kStep - 1) / kStep, [](int) {});
      w.finish(srow, sml, nh);
    }
    // whole pairs go to out; a piece of a cut pair goes to workspace slot
    // piece + (pair index), distinct for every piece of the stream, whose
    // rows are [kv head in the group][query head]
    if (lane == 0) {
      int* m = meta + kStreamMeta * i;
      m[0] = whole ? s * a.Hq + h0 : ((piece + s * Y + y) * HG + hi) * nhs;
      m[1] = nh;
      m[2] = whole ? 1 : 0;
    }
    x += st1 - st0;
  }
  flush();

}

// ---------------------------------------------------------------- launchers

template <typename K>
int raise_lds_limit(K kern) {
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(bf16_lds_limit())) != hipSuccess) {
    set_error("paged attention (bf16): cannot raise the LDS limit");
    return PKV_ERR_HIP;
  }
  return PKV_OK;
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
    if (const int rc = raise_lds_limit(kern)) return rc;
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

template <int D, int B, int HG, bool NT, bool KL>
int launch_stream_one(const AttnArgs& a, hipStream_t stream) {
  auto kern = attention_bf16_stream_kernel<D, B, HG, NT, KL>;
  static bool attr_set = false;
  if (!attr_set) {
    if (const int rc = raise_lds_limit(kern)) return rc;
    attr_set = true;
  }
  const size_t lds = static_cast<size_t>(kWaves) * a.stream_wave_floats * sizeof(float);
  kern<<<dim3(a.stream_waves / kWaves), dim3(kThreads), lds, stream>>>(a);
  return check_launch("paged attention (bf16, stream schedule)");
}

template <int D, int B, int HG>
int launch_stream_hg(const AttnArgs& a, hipStream_t stream) {
  const bool nt = a.nontemporal != 0, kl = a.k_via_lds != 0;
  if (nt) return kl ? launch_stream_one<D, B, HG, true, true>(a, stream)
                    : launch_stream_one<D, B, HG, true, false>(a, stream);
  return kl ? launch_stream_one<D, B, HG, false, true>(a, stream)
            : launch_stream_one<D, B, HG, false, false>(a, stream);
}

template <int D, int B>
int launch_stream(const AttnArgs& a, hipStream_t stream) {
  const int HG = bf16_heads_per_group(a.Hkv);
  if (HG == 4) return launch_stream_hg<D, B, 4>(a, stream);
  if (HG == 2) return launch_stream_hg<D, B, 2>(a, stream);
  return launch_stream_hg<D, B, 1>(a, stream);
}

}  // namespace

int launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0) return PKV_OK;
  if (a.stream) {
    if (static_cast<size_t>(kWaves) * a.stream_wave_floats * sizeof(float) > bf16_lds_limit()) {
      set_error("paged attention (bf16): the stream schedule needs too much LDS");
      return PKV_ERR_UNSUPPORTED;
    }
    switch (a.D * 1000 + a.B) {
      case 64016: return launch_stream<64, 16>(a, stream);
      case 64032: return launch_stream<64, 32>(a, stream);
      case 64064: return launch_stream<64, 64>(a, stream);
      case 128016: return launch_stream<128, 16>(a, stream);
      case 128032: return launch_stream<128, 32>(a, stream);
      case 128064: return launch_stream<128, 64>(a, stream);
      default: break;
    }
  } else {
    switch (a.D * 1000 + a.B) {
      case 64016: return launch<64, 16>(a, stream);
      case 64032: return launch<64, 32>(a, stream);
      case 64064: return launch<64, 64>(a, stream);
      case 128016: return launch<128, 16>(a, stream);
      case 128032: return launch<128, 32>(a, stream);
      case 128064: return launch<128, 64>(a, stream);
      default: break;
    }
  }
  set_error("paged attention (bf16): head_size %d with block_size %d is not built", a.D, a.B);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
