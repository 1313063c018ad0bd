// Paged decode attention for bf16 caches on gfx950 matrix cores, fixed
// partitions (an explicit partition size, or batches whose (sequence,
// kv-head group) units fill the GPU, read whole).  The per-wave arithmetic
// (table walk, MFMA scores, online softmax, P.V) is in attention_bf16_wave.hpp;
// the balanced stream schedule in attention_bf16_stream.hip.
//
// A workgroup of 4 waves covers HG consecutive kv heads x 4/HG runs of
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

template <int D, int B, int HG, bool NT, bool KL, bool CMP>
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
  if constexpr (CMP) {
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
  int y_dense = blockIdx.y;
  int x_dense = blockIdx.x;
  if (!CMP && a.xcd_blocked) {
    // Workgroup b (in dispatch order) runs on XCD b mod 8: renumber so that
    // XCD i takes the i-th contiguous eighth of the (sequence, pair, run)
    // items, and sequences adjacent in the batch -- forks that share a
    // prompt's blocks -- read them through one L2.
    const int64_t n = static_cast<int64_t>(gridDim.x) * gridDim.y * gridDim.z;
    const int64_t b = blockIdx.x + static_cast<int64_t>(gridDim.x) * (blockIdx.y + static_cast<int64_t>(gridDim.y) * blockIdx.z);
    const int64_t q = n / kXcds, r = n % kXcds;
    const int64_t xcd = b % kXcds;
    const int64_t item = xcd * q + min(xcd, r) + b / kXcds;
    x_dense = static_cast<int>(item % gridDim.x);
    y_dense = static_cast<int>((item / gridDim.x) % gridDim.y);
    s_dense = static_cast<int>(item / (static_cast<int64_t>(gridDim.x) * gridDim.y));
  }
  if (!CMP && a.longest_first) {
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
      if (rank == s_dense) s_pick = c;
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

  if constexpr (!CMP) {
    item(s_dense, y_dense, x_dense);
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

// ---------------------------------------------------------------- launchers

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

template <int D, int B, int HG, bool NT, bool KL, bool CMP>
int launch_one(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
  auto kern = attention_bf16_kernel<D, B, HG, NT, KL, CMP>;
  if (const int rc = raise_lds_limit(reinterpret_cast<const void*>(kern))) return rc;
  if constexpr (CMP) {
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

template <int D, int B, int HG, bool CMP>
int launch_cmp(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
  const bool nt = a.nontemporal != 0, kl = a.k_via_lds != 0;
  if (nt) return kl ? launch_one<D, B, HG, true, true, CMP>(a, grid, lds, stream)
                    : launch_one<D, B, HG, true, false, CMP>(a, grid, lds, stream);
  return kl ? launch_one<D, B, HG, false, true, CMP>(a, grid, lds, stream)
            : launch_one<D, B, HG, false, false, CMP>(a, grid, lds, stream);
}

template <int D, int B, int HG>
int launch_hg(const AttnArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
  return a.compact ? launch_cmp<D, B, HG, true>(a, grid, lds, stream)
                   : launch_cmp<D, B, HG, false>(a, grid, lds, stream);
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
  if (a.stream) return launch_attention_bf16_stream(a, stream);
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
  set_error("paged attention (bf16): head_size %d with block_size %d is not built", a.D, a.B);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
