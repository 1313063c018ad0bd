// Paged decode attention for bf16 caches on gfx950: the stream schedule.
//
// Used with automatic partitioning when a batch has too few (sequence,
// kv-head group) units to fill the GPU with whole sequences.  The work is the
// list of (sequence s, group of HG kv heads, query-head chunk) units, each a
// run of cdiv(L_s, 32) steps, laid end to end in unit order.  A persistent
// grid of one round of resident workgroups cuts this stream into equal
// contiguous pieces, 4/HG per workgroup, each read by HG waves (one kv head
// each, walking the same tokens), so every wave -- and every CU -- reads the
// same number of K/V bytes whatever the mix of context lengths.  A unit
// lying inside one piece is finished there and written to out; a unit cut
// into several pieces leaves one partial result per piece in consecutive
// workspace slots, combined afterwards by the log-sum-exp merge.  Given the
// step's new key/value rows, the launch also stores each sequence's new token
// (the decode step's write) before reading it back with the rest.
#include "attention_bf16_wave.hpp"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;  // accelerator complexes (each with its own L2) of an MI355X
using wave::kStep;

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
    // With new tokens given (and the in-launch write chosen), each sequence's
    // token L - 1 is stored into the cache by the piece that reads the
    // sequence's last step (one row per kv head; every query-head chunk's
    // wave stores the same bytes) before that piece reads it back like the
    // others (the fences in store_new order the storing lanes' stores before
    // the loading lanes' loads), and no other piece of this launch reads the
    // row.  The slot rule and its -1
    // cases are the write kernel's; phys is the token's table entry.  Returns
    // false when it is out of range.  The rows are loaded first (their
    // latency overlaps the table lookup).
    uint4 kk = make_uint4(0, 0, 0, 0), vv = kk;
    auto load_new = [&]() {
      if (lane < D / 8) {
        const int64_t nrow = (static_cast<int64_t>(s) * a.Hkv + kvh) * D + 8 * lane;
        kk = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k_new) + nrow);
        vv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v_new) + nrow);
      }
    };
    auto store_new = [&](int phys) -> bool {
      if (phys < 0 || phys >= a.NB) return false;
      if (lane < D / 8) {
        const int64_t dst = (static_cast<int64_t>(phys) * B + (L - 1) % B) * a.Hkv * D +
                            static_cast<int64_t>(kvh) * D + 8 * lane;
        uint16_t* cache = static_cast<uint16_t*>(const_cast<void*>(a.kv));
        *reinterpret_cast<uint4*>(cache + dst) = kk;
        *reinterpret_cast<uint4*>(cache + static_cast<int64_t>(a.NB) * B * a.Hkv * D + dst) = vv;
      }
      // Other lanes of this wave read the rows just stored: a wavefront-scope
      // release/acquire orders the stores before those loads.  (gfx950 needs
      // no instruction for it -- a wavefront's memory operations are performed
      // in order -- so the fences only bind the compiler.)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      return true;
    };
    if (L < 0 || L > a.max_len || (L + B - 1) / B > a.width) {
      // an invalid sequence is one step, so always whole: NaN output (its
      // new token is still stored, as the write kernel would)
      if (a.k_new != nullptr && L > 0 && (L - 1) / B < a.width) {
        load_new();
        store_new(a.tables[static_cast<int64_t>(s) * a.width + (L - 1) / B]);
      }
      for (int e = lane; e < nh * SROW; e += 64) srow[e] = NAN;
    } else {
      const int t0 = st0 * kStep;
      const int t1 = min(L, st1 * kStep);
      const bool append = a.k_new != nullptr && L > 0 && t1 == L;
      if (append) load_new();
      w.begin(a, s, kvh, h0, nh, t0, t1);
      bool bad_new = false;
      if (append) {
        // the new token's table entry: from the window begin() loaded (the
        // run's first WIN steps), else from the table
        const int qn = (L - 1 - t0) / kStep;
        const int pn = ((L - 1 - t0) % kStep) / (kStep / Wv::EPS);
        const int phys = qn < Wv::WIN ? __builtin_amdgcn_readlane(w.win, Wv::EPS * qn + pn)
                                      : a.tables[static_cast<int64_t>(s) * a.width + (L - 1) / B];
        bad_new = !store_new(phys);
      }
      w.run_single((t1 - t0 + kStep - 1) / kStep, [](int) {});
      if (bad_new) w.bad_blk = true;  // (the step reading it flags it too)
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

template <int D, int B, int HG, bool NT, bool KL>
int launch_stream_one(const AttnArgs& a, hipStream_t stream) {
  auto kern = attention_bf16_stream_kernel<D, B, HG, NT, KL>;
  if (const int rc = raise_lds_limit(reinterpret_cast<const void*>(kern))) return rc;
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

int launch_attention_bf16_stream(const AttnArgs& a, hipStream_t stream) {
  if (a.S == 0) return PKV_OK;
  if (static_cast<size_t>(kWaves) * a.stream_wave_floats * sizeof(float) > bf16_lds_limit()) {
    set_error("paged attention (bf16): the stream schedule needs too much LDS");
    return PKV_ERR_UNSUPPORTED;
  }
  switch (a.D * 1000 + a.B) {
    case 64008: return launch_stream<64, 8>(a, stream);
    case 64016: return launch_stream<64, 16>(a, stream);
    case 64032: return launch_stream<64, 32>(a, stream);
    case 64064: return launch_stream<64, 64>(a, stream);
    case 128008: return launch_stream<128, 8>(a, stream);
    case 128016: return launch_stream<128, 16>(a, stream);
    case 128032: return launch_stream<128, 32>(a, stream);
    case 128064: return launch_stream<128, 64>(a, stream);
    default: break;
  }
  set_error("paged attention (bf16): head_size %d with block_size %d is not built", a.D, a.B);
  return PKV_ERR_UNSUPPORTED;
}

}  // namespace pkv
