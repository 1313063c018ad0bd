// Host-side KV block manager: the allocator that hands the decode path its
// block tables and slots.
//
// * A pool of physical blocks, each with a reference count: a block shared by
//   several logical blocks (forked samples, prefix-cache hits) counts each of
//   them (studying-code.tistory.com vLLM review, "요청 완료 후 메모리 관리").
// * Free blocks wait in a queue (an intrusive doubly linked list over block
//   ids, so a prefix-cache hit can leave it from the middle in O(1)).
//   Allocation takes the head; a finished request returns its blocks whose
//   count reaches zero to the tail, last block first (itan.pw walk-through of
//   vLLM's KVCacheManager, "プレイフィックスキャッシュの詳細", times 4-6).
// * Fork shares the parent's blocks and raises their counts; before a token
//   is written into a block with count > 1 the writer takes a fresh block and
//   reports a (source, destination) copy, and the old count drops by one
//   (the review's "생성 단계에서의 Copy-on-Write"; tech.blogsailing.com
//   explainer, section 3).
// * Full blocks get a chain hash, SHA-256(previous hash || the block's token
//   ids as little-endian int32), and enter the prefix cache; a new request's
//   hits are its leading full blocks -- at most (n - 1) / B of them -- up to
//   the first miss; a cached block taken from the free queue loses its entry
//   (the walk-through, "プレイフィックスキャッシュの詳細").
// * A group of sequences is swapped to a CPU pool and back all or nothing;
//   a request the pool cannot satisfy is refused with nothing changed.
//
// Not thread-safe: one manager is used by one thread at a time.
#include "paged_kv.h"

#include <cmath>
#include <cstdint>
#include <cstring>
#include <deque>
#include <unordered_map>
#include <unordered_set>
#include <vector>

namespace pkv {
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

namespace {

// ---------------------------------------------------------------- SHA-256

// SHA-256 as FIPS 180-4 defines it.  The round constants are the first 32
// bits of the fractional parts of the cube roots of the first 64 primes, the
// initial hash value those of the square roots of the first 8 primes; both
// are derived here with exact integer roots.
class Sha256 {
 public:
  static const Sha256& get() {
    static const Sha256 inst;
    return inst;
  }

  void digest(const uint8_t* msg, size_t len, uint8_t out[32]) const {
    uint32_t h[8];
    std::memcpy(h, h0_, sizeof h);
    const uint64_t bits = static_cast<uint64_t>(len) * 8;
    size_t full = len / 64;
    for (size_t i = 0; i < full; ++i) block(h, msg + 64 * i);
    uint8_t tail[128] = {};
    const size_t rest = len - 64 * full;
    std::memcpy(tail, msg + 64 * full, rest);
    tail[rest] = 0x80;
    const size_t tail_len = rest + 1 + 8 <= 64 ? 64 : 128;
    for (int k = 0; k < 8; ++k) tail[tail_len - 1 - k] = static_cast<uint8_t>(bits >> (8 * k));
    for (size_t off = 0; off < tail_len; off += 64) block(h, tail + off);
    for (int i = 0; i < 8; ++i)
      for (int k = 0; k < 4; ++k) out[4 * i + k] = static_cast<uint8_t>(h[i] >> (24 - 8 * k));
  }

 private:
  uint32_t k_[64];
  uint32_t h0_[8];

  static uint64_t iroot(unsigned __int128 x, int n) {
    // floor(x^(1/n)) for n in {2, 3}
    auto pw = [n](unsigned __int128 r) { return n == 2 ? r * r : r * r * r; };
    uint64_t r = static_cast<uint64_t>(n == 2 ? sqrtl(static_cast<long double>(x))
                                              : cbrtl(static_cast<long double>(x)));
    while (r > 0 && pw(r) > x) --r;
    while (pw(static_cast<unsigned __int128>(r) + 1) <= x) ++r;
    return r;
  }

  Sha256() {
    int primes[64];
    for (int n = 2, c = 0; c < 64; ++n) {
      bool prime = true;
      for (int d = 2; d * d <= n; ++d)
        if (n % d == 0) { prime = false; break; }
      if (prime) primes[c++] = n;
    }
    for (int i = 0; i < 64; ++i)
      k_[i] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(primes[i]) << 96, 3));
    for (int i = 0; i < 8; ++i)
      h0_[i] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(primes[i]) << 64, 2));
  }

  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

  void block(uint32_t h[8], const uint8_t* p) const {
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t{p[4 * t]} << 24) | (uint32_t{p[4 * t + 1]} << 16) |
             (uint32_t{p[4 * t + 2]} << 8) | uint32_t{p[4 * t + 3]};
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = s1 + w[t - 7] + s0 + w[t - 16];
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = hh + S1 + ch + k_[t] + w[t];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + maj;
      hh = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }
};

struct Hash {
  uint8_t b[32];
  bool operator==(const Hash& o) const { return std::memcmp(b, o.b, 32) == 0; }
};
struct HashKey {
  size_t operator()(const Hash& h) const {
    size_t v;
    std::memcpy(&v, h.b, sizeof v);
    return v;
  }
};

// hash of a full block: SHA-256(parent || tokens as little-endian int32)
Hash chain_hash(const Hash& parent, const int32_t* tokens, int n) {
  std::vector<uint8_t> msg(32 + 4 * static_cast<size_t>(n));
  std::memcpy(msg.data(), parent.b, 32);
  for (int i = 0; i < n; ++i) {
    const uint32_t t = static_cast<uint32_t>(tokens[i]);
    for (int k = 0; k < 4; ++k) msg[32 + 4 * i + k] = static_cast<uint8_t>(t >> (8 * k));
  }
  Hash h;
  Sha256::get().digest(msg.data(), msg.size(), h.b);
  return h;
}

// ---------------------------------------------------------------- free queue

class FreeQueue {
 public:
  explicit FreeQueue(int n) : prev_(n, -1), next_(n, -1), in_(n, 0) {}
  int size() const { return size_; }
  bool contains(int b) const { return in_[b] != 0; }
  int front() const { return head_; }
  int next(int b) const { return next_[b]; }
  void push_back(int b) {
    prev_[b] = tail_;
    next_[b] = -1;
    if (tail_ >= 0) next_[tail_] = b; else head_ = b;
    tail_ = b;
    in_[b] = 1;
    ++size_;
  }
  void remove(int b) {
    if (prev_[b] >= 0) next_[prev_[b]] = next_[b]; else head_ = next_[b];
    if (next_[b] >= 0) prev_[next_[b]] = prev_[b]; else tail_ = prev_[b];
    in_[b] = 0;
    --size_;
  }
  int pop_front() {
    const int b = head_;
    remove(b);
    return b;
  }
  void clear() {
    while (size_ > 0) pop_front();
  }

 private:
  std::vector<int> prev_, next_;
  std::vector<uint8_t> in_;
  int head_ = -1, tail_ = -1, size_ = 0;
};

struct Seq {
  std::vector<int32_t> table;   // physical (or, swapped, CPU) block of each logical block
  std::vector<int32_t> tokens;  // token ids so far
  std::vector<Hash> hashes;     // chain hash of each full block so far
  bool swapped = false;
};

}  // namespace
}  // namespace pkv

struct pkv_block_manager {
  int N, B;
  bool prefix;
  std::vector<int32_t> ref;
  std::vector<uint8_t> has_hash;
  std::vector<pkv::Hash> hash_of;
  std::unordered_map<pkv::Hash, int32_t, pkv::HashKey> cache;
  pkv::FreeQueue free;
  std::deque<int32_t> cpu_free;
  std::vector<int32_t> cpu_ref;
  std::unordered_map<int64_t, pkv::Seq> seqs;

  pkv_block_manager(int n, int b, bool p, int ncpu)
      : N(n), B(b), prefix(p), ref(n, 0), has_hash(n, 0), hash_of(n), free(n), cpu_ref(ncpu, 0) {
    for (int i = 0; i < n; ++i) free.push_back(i);
    for (int i = 0; i < ncpu; ++i) cpu_free.push_back(i);
  }

  int take() {
    const int b = free.pop_front();
    if (has_hash[b]) {  // eviction on reuse
      auto it = cache.find(hash_of[b]);
      if (it != cache.end() && it->second == b) cache.erase(it);
      has_hash[b] = 0;
    }
    ref[b] = 1;
    return b;
  }
  void touch(int b) {
    if (ref[b] == 0) free.remove(b);
    ++ref[b];
  }
  void release(int b) {
    if (--ref[b] == 0) free.push_back(b);
  }
  void cache_full(pkv::Seq& s) {
    while (static_cast<int>(s.hashes.size()) < static_cast<int>(s.tokens.size()) / B) {
      const size_t i = s.hashes.size();
      const pkv::Hash parent = i ? s.hashes.back() : pkv::Hash{};
      const pkv::Hash h = pkv::chain_hash(parent, s.tokens.data() + i * B, B);
      s.hashes.push_back(h);
      if (prefix && !s.swapped) {
        const int b = s.table[i];
        cache.emplace(h, b);  // keeps an existing entry for the same content
        if (!has_hash[b]) {
          hash_of[b] = h;
          has_hash[b] = 1;
        }
      }
    }
  }
};

using pkv::set_error;
using pkv::clear_error;

namespace {

pkv::Seq* find_seq(pkv_block_manager* bm, int64_t id) {
  auto it = bm->seqs.find(id);
  if (it == bm->seqs.end()) {
    set_error("block manager: no sequence %lld", static_cast<long long>(id));
    return nullptr;
  }
  return &it->second;
}

bool check_bm(pkv_block_manager* bm) {
  if (!bm) set_error("block manager: null manager");
  return bm != nullptr;
}

// Blocks used by a group of sequences, in first-use order, with how many
// table entries of the group point at each.
void group_blocks(pkv_block_manager* bm, const std::vector<pkv::Seq*>& group,
                  std::vector<int32_t>* blocks, std::unordered_map<int32_t, int32_t>* uses) {
  for (pkv::Seq* s : group)
    for (int32_t b : s->table) {
      if (uses->find(b) == uses->end()) blocks->push_back(b);
      ++(*uses)[b];
    }
  (void)bm;
}

bool collect_group(pkv_block_manager* bm, const int64_t* ids, int n, bool want_swapped,
                   std::vector<pkv::Seq*>* group) {
  std::unordered_set<int64_t> seen;
  for (int i = 0; i < n; ++i) {
    if (!seen.insert(ids[i]).second) {
      set_error("block manager: sequence %lld listed twice", static_cast<long long>(ids[i]));
      return false;
    }
    pkv::Seq* s = find_seq(bm, ids[i]);
    if (!s) return false;
    if (s->swapped != want_swapped) {
      set_error("block manager: sequence %lld is %s", static_cast<long long>(ids[i]),
                s->swapped ? "swapped out" : "not swapped out");
      return false;
    }
    group->push_back(s);
  }
  return true;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int num_blocks, int block_size, int prefix_caching,
                                 int num_cpu_blocks) {
  clear_error();
  if (num_blocks <= 0 || block_size <= 0 || num_cpu_blocks < 0) {
    set_error("block manager: bad sizes (blocks %d, block size %d, cpu blocks %d)", num_blocks,
              block_size, num_cpu_blocks);
    return nullptr;
  }
  try {
    return new pkv_block_manager(num_blocks, block_size, prefix_caching != 0, num_cpu_blocks);
  } catch (...) {
    set_error("block manager: out of host memory");
    return nullptr;
  }
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_set_free_order(pkv_block_manager* bm, const int32_t* order, int n) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (!bm->seqs.empty() || n != bm->N || !order) {
    set_error("block manager: the free order is set on a fresh manager, for all %d blocks", bm->N);
    return PKV_ERR_INVALID;
  }
  std::vector<uint8_t> seen(bm->N, 0);
  for (int i = 0; i < n; ++i) {
    if (order[i] < 0 || order[i] >= bm->N || seen[order[i]]) {
      set_error("block manager: the free order is not a permutation of the blocks");
      return PKV_ERR_INVALID;
    }
    seen[order[i]] = 1;
  }
  bm->free.clear();
  for (int i = 0; i < n; ++i) bm->free.push_back(order[i]);
  return PKV_OK;
}

int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int num_tokens,
                    int* num_cached_tokens) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (num_tokens < 0 || (num_tokens > 0 && !tokens)) {
    set_error("block manager: bad tokens");
    return PKV_ERR_INVALID;
  }
  if (bm->seqs.count(seq)) {
    set_error("block manager: sequence %lld exists", static_cast<long long>(seq));
    return PKV_ERR_INVALID;
  }
  const int B = bm->B;
  const int need = (num_tokens + B - 1) / B;
  std::vector<int32_t> hits;
  if (bm->prefix && num_tokens > 0) {
    pkv::Hash parent{};
    for (int i = 0; i < (num_tokens - 1) / B; ++i) {
      const pkv::Hash h = pkv::chain_hash(parent, tokens + static_cast<size_t>(i) * B, B);
      auto it = bm->cache.find(h);
      if (it == bm->cache.end()) break;
      hits.push_back(it->second);
      parent = h;
    }
  }
  int in_queue = 0;
  for (int32_t b : hits) in_queue += bm->ref[b] == 0;
  if (bm->free.size() - in_queue < need - static_cast<int>(hits.size())) {
    set_error("block manager: %d free blocks, %d needed", bm->free.size() - in_queue,
              need - static_cast<int>(hits.size()));
    return PKV_ERR_NO_BLOCKS;
  }
  pkv::Seq s;
  for (int32_t b : hits) bm->touch(b);
  s.table = hits;
  while (static_cast<int>(s.table.size()) < need) s.table.push_back(bm->take());
  s.tokens.assign(tokens, tokens + num_tokens);
  pkv::Seq& stored = bm->seqs.emplace(seq, std::move(s)).first->second;
  bm->cache_full(stored);
  if (num_cached_tokens) *num_cached_tokens = static_cast<int>(hits.size()) * B;
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq, const int32_t* tokens, int n,
                  int64_t* slots, int32_t* copy_src, int32_t* copy_dst, int* num_copies) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  pkv::Seq* s = find_seq(bm, seq);
  if (!s) return PKV_ERR_INVALID;
  if (s->swapped) {
    set_error("block manager: sequence %lld is swapped out", static_cast<long long>(seq));
    return PKV_ERR_INVALID;
  }
  if (n < 0 || (n > 0 && (!tokens || !slots || !copy_src || !copy_dst))) {
    set_error("block manager: bad append arguments");
    return PKV_ERR_INVALID;
  }
  const int B = bm->B;
  if (n > 0) {
    // one block per new logical block and per shared block written
    const int first = static_cast<int>(s->tokens.size()) / B;
    const int last = (static_cast<int>(s->tokens.size()) + n - 1) / B;
    int need = 0;
    for (int lb = first; lb <= last; ++lb)
      need += lb >= static_cast<int>(s->table.size()) || bm->ref[s->table[lb]] > 1;
    if (need > bm->free.size()) {
      set_error("block manager: %d free blocks, %d needed", bm->free.size(), need);
      return PKV_ERR_NO_BLOCKS;
    }
  }
  int nc = 0;
  for (int k = 0; k < n; ++k) {
    const int p = static_cast<int>(s->tokens.size());
    const int lb = p / B;
    if (lb == static_cast<int>(s->table.size())) {
      s->table.push_back(bm->take());
    } else if (bm->ref[s->table[lb]] > 1) {
      const int old = s->table[lb];
      const int nb = bm->take();
      copy_src[nc] = old;
      copy_dst[nc] = nb;
      ++nc;
      --bm->ref[old];  // still held by the other sharers
      s->table[lb] = nb;
    }
    slots[k] = static_cast<int64_t>(s->table[lb]) * B + p % B;
    s->tokens.push_back(tokens[k]);
    bm->cache_full(*s);
  }
  if (num_copies) *num_copies = nc;
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  pkv::Seq* s = find_seq(bm, parent);
  if (!s) return PKV_ERR_INVALID;
  if (s->swapped || bm->seqs.count(child)) {
    set_error("block manager: cannot fork %lld into %lld", static_cast<long long>(parent),
              static_cast<long long>(child));
    return PKV_ERR_INVALID;
  }
  pkv::Seq c = *s;
  for (int32_t b : c.table) ++bm->ref[b];
  bm->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* bm, int64_t seq) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  pkv::Seq* s = find_seq(bm, seq);
  if (!s) return PKV_ERR_INVALID;
  for (auto it = s->table.rbegin(); it != s->table.rend(); ++it) {
    if (s->swapped) {
      if (--bm->cpu_ref[*it] == 0) bm->cpu_free.push_back(*it);
    } else {
      bm->release(*it);
    }
  }
  bm->seqs.erase(seq);
  return PKV_OK;
}

int pkv_bm_swap_out(pkv_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* gpu_blocks,
                    int32_t* cpu_blocks, int capacity, int* num_copies) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (num_seqs <= 0 || !seqs || !gpu_blocks || !cpu_blocks) {
    set_error("block manager: bad swap arguments");
    return PKV_ERR_INVALID;
  }
  std::vector<pkv::Seq*> group;
  if (!collect_group(bm, seqs, num_seqs, false, &group)) return PKV_ERR_INVALID;
  std::vector<int32_t> blocks;
  std::unordered_map<int32_t, int32_t> uses;
  group_blocks(bm, group, &blocks, &uses);
  for (int32_t b : blocks)
    if (bm->ref[b] != uses[b]) {
      set_error("block manager: block %d is shared outside the group", b);
      return PKV_ERR_INVALID;
    }
  if (static_cast<int>(blocks.size()) > capacity) {
    set_error("block manager: %zu copies, room for %d", blocks.size(), capacity);
    return PKV_ERR_INVALID;
  }
  if (blocks.size() > bm->cpu_free.size()) {
    set_error("block manager: %zu free CPU blocks, %zu needed", bm->cpu_free.size(), blocks.size());
    return PKV_ERR_NO_BLOCKS;
  }
  std::unordered_map<int32_t, int32_t> to_cpu;
  for (size_t i = 0; i < blocks.size(); ++i) {
    const int32_t c = bm->cpu_free.front();
    bm->cpu_free.pop_front();
    to_cpu[blocks[i]] = c;
    bm->cpu_ref[c] = uses[blocks[i]];
    gpu_blocks[i] = blocks[i];
    cpu_blocks[i] = c;
  }
  for (pkv::Seq* s : group) {
    for (int32_t& b : s->table) b = to_cpu[b];
    s->swapped = true;
  }
  for (auto it = blocks.rbegin(); it != blocks.rend(); ++it) {
    const int b = *it;
    if (bm->has_hash[b]) {
      auto c = bm->cache.find(bm->hash_of[b]);
      if (c != bm->cache.end() && c->second == b) bm->cache.erase(c);
      bm->has_hash[b] = 0;
    }
    bm->ref[b] = 0;
    bm->free.push_back(b);
  }
  if (num_copies) *num_copies = static_cast<int>(blocks.size());
  return PKV_OK;
}

int pkv_bm_swap_in(pkv_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* cpu_blocks,
                   int32_t* gpu_blocks, int capacity, int* num_copies) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (num_seqs <= 0 || !seqs || !gpu_blocks || !cpu_blocks) {
    set_error("block manager: bad swap arguments");
    return PKV_ERR_INVALID;
  }
  std::vector<pkv::Seq*> group;
  if (!collect_group(bm, seqs, num_seqs, true, &group)) return PKV_ERR_INVALID;
  std::vector<int32_t> blocks;
  std::unordered_map<int32_t, int32_t> uses;
  group_blocks(bm, group, &blocks, &uses);
  for (int32_t b : blocks)
    if (bm->cpu_ref[b] != uses[b]) {
      set_error("block manager: CPU block %d is shared outside the group", b);
      return PKV_ERR_INVALID;
    }
  if (static_cast<int>(blocks.size()) > capacity) {
    set_error("block manager: %zu copies, room for %d", blocks.size(), capacity);
    return PKV_ERR_INVALID;
  }
  if (static_cast<int>(blocks.size()) > bm->free.size()) {
    set_error("block manager: %d free blocks, %zu needed", bm->free.size(), blocks.size());
    return PKV_ERR_NO_BLOCKS;
  }
  std::unordered_map<int32_t, int32_t> to_gpu;
  for (size_t i = 0; i < blocks.size(); ++i) {
    const int32_t g = bm->take();
    to_gpu[blocks[i]] = g;
    bm->ref[g] = uses[blocks[i]];
    cpu_blocks[i] = blocks[i];
    gpu_blocks[i] = g;
  }
  for (pkv::Seq* s : group) {
    for (int32_t& b : s->table) b = to_gpu[b];
    s->swapped = false;
  }
  for (auto it = blocks.rbegin(); it != blocks.rend(); ++it) {
    bm->cpu_ref[*it] = 0;
    bm->cpu_free.push_back(*it);
  }
  if (bm->prefix)
    for (pkv::Seq* s : group)
      for (size_t i = 0; i < s->hashes.size(); ++i) {
        const int b = s->table[i];
        bm->cache.emplace(s->hashes[i], b);
        if (!bm->has_hash[b]) {
          bm->hash_of[b] = s->hashes[i];
          bm->has_hash[b] = 1;
        }
      }
  if (num_copies) *num_copies = static_cast<int>(blocks.size());
  return PKV_OK;
}

int pkv_bm_num_tokens(pkv_block_manager* bm, int64_t seq) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  pkv::Seq* s = find_seq(bm, seq);
  return s ? static_cast<int>(s->tokens.size()) : PKV_ERR_INVALID;
}

int pkv_bm_is_swapped(pkv_block_manager* bm, int64_t seq) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  pkv::Seq* s = find_seq(bm, seq);
  return s ? (s->swapped ? 1 : 0) : PKV_ERR_INVALID;
}

int pkv_bm_block_table(pkv_block_manager* bm, int64_t seq, int32_t* out, int capacity) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  pkv::Seq* s = find_seq(bm, seq);
  if (!s) return PKV_ERR_INVALID;
  const int n = static_cast<int>(s->table.size());
  for (int i = 0; i < n && i < capacity && out; ++i) out[i] = s->table[i];
  return n;
}

int pkv_bm_slots(pkv_block_manager* bm, int64_t seq, int begin, int end, int64_t* out) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  pkv::Seq* s = find_seq(bm, seq);
  if (!s) return PKV_ERR_INVALID;
  if (begin < 0 || end < begin || end > static_cast<int>(s->tokens.size()) || (end > begin && !out) ||
      s->swapped) {
    set_error("block manager: bad slot range [%d, %d) of %zu tokens", begin, end, s->tokens.size());
    return PKV_ERR_INVALID;
  }
  for (int p = begin; p < end; ++p)
    out[p - begin] = static_cast<int64_t>(s->table[p / bm->B]) * bm->B + p % bm->B;
  return PKV_OK;
}

int pkv_bm_batch_tables(pkv_block_manager* bm, const int64_t* seqs, int num_seqs, int32_t* tables,
                        int table_width, int32_t* context_lens) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (num_seqs < 0 || table_width <= 0 || (num_seqs > 0 && (!seqs || !tables || !context_lens))) {
    set_error("block manager: bad batch arguments");
    return PKV_ERR_INVALID;
  }
  for (int i = 0; i < num_seqs; ++i) {
    pkv::Seq* s = find_seq(bm, seqs[i]);
    if (!s) return PKV_ERR_INVALID;
    if (s->swapped || static_cast<int>(s->table.size()) > table_width) {
      set_error("block manager: sequence %lld is swapped out or has more than %d blocks",
                static_cast<long long>(seqs[i]), table_width);
      return PKV_ERR_INVALID;
    }
  }
  for (int i = 0; i < num_seqs; ++i) {
    const pkv::Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + static_cast<int64_t>(i) * table_width;
    for (int j = 0; j < table_width; ++j)
      row[j] = j < static_cast<int>(s.table.size()) ? s.table[j] : INT32_MIN;
    context_lens[i] = static_cast<int32_t>(s.tokens.size());
  }
  return PKV_OK;
}

int pkv_bm_ref_count(pkv_block_manager* bm, int block) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (block < 0 || block >= bm->N) {
    set_error("block manager: no block %d", block);
    return PKV_ERR_INVALID;
  }
  return bm->ref[block];
}

int pkv_bm_num_free(pkv_block_manager* bm) {
  clear_error();
  return check_bm(bm) ? bm->free.size() : PKV_ERR_INVALID;
}

int pkv_bm_free_queue(pkv_block_manager* bm, int32_t* out, int capacity) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  int i = 0;
  for (int b = bm->free.front(); b >= 0; b = bm->free.next(b), ++i)
    if (out && i < capacity) out[i] = b;
  return i;
}

int pkv_bm_block_hash(pkv_block_manager* bm, int block, uint8_t* out) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (block < 0 || block >= bm->N || !out) {
    set_error("block manager: no block %d", block);
    return PKV_ERR_INVALID;
  }
  if (!bm->has_hash[block]) return 0;
  std::memcpy(out, bm->hash_of[block].b, 32);
  return 1;
}

int pkv_bm_is_cached(pkv_block_manager* bm, int block) {
  clear_error();
  if (!check_bm(bm)) return PKV_ERR_INVALID;
  if (block < 0 || block >= bm->N) {
    set_error("block manager: no block %d", block);
    return PKV_ERR_INVALID;
  }
  if (!bm->has_hash[block]) return 0;
  auto it = bm->cache.find(bm->hash_of[block]);
  return it != bm->cache.end() && it->second == block ? 1 : 0;
}

}  // extern "C"
