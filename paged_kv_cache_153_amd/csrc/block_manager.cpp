// block_manager.cpp — host block manager behind the pa_bm_* C ABI.
//
// A pool of fixed-size physical KV blocks and one block table per sequence
// ([KVPA] "KV Cache与PagedAttention深度解析" §4.2 block tables, §5.1 block
// manager duties: free pool, allocate, reclaim, copy-on-write; §5.3 growth
// by one block when ceil((t+1)/bs) exceeds the table; §8.2-§8.3 reference
// counts).  Sharing and copy-on-write follow [NANO] (zwxr.cn walkthrough)
// §2.3: every table holding a block adds one reference; a sequence that is
// about to write into a block with count > 1 takes a fresh block, copies it
// (the device copy is the caller's, from the returned pair) and repoints its
// own table entry, while the other holders keep the original.
//
// Policy: the free pool is a stack that starts as [0, 1, ..., NB-1] and hands
// out from the top, like the pop()/append pool of [KV2P] "KV Cache从原理到实战"
// §6.2.  Every call checks all its preconditions before it changes anything,
// so a failing call leaves the manager as it was.  With PA_LOG=1 in the
// environment every allocation and release is logged to stderr with the
// sequence, block, count and free-pool size ([NANO] §4.5 logging advice).
//
// Prefix cache (pa_bm_enable_prefix_cache; [KVPA] §8.1-§8.2, [KV2P] §4.2-§4.3,
// [NANO] §3.2 and §4.3): every full block that a sequence registers is keyed
// by a chain hash of its token ids and position, h_i = FNV-1a-64(le64(h_{i-1})
// || le32 token ids), h_{-1} = 0.  A new prompt walks its full blocks from the
// start while they are cached (hash, parent hash and token ids all equal) and
// takes a reference on each; the rest gets fresh blocks.  A cached block whose
// count reaches 0 stays cached but evictable; fresh blocks come from the free
// pool first, then by evicting the least recently released evictable block,
// blocks with at least protect_hits hits last.  With admit_after > 1 a full
// block enters the cache only at the admit_after-th registration of its key
// (the other remedy [KV2P] §4.3 gives for a cache polluted by one-off
// prompts); the keys still below that count are remembered for at most
// num_blocks keys, the one seen least recently forgotten first.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <list>
#include <new>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "internal.h"

struct pa_bm {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t num_tokens = 0;
    std::vector<int32_t> tokens;  // known token ids (a prefix of the sequence)
    int64_t registered = 0;       // leading blocks already in the cache chain
  };
  struct Key {  // a cached block's identity
    bool cached = false;
    uint64_t hash = 0, parent = 0;
    std::vector<int32_t> tokens;
  };
  int64_t num_blocks = 0;
  int block_size = 0;
  std::vector<int32_t> free_list;  // stack; back() is handed out next
  std::vector<int32_t> refs;
  std::unordered_map<int64_t, Seq> seqs;
  bool log = false;
  // prefix cache
  bool cache_on = false;
  int protect_hits = 0;
  int admit_after = 1;
  // keys registered fewer than admit_after times: (key, count), least
  // recently seen first, and where each key sits in that list
  std::list<std::pair<uint64_t, int>> sightings;
  std::unordered_map<uint64_t, std::list<std::pair<uint64_t, int>>::iterator> sighting_at;
  std::unordered_map<uint64_t, int32_t> cache;
  std::vector<Key> keys;
  std::vector<int64_t> hits;
  std::set<std::tuple<int, uint64_t, int32_t>> evictable;  // (protected, clock, block)
  std::vector<uint64_t> ev_clock;
  std::vector<int> ev_prot;
  uint64_t clock = 0;
  int64_t lookups = 0, hit_blocks = 0, miss_blocks = 0, evictions = 0, held_back = 0;

  // Counts one more registration of key h; true once it reaches admit_after
  // (the key is then forgotten here: it enters the cache).
  bool admit(uint64_t h) {
    if (admit_after <= 1) return true;
    int seen = 1;
    auto at = sighting_at.find(h);
    if (at != sighting_at.end()) {
      seen += at->second->second;
      sightings.erase(at->second);
      sighting_at.erase(at);
    }
    if (seen >= admit_after) return true;
    sightings.emplace_back(h, seen);
    sighting_at[h] = std::prev(sightings.end());
    while ((int64_t)sightings.size() > num_blocks) {
      sighting_at.erase(sightings.front().first);
      sightings.pop_front();
    }
    ++held_back;
    return false;
  }

  int64_t available() const { return (int64_t)free_list.size() + (int64_t)evictable.size(); }

  int32_t take(int64_t seq) {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.back();
      free_list.pop_back();
    } else {  // evict the least recently released block, unprotected first
      b = std::get<2>(*evictable.begin());
      evictable.erase(evictable.begin());
      cache.erase(keys[b].hash);
      keys[b] = Key();
      hits[b] = 0;
      ++evictions;
    }
    refs[b] = 1;
    if (log)
      std::fprintf(stderr, "[pa_bm] take seq=%lld block=%d ref=1 free=%zu\n", (long long)seq, b,
                   free_list.size());
    return b;
  }
  void release(int64_t seq, int32_t b) {
    refs[b] -= 1;
    if (refs[b] == 0) {
      if (keys[b].cached) {
        const int prot = protect_hits > 0 && hits[b] >= protect_hits;
        evictable.insert({prot, clock, b});
        ev_clock[b] = clock;
        ev_prot[b] = prot;
        ++clock;
      } else {
        free_list.push_back(b);
      }
    }
    if (log)
      std::fprintf(stderr, "[pa_bm] drop seq=%lld block=%d ref=%d free=%zu\n", (long long)seq, b,
                   refs[b], free_list.size());
  }
  // a reference on a cached block (a prefix hit)
  void hold(int32_t b) {
    if (refs[b] == 0) evictable.erase({ev_prot[b], ev_clock[b], b});
    refs[b] += 1;
    hits[b] += 1;
  }
  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
};

namespace {

using pa::fail;

// 64-bit FNV-1a (published definition: per octet, xor then multiply by the
// prime) over the parent hash (8 bytes, little endian) and the block's token
// ids (4 bytes each, little endian).
uint64_t block_hash(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = 0xCBF29CE484222325ull;
  auto octet = [&](uint8_t x) {
    h ^= x;
    h *= 0x100000001B3ull;
  };
  for (int i = 0; i < 8; ++i) octet((uint8_t)(parent >> (8 * i)));
  for (int k = 0; k < n; ++k) {
    const uint32_t t = (uint32_t)tokens[k];
    for (int i = 0; i < 4; ++i) octet((uint8_t)(t >> (8 * i)));
  }
  return h;
}

int need_seq(const pa_bm* bm, int64_t seq) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (!bm->seqs.count(seq))
    return fail(PA_ERR_NOT_FOUND, "unknown sequence " + std::to_string(seq));
  return PA_OK;
}

// Fresh blocks the next append of `s` needs, given extra reference drops
// already planned in this batch (`dropped`).
int plan_append(const pa_bm* bm, const pa_bm::Seq& s,
                std::unordered_map<int32_t, int>& dropped) {
  if (s.num_tokens % bm->block_size == 0) return 1;
  const int32_t last = s.blocks.back();
  if (bm->refs[last] <= 1) return 0;  // private last block: written in place
  const auto it = dropped.find(last);
  const int already = it == dropped.end() ? 0 : it->second;
  if (bm->refs[last] - already > 1) {
    dropped[last] = already + 1;
    return 1;
  }
  return 0;
}

// Apply one append (preconditions already checked).
void do_append(pa_bm* bm, int64_t seq, pa_bm::Seq& s, int64_t* slot, int32_t* cow_src,
               int32_t* cow_dst) {
  const int64_t t = s.num_tokens;
  const int64_t row = t % bm->block_size;
  int32_t src = -1, dst = -1;
  if (row == 0) {
    s.blocks.push_back(bm->take(seq));
  } else if (bm->refs[s.blocks.back()] > 1) {
    src = s.blocks.back();
    dst = bm->take(seq);
    bm->release(seq, src);  // stays > 0: another table still holds it
    s.blocks.back() = dst;
  }
  s.num_tokens = t + 1;
  *slot = (int64_t)s.blocks.back() * bm->block_size + row;
  *cow_src = src;
  *cow_dst = dst;
}

}  // namespace

extern "C" {

pa_bm* pa_bm_create(int64_t num_blocks, int block_size) {
  pa::clear_error();
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) {
    fail(PA_ERR_INVALID_ARG, "num_blocks must be in [1, 2^31) and block_size positive");
    return nullptr;
  }
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->free_list.resize(num_blocks);
    for (int64_t i = 0; i < num_blocks; ++i) bm->free_list[i] = (int32_t)i;
    bm->refs.assign(num_blocks, 0);
    bm->keys.resize(num_blocks);
    bm->hits.assign(num_blocks, 0);
    bm->ev_clock.assign(num_blocks, 0);
    bm->ev_prot.assign(num_blocks, 0);
    const char* env = std::getenv("PA_LOG");
    bm->log = env && env[0] == '1';
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_allocate(pa_bm* bm, int64_t seq, int64_t num_tokens) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "negative token count");
  if (bm->seqs.count(seq))
    return fail(PA_ERR_INVALID_ARG, "sequence " + std::to_string(seq) + " already exists");
  const int64_t needed = bm->blocks_for(num_tokens);
  if (bm->available() < needed) return fail(PA_ERR_OOM, "out of KV cache blocks");
  try {
    pa_bm::Seq s;
    s.blocks.reserve(needed);
    for (int64_t i = 0; i < needed; ++i) s.blocks.push_back(bm->take(seq));
    s.num_tokens = num_tokens;
    bm->seqs.emplace(seq, std::move(s));
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  return PA_OK;
}

int pa_bm_share(pa_bm* bm, int64_t seq, const int32_t* blocks, int n, int64_t num_tokens) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (n < 0 || (n > 0 && !blocks) || num_tokens < 0 || bm->blocks_for(num_tokens) != n)
    return fail(PA_ERR_INVALID_ARG, "token count does not match the shared blocks");
  for (int i = 0; i < n; ++i) {
    const int32_t b = blocks[i];
    if (b < 0 || b >= bm->num_blocks || bm->refs[b] == 0)
      return fail(PA_ERR_INVALID_ARG, "block " + std::to_string(b) + " is not held");
  }
  auto it = bm->seqs.find(seq);
  if (it != bm->seqs.end() && it->second.num_tokens % bm->block_size != 0)
    return fail(PA_ERR_INVALID_ARG, "sequence ends inside a block");
  try {
    pa_bm::Seq& s = bm->seqs[seq];
    s.blocks.reserve(s.blocks.size() + n);
    for (int i = 0; i < n; ++i) {
      bm->refs[blocks[i]] += 1;
      s.blocks.push_back(blocks[i]);
    }
    s.num_tokens += num_tokens;
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  return PA_OK;
}

int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  pa::clear_error();
  if (int st = need_seq(bm, parent)) return st;
  if (bm->seqs.count(child))
    return fail(PA_ERR_INVALID_ARG, "sequence " + std::to_string(child) + " already exists");
  try {
    pa_bm::Seq copy = bm->seqs.at(parent);
    for (int32_t b : copy.blocks) bm->refs[b] += 1;
    bm->seqs.emplace(child, std::move(copy));
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  return PA_OK;
}

int pa_bm_append_slot(pa_bm* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
                      int32_t* cow_dst) {
  pa::clear_error();
  if (!slot || !cow_src || !cow_dst) return fail(PA_ERR_INVALID_ARG, "null output pointer");
  if (int st = need_seq(bm, seq)) return st;
  pa_bm::Seq& s = bm->seqs.at(seq);
  std::unordered_map<int32_t, int> dropped;
  if (bm->available() < plan_append(bm, s, dropped))
    return fail(PA_ERR_OOM, "out of KV cache blocks");
  do_append(bm, seq, s, slot, cow_src, cow_dst);
  return PA_OK;
}

int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, int n, int64_t* slots,
                       int32_t* cow_pairs, int* num_cow) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_cow)
    return fail(PA_ERR_INVALID_ARG, "bad arguments");
  // the first position that repeats an earlier sequence (n if none), found
  // by sorting (id, position) pairs: a batch reports the same first error a
  // sequential run would, without a hash-set node per sequence
  int first_repeat = n;
  std::vector<pa_bm::Seq*> rows;
  try {
    std::vector<std::pair<int64_t, int>> order((size_t)n);
    for (int i = 0; i < n; ++i) order[i] = {seqs[i], i};
    std::sort(order.begin(), order.end());
    for (int i = 1; i < n; ++i)
      if (order[i].first == order[i - 1].first) first_repeat = std::min(first_repeat, order[i].second);
    rows.resize((size_t)n);
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  std::unordered_map<int32_t, int> dropped;  // only shared last blocks enter
  int64_t needed = 0;
  for (int i = 0; i < n; ++i) {
    if (i == first_repeat) return fail(PA_ERR_INVALID_ARG, "sequence repeated in one batch");
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_NOT_FOUND, "unknown sequence " + std::to_string(seqs[i]));
    rows[i] = &it->second;  // stable: nothing is inserted or erased below
    // fail at the first sequence that would not fit, as a sequential run would
    needed += plan_append(bm, *rows[i], dropped);
    if (bm->available() < needed) return fail(PA_ERR_OOM, "out of KV cache blocks");
  }
  int k = 0;
  for (int i = 0; i < n; ++i) {
    int32_t src, dst;
    do_append(bm, seqs[i], *rows[i], &slots[i], &src, &dst);
    if (src >= 0) {
      cow_pairs[2 * k] = src;
      cow_pairs[2 * k + 1] = dst;
      ++k;
    }
  }
  *num_cow = k;
  return PA_OK;
}

int pa_bm_free(pa_bm* bm, int64_t seq) {
  pa::clear_error();
  if (int st = need_seq(bm, seq)) return st;
  auto it = bm->seqs.find(seq);
  for (int32_t b : it->second.blocks) bm->release(seq, b);
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_block_table(const pa_bm* bm, int64_t seq, int32_t* out, int cap, int* n,
                      int64_t* num_tokens) {
  pa::clear_error();
  if (int st = need_seq(bm, seq)) return st;
  if (cap < 0 || (cap > 0 && !out)) return fail(PA_ERR_INVALID_ARG, "bad output buffer");
  const pa_bm::Seq& s = bm->seqs.at(seq);
  const int len = (int)s.blocks.size();
  for (int i = 0; i < len && i < cap; ++i) out[i] = s.blocks[i];
  if (n) *n = len;
  if (num_tokens) *num_tokens = s.num_tokens;
  return PA_OK;
}

int pa_bm_block_tables(const pa_bm* bm, const int64_t* seqs, int n, int32_t* tables,
                       int max_blocks, int32_t* context_lens) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (n < 0 || max_blocks <= 0 || (n > 0 && (!seqs || !tables || !context_lens)))
    return fail(PA_ERR_INVALID_ARG, "bad arguments");
  std::vector<const pa_bm::Seq*> rows;
  try {
    rows.resize((size_t)n);
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_NOT_FOUND, "unknown sequence " + std::to_string(seqs[i]));
    if ((int64_t)it->second.blocks.size() > max_blocks)
      return fail(PA_ERR_INVALID_ARG, "table longer than max_blocks");
    if (it->second.num_tokens > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "context length does not fit int32");
    rows[i] = &it->second;
  }
  for (int i = 0; i < n; ++i) {
    const pa_bm::Seq& s = *rows[i];
    int32_t* row = tables + (int64_t)i * max_blocks;
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + s.blocks.size(), row + max_blocks, -1);
    context_lens[i] = (int32_t)s.num_tokens;
  }
  return PA_OK;
}

int pa_bm_stats(const pa_bm* bm, int64_t* num_free, int64_t* num_used, int64_t* num_shared) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  int64_t used = 0, shared = 0;
  for (int32_t c : bm->refs) {
    used += c >= 1;
    shared += c >= 2;
  }
  if (num_free) *num_free = bm->available();
  if (num_used) *num_used = used;
  if (num_shared) *num_shared = shared;
  return PA_OK;
}

int pa_bm_enable_prefix_cache(pa_bm* bm, int protect_hits, int admit_after) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (!bm->seqs.empty() || protect_hits < 0 || admit_after < 1)
    return fail(PA_ERR_INVALID_ARG, "enable the prefix cache on an empty manager");
  bm->cache_on = true;
  bm->protect_hits = protect_hits;
  bm->admit_after = admit_after;
  return PA_OK;
}

int pa_bm_allocate_prompt(pa_bm* bm, int64_t seq, const int32_t* tokens, int64_t n,
                          int64_t* cached_tokens) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (!bm->cache_on) return fail(PA_ERR_INVALID_ARG, "prefix cache is off");
  if (n < 0 || (n > 0 && !tokens)) return fail(PA_ERR_INVALID_ARG, "bad token array");
  if (bm->seqs.count(seq))
    return fail(PA_ERR_INVALID_ARG, "sequence " + std::to_string(seq) + " already exists");
  const int bs = bm->block_size;
  std::vector<int32_t> matched;
  uint64_t parent = 0;
  int64_t evictable_hits = 0;
  for (int64_t i = 0; i < n / bs; ++i) {
    const int32_t* blk = tokens + i * bs;
    const uint64_t h = block_hash(parent, blk, bs);
    auto it = bm->cache.find(h);
    if (it == bm->cache.end()) break;
    const pa_bm::Key& k = bm->keys[it->second];
    if (k.parent != parent || !std::equal(k.tokens.begin(), k.tokens.end(), blk)) break;
    matched.push_back(it->second);
    evictable_hits += bm->refs[it->second] == 0;
    parent = h;
  }
  const int64_t needed = bm->blocks_for(n) - (int64_t)matched.size();
  if (bm->available() - evictable_hits < needed) return fail(PA_ERR_OOM, "out of KV cache blocks");
  try {
    pa_bm::Seq s;
    s.blocks.reserve(bm->blocks_for(n));
    s.tokens.assign(tokens, tokens + n);
    bm->seqs.reserve(bm->seqs.size() + 1);
    bm->lookups += 1;
    bm->hit_blocks += (int64_t)matched.size();
    bm->miss_blocks += n / bs - (int64_t)matched.size();
    for (int32_t b : matched) {
      bm->hold(b);
      s.blocks.push_back(b);
    }
    for (int64_t i = 0; i < needed; ++i) s.blocks.push_back(bm->take(seq));
    s.num_tokens = n;
    s.registered = (int64_t)matched.size();
    bm->seqs.emplace(seq, std::move(s));
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  if (cached_tokens) *cached_tokens = (int64_t)matched.size() * bs;
  return PA_OK;
}

int pa_bm_record_tokens(pa_bm* bm, int64_t seq, const int32_t* tokens, int64_t n) {
  pa::clear_error();
  if (int st = need_seq(bm, seq)) return st;
  if (n < 0 || (n > 0 && !tokens)) return fail(PA_ERR_INVALID_ARG, "bad token array");
  pa_bm::Seq& s = bm->seqs.at(seq);
  if ((int64_t)s.tokens.size() + n != s.num_tokens)
    return fail(PA_ERR_INVALID_ARG, "token ids must complete the known prefix");
  try {
    s.tokens.insert(s.tokens.end(), tokens, tokens + n);
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  return PA_OK;
}

int pa_bm_register(pa_bm* bm, int64_t seq, int64_t* newly_cached) {
  pa::clear_error();
  if (int st = need_seq(bm, seq)) return st;
  if (!bm->cache_on) return fail(PA_ERR_INVALID_ARG, "prefix cache is off");
  pa_bm::Seq& s = bm->seqs.at(seq);
  const int bs = bm->block_size;
  const int64_t full = (int64_t)s.tokens.size() / bs;
  int64_t added = 0;
  try {
    uint64_t parent = 0;
    for (int64_t i = 0; i < full; ++i) {
      const int32_t* blk = s.tokens.data() + i * bs;
      const uint64_t h = block_hash(parent, blk, bs);
      if (i >= s.registered) {
        const int32_t b = s.blocks[i];
        if (!bm->cache.count(h) && !bm->keys[b].cached && bm->admit(h)) {
          pa_bm::Key& k = bm->keys[b];
          k.tokens.assign(blk, blk + bs);
          k.hash = h;
          k.parent = parent;
          k.cached = true;
          bm->cache.emplace(h, b);
          ++added;
        }
      }
      parent = h;
    }
  } catch (...) {
    return fail(PA_ERR_OOM, "host memory exhausted");
  }
  s.registered = full;
  if (newly_cached) *newly_cached = added;
  return PA_OK;
}

int pa_bm_prefix_stats(const pa_bm* bm, int64_t* out) {
  pa::clear_error();
  if (!bm || !out) return fail(PA_ERR_INVALID_ARG, "null argument");
  int64_t cached = 0;
  for (const auto& k : bm->keys) cached += k.cached;
  out[0] = cached;
  out[1] = (int64_t)bm->evictable.size();
  out[2] = bm->lookups;
  out[3] = bm->hit_blocks;
  out[4] = bm->miss_blocks;
  out[5] = bm->evictions;
  out[6] = bm->held_back;
  return PA_OK;
}

int pa_bm_ref_count(const pa_bm* bm, int32_t block) {
  pa::clear_error();
  if (!bm) return fail(PA_ERR_INVALID_ARG, "null block manager");
  if (block < 0 || block >= bm->num_blocks) return fail(PA_ERR_INVALID_ARG, "block out of range");
  return bm->refs[block];
}

}  // extern "C"
