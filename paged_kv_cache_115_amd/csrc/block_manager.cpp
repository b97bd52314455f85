// Host block manager: free list, per-sequence block tables, reference counts
// and copy-on-write for shared prefixes.  Plain C++ on the CPU.
//
// Behaviour (pages):
//  - blocks leave one global free list on demand; any free block fits any
//    request (llminference.xinbetween.com S06 "PagedAttention", "The
//    solution"); a retired block is reused first;
//  - a sequence takes a new block whenever its length is a multiple of B
//    before a write; the slot of position t is table[t/B]*B + t%B
//    (mercemay.com "Paged KV Cache Allocation and the Block Table", "Blocks,
//    tables, and the indirection"; synapticradio.com "The KV Cache Is an
//    Allocator Problem", equation in "What the trace shows");
//  - counts per block; fork aliases a table; retiring decrements and frees
//    only blocks reaching zero; the first write into a shared, partly filled
//    block copies it (mercemay.com "Sharing blocks between sequences";
//    aicassindra.com "tm_paged_attention_deep", "Copy-on-write for shared
//    prefixes");
//  - when blocks run out, a sequence's blocks can be copied to host memory
//    and back instead of recomputing it (mercemay.com, "Three ways contiguous
//    reservation loses memory"; S06, third exercise).  Host memory is a
//    second pool of blocks with its own free list and counts under the same
//    discipline; the distinct blocks of the listed tables move once each, so
//    sharing survives the round trip.
//  - prefix caching across requests: block contents are hashed so that any
//    two requests with a common prefix share the same physical blocks
//    (S06, "What's next"; the same page's production notes on a radix tree
//    of prefixes).  A cached block is keyed by (parent cached block, its B
//    token ids), found through a 64-bit hash of that pair and then compared
//    exactly, so a hash collision is a miss, never a wrong share; by
//    induction over the parents the key is the block's whole token prefix.
//    Cached blocks whose count drops to zero stay cached and become
//    evictable; new blocks come from the free list first, then from the least
//    recently retired evictable block (a retiring table's blocks are ranked
//    deepest first), and evicting a block drops every cached block below it.
// Appends and swaps are all-or-nothing: a request that does not fit changes
// nothing.
#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "internal.h"

using pagedkv::fail;

struct pa_bm {
  pagedkv::StepPlanCache plan_cache;  // pa_bm_prepare_decode_step's plan reuse
  struct Seq {
    std::vector<int32_t> table;     // host-pool blocks while swapped
    int32_t len = 0;
    bool swapped = false;
    uint64_t stamp = 0;             // batch calls: the call that last listed the sequence
  };
  uint64_t stamp_now = 0;           // batch calls: stamp of the current call
  std::vector<Seq*> step_seqs;      // pa_bm_prepare_decode_step: the batch, resolved once
  // One pool of blocks: free list and counts.
  struct Pool {
    std::vector<int32_t> free_stack;  // back() is handed out next
    std::vector<int32_t> refcount;
    void reset(int32_t n) {
      refcount.assign(n, 0);
      free_stack.resize(n);
      for (int32_t i = 0; i < n; ++i) free_stack[n - 1 - i] = i;
    }
    // Drop one count of every block of `table`; blocks reaching zero go back
    // on the list in table order.
    void release(const std::vector<int32_t>& table) {
      for (int32_t b : table)
        if (--refcount[b] == 0) free_stack.push_back(b);
    }
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  Pool dev;
  Pool host;
  std::map<int64_t, Seq> seqs;      // ordered: deterministic checks and stats
  int64_t alloc_failures = 0;
  int64_t cow_copies = 0;
  int64_t swap_out_blocks = 0;
  int64_t swap_in_blocks = 0;
  int32_t num_swapped = 0;

  // Prefix cache.
  struct Cached {
    int32_t parent = -1;          // cached block holding the previous B tokens; -1 at position 0
    uint64_t hash = 0;
    std::vector<int32_t> tokens;  // this block's B token ids
    std::vector<int32_t> children;
  };
  bool prefix_cache = false;
  std::unordered_map<int32_t, Cached> cached;          // block -> entry
  std::unordered_multimap<uint64_t, int32_t> index;    // hash -> block
  std::set<std::pair<int64_t, int32_t>> evictable;     // (retire tick, block), count 0
  std::vector<int64_t> tick_of;                        // retire tick of an evictable block, else -1
  int64_t tick = 0;
  int64_t prefix_query_tokens = 0;
  int64_t prefix_hit_tokens = 0;

  int64_t capacity() const { return (int64_t)dev.free_stack.size() + (int64_t)evictable.size(); }

  static uint64_t mix(uint64_t x) {  // splitmix64 finalizer
    x += 0x9e3779b97f4a7c15ull;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
    return x ^ (x >> 31);
  }
  uint64_t key_hash(int32_t parent, const int32_t* tok) const {
    uint64_t h = mix((uint64_t)(int64_t)parent);
    for (int32_t i = 0; i < block_size; ++i) h = mix(h ^ (uint32_t)tok[i]);
    return h;
  }
  // The cached block holding `tok` after `parent`, or -1.
  int32_t lookup(int32_t parent, const int32_t* tok) const {
    auto range = index.equal_range(key_hash(parent, tok));
    for (auto it = range.first; it != range.second; ++it) {
      const Cached& c = cached.at(it->second);
      if (c.parent == parent && std::equal(c.tokens.begin(), c.tokens.end(), tok)) return it->second;
    }
    return -1;
  }
  void insert_cached(int32_t b, int32_t parent, const int32_t* tok) {
    Cached c;
    c.parent = parent;
    c.hash = key_hash(parent, tok);
    c.tokens.assign(tok, tok + block_size);
    index.emplace(c.hash, b);
    if (parent >= 0) cached.at(parent).children.push_back(b);
    cached.emplace(b, std::move(c));
  }
  // Forget block b's cache entry (and its evictable rank).
  void uncache(int32_t b) {
    Cached& c = cached.at(b);
    auto range = index.equal_range(c.hash);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        index.erase(it);
        break;
      }
    if (c.parent >= 0) {
      auto pit = cached.find(c.parent);
      if (pit != cached.end()) {
        auto& ch = pit->second.children;
        ch.erase(std::find(ch.begin(), ch.end(), b));
      }
    }
    if (tick_of[b] >= 0) {
      evictable.erase({tick_of[b], b});
      tick_of[b] = -1;
    }
    cached.erase(b);
  }

  // A block for a new table entry, count 1: the free list first, then the
  // least recently retired evictable block, whose cached descendants (no
  // longer reachable) go to the free list in ascending id order.
  int32_t pop() {
    int32_t b;
    if (!dev.free_stack.empty()) {
      b = dev.free_stack.back();
      dev.free_stack.pop_back();
    } else {
      b = evictable.begin()->second;
      std::vector<int32_t> below, todo(cached.at(b).children);
      while (!todo.empty()) {
        const int32_t x = todo.back();
        todo.pop_back();
        below.push_back(x);
        for (int32_t y : cached.at(x).children) todo.push_back(y);
      }
      std::sort(below.begin(), below.end());
      for (int32_t x : below) {
        uncache(x);
        dev.free_stack.push_back(x);
      }
      uncache(b);
    }
    dev.refcount[b] = 1;
    return b;
  }

  // Retire a device table: counts drop in table order, uncached blocks at
  // zero return to the free list in that order; cached blocks at zero become
  // evictable, ranked deepest first.
  void release_dev(const std::vector<int32_t>& table) {
    for (int32_t b : table)
      if (--dev.refcount[b] == 0 && !cached.count(b)) dev.free_stack.push_back(b);
    for (auto it = table.rbegin(); it != table.rend(); ++it) {
      const int32_t b = *it;
      if (dev.refcount[b] == 0 && cached.count(b) && tick_of[b] < 0) {
        tick_of[b] = tick++;
        evictable.emplace(tick_of[b], b);
      }
    }
  }

  // Free blocks that appending n_new tokens to (len, table) would consume.
  // `delta` carries count decrements from earlier sequences of the same step
  // so that a block shared by several writers is copied by all but the last.
  int64_t needs(const Seq* s, int32_t n_new, std::unordered_map<int32_t, int32_t>& delta) const {
    const int64_t len = s ? s->len : 0;
    const int64_t have = s ? (int64_t)s->table.size() : 0;
    int64_t need = (len + n_new + block_size - 1) / block_size - have;
    if (n_new > 0 && s && len % block_size != 0) {
      const int32_t last = s->table.back();
      auto it = delta.find(last);
      const int32_t d = it == delta.end() ? 0 : it->second;
      if (dev.refcount[last] + d > 1) {
        need += 1;
        delta[last] = d - 1;
      }
    }
    return need;
  }

  // Append without a capacity check; writes slots and at most one CoW pair.
  void append_unchecked(int64_t id, int32_t n_new, int64_t* slots, int32_t* cow, int32_t* n_cow) {
    append_unchecked(seqs[id], n_new, slots, cow, n_cow);
  }
  void append_unchecked(Seq& s, int32_t n_new, int64_t* slots, int32_t* cow, int32_t* n_cow) {
    const int32_t B = block_size;
    if (n_new > 0 && s.len % B != 0 && dev.refcount[s.table.back()] > 1) {
      const int32_t src = s.table.back();
      const int32_t dst = pop();
      dev.refcount[src] -= 1;
      s.table.back() = dst;
      cow[2 * *n_cow] = src;
      cow[2 * *n_cow + 1] = dst;
      *n_cow += 1;
      cow_copies += 1;
    }
    for (int32_t i = 0; i < n_new; ++i) {
      const int64_t t = (int64_t)s.len + i;
      if (t % B == 0) s.table.push_back(pop());
      slots[i] = (int64_t)s.table[t / B] * B + t % B;
    }
    s.len += n_new;
  }
};

extern "C" pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order) {
  if (num_blocks <= 0 || block_size <= 0) {
    fail(PA_ERR_INVALID, "pa_bm_create: num_blocks=%d block_size=%d must be positive", num_blocks,
         block_size);
    return nullptr;
  }
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) {
    fail(PA_ERR_INVALID, "pa_bm_create: host allocation failed");
    return nullptr;
  }
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->dev.refcount.assign(num_blocks, 0);
  bm->tick_of.assign(num_blocks, -1);
  bm->dev.free_stack.resize(num_blocks);
  if (initial_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = initial_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        fail(PA_ERR_INVALID, "pa_bm_create: initial_order is not a permutation (entry %d = %d)", i, b);
        return nullptr;
      }
      seen[b] = 1;
      bm->dev.free_stack[num_blocks - 1 - i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->dev.free_stack[num_blocks - 1 - i] = i;
  }
  return bm;
}

extern "C" void pa_bm_destroy(pa_bm* bm) { delete bm; }

pagedkv::StepPlanCache& pagedkv::step_plan_cache(pa_bm* bm) { return bm->plan_cache; }

extern "C" pa_status pa_bm_set_plan_reuse(pa_bm* bm, int32_t max_advances) {
  if (!bm || max_advances < 0) return fail(PA_ERR_INVALID, "pa_bm_set_plan_reuse: bad arguments");
  bm->plan_cache.max_advances = max_advances;
  bm->plan_cache.valid = false;
  return PA_OK;
}

extern "C" pa_status pa_bm_append(pa_bm* bm, int64_t seq, int32_t n_new, int64_t* slots_out,
                                  int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!bm || n_new < 0 || (n_new > 0 && !slots_out) || !n_cow_out)
    return fail(PA_ERR_INVALID, "pa_bm_append: bad arguments");
  *n_cow_out = 0;
  auto it = bm->seqs.find(seq);
  const pa_bm::Seq* s = it == bm->seqs.end() ? nullptr : &it->second;
  if (s && s->swapped) return fail(PA_ERR_INVALID, "pa_bm_append: sequence %lld is swapped out", (long long)seq);
  std::unordered_map<int32_t, int32_t> delta;
  const int64_t need = bm->needs(s, n_new, delta);
  if (!delta.empty() && !cow_pairs_out)
    return fail(PA_ERR_INVALID, "pa_bm_append: a copy-on-write pair is due but cow_pairs_out is NULL");
  if (need > bm->capacity()) {
    bm->alloc_failures += 1;
    return fail(PA_ERR_OOM, "pa_bm_append: sequence %lld needs %lld blocks, %lld free", (long long)seq,
                (long long)need, (long long)bm->capacity());
  }
  int32_t dummy[2];
  bm->append_unchecked(seq, n_new, slots_out, cow_pairs_out ? cow_pairs_out : dummy, n_cow_out);
  return PA_OK;
}

// One token for each of `num` sequences, resolved in `ptr` (null: a new
// sequence); all or nothing.  Listed sequences are stamped with a fresh stamp
// to find repeats in one pass (a repeat among new sequences is found by a
// sort, only when there are new ones).
static pa_status append_batch(pa_bm* bm, const int64_t* seqs, int32_t num, pa_bm::Seq* const* ptr, int64_t* slots_out,
                              int32_t* cow_pairs_out, int32_t* n_cow_out, const char* who) {
  *n_cow_out = 0;
  const uint64_t stamp = ++bm->stamp_now;
  int32_t fresh = 0;
  for (int32_t i = 0; i < num; ++i) {
    pa_bm::Seq* s = ptr[i];
    if (!s) {
      fresh += 1;
      continue;
    }
    if (s->swapped) return fail(PA_ERR_INVALID, "%s: sequence %lld is swapped out", who, (long long)seqs[i]);
    if (s->stamp == stamp) return fail(PA_ERR_INVALID, "%s: a sequence is listed twice", who);
    s->stamp = stamp;
  }
  if (fresh > 1) {
    std::vector<int64_t> ids;
    ids.reserve(fresh);
    for (int32_t i = 0; i < num; ++i)
      if (!ptr[i]) ids.push_back(seqs[i]);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return fail(PA_ERR_INVALID, "%s: a sequence is listed twice", who);
  }
  std::unordered_map<int32_t, int32_t> delta;
  int64_t need = 0;
  for (int32_t i = 0; i < num; ++i) need += bm->needs(ptr[i], 1, delta);
  if (need > bm->capacity()) {
    bm->alloc_failures += 1;
    return fail(PA_ERR_OOM, "%s: step needs %lld blocks, %lld free", who, (long long)need,
                (long long)bm->capacity());
  }
  for (int32_t i = 0; i < num; ++i) {
    if (ptr[i])
      bm->append_unchecked(*ptr[i], 1, slots_out + i, cow_pairs_out, n_cow_out);
    else
      bm->append_unchecked(seqs[i], 1, slots_out + i, cow_pairs_out, n_cow_out);
  }
  return PA_OK;
}

extern "C" pa_status pa_bm_append_step(pa_bm* bm, const int64_t* seqs, int32_t num, int64_t* slots_out,
                                       int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!bm || num < 0 || (num > 0 && (!seqs || !slots_out || !cow_pairs_out)) || !n_cow_out)
    return fail(PA_ERR_INVALID, "pa_bm_append_step: bad arguments");
  std::vector<pa_bm::Seq*> ptr(num);
  for (int32_t i = 0; i < num; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    ptr[i] = it == bm->seqs.end() ? nullptr : &it->second;
  }
  return append_batch(bm, seqs, num, ptr.data(), slots_out, cow_pairs_out, n_cow_out, "pa_bm_append_step");
}

pa_status pagedkv::bm_step_resolve(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* lens, const char* who) {
  bm->step_seqs.assign(num, nullptr);
  for (int32_t i = 0; i < num; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "%s: unknown sequence %lld", who, (long long)seqs[i]);
    if (it->second.swapped) return fail(PA_ERR_INVALID, "%s: sequence %lld is swapped out", who, (long long)seqs[i]);
    bm->step_seqs[i] = &it->second;
    lens[i] = it->second.len;
  }
  return PA_OK;
}

pa_status pagedkv::bm_step_append(pa_bm* bm, const int64_t* seqs, int32_t num, int64_t* slots, int32_t* cows,
                                  int32_t* n_cows, const char* who) {
  if ((int32_t)bm->step_seqs.size() != num) return fail(PA_ERR_INVALID, "%s: batch not resolved", who);
  return append_batch(bm, seqs, num, bm->step_seqs.data(), slots, cows, n_cows, who);
}

pa_status pagedkv::bm_step_tables(pa_bm* bm, int32_t num, int32_t* tables, int32_t max_blocks, const char* who) {
  if ((int32_t)bm->step_seqs.size() != num) return fail(PA_ERR_INVALID, "%s: batch not resolved", who);
  for (int32_t i = 0; i < num; ++i) {
    const std::vector<int32_t>& t = bm->step_seqs[i]->table;
    if ((int64_t)t.size() > max_blocks)
      return fail(PA_ERR_INVALID, "%s: a sequence holds %zu blocks, rows hold %d", who, t.size(), max_blocks);
    if (!t.empty()) std::memcpy(tables + (int64_t)i * max_blocks, t.data(), sizeof(int32_t) * t.size());
  }
  return PA_OK;
}

extern "C" pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_fork: null manager");
  auto p = bm->seqs.find(parent);
  if (p == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "pa_bm_fork: unknown parent %lld", (long long)parent);
  if (p->second.swapped) return fail(PA_ERR_INVALID, "pa_bm_fork: parent %lld is swapped out", (long long)parent);
  if (bm->seqs.count(child)) return fail(PA_ERR_INVALID, "pa_bm_fork: child %lld exists", (long long)child);
  pa_bm::Seq copy = p->second;
  for (int32_t b : copy.table) bm->dev.refcount[b] += 1;
  bm->seqs.emplace(child, std::move(copy));
  return PA_OK;
}

extern "C" pa_status pa_bm_free(pa_bm* bm, int64_t seq) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_free: null manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_OK;
  if (it->second.swapped) {
    bm->host.release(it->second.table);
    bm->num_swapped -= 1;
  } else {
    bm->release_dev(it->second.table);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

extern "C" int32_t pa_bm_table(const pa_bm* bm, int64_t seq, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  const auto& t = it->second.table;
  const int32_t n = (int32_t)t.size();
  if (out && cap > 0) std::memcpy(out, t.data(), sizeof(int32_t) * std::min(n, cap));
  return n;
}

extern "C" pa_status pa_bm_export(const pa_bm* bm, const int64_t* seqs, int32_t num, int32_t max_blocks,
                                  int32_t* tables_out, int32_t* lens_out) {
  if (!bm || num < 0 || max_blocks < 0 || (num > 0 && (!seqs || !tables_out || !lens_out)))
    return fail(PA_ERR_INVALID, "pa_bm_export: bad arguments");
  for (int32_t i = 0; i < num; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_NOT_FOUND, "pa_bm_export: unknown sequence %lld", (long long)seqs[i]);
    if (it->second.swapped)
      return fail(PA_ERR_INVALID, "pa_bm_export: sequence %lld is swapped out", (long long)seqs[i]);
    const auto& t = it->second.table;
    if ((int64_t)t.size() > max_blocks)
      return fail(PA_ERR_INVALID, "pa_bm_export: sequence %lld has %zu blocks > max_blocks %d",
                  (long long)seqs[i], t.size(), max_blocks);
  }
  for (int32_t i = 0; i < num; ++i) {
    const auto& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    std::fill(row, row + max_blocks, 0);
    std::copy(s.table.begin(), s.table.end(), row);
    lens_out[i] = s.len;
  }
  return PA_OK;
}

extern "C" pa_status pa_bm_prefix_groups(const pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* group_out,
                                         int32_t* prefix_tokens_out) {
  if (!bm || num < 0 || (num > 0 && (!seqs || !group_out || !prefix_tokens_out)))
    return fail(PA_ERR_INVALID, "pa_bm_prefix_groups: bad arguments");
  std::vector<const pa_bm::Seq*> batch(num);
  for (int32_t i = 0; i < num; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end())
      return fail(PA_ERR_NOT_FOUND, "pa_bm_prefix_groups: unknown sequence %lld", (long long)seqs[i]);
    if (it->second.swapped)
      return fail(PA_ERR_INVALID, "pa_bm_prefix_groups: sequence %lld is swapped out", (long long)seqs[i]);
    batch[i] = &it->second;
  }
  // Group by first physical block: the batch position of the first sequence
  // holding that block.
  std::unordered_map<int32_t, int32_t> first_pos;
  std::vector<int32_t> members(num, 0);
  for (int32_t i = 0; i < num; ++i) {
    group_out[i] = -1;
    prefix_tokens_out[i] = 0;
    if (batch[i]->table.empty()) continue;
    auto ins = first_pos.emplace(batch[i]->table[0], i);
    group_out[i] = ins.first->second;
    members[ins.first->second] += 1;
  }
  // Shared tokens of a group: its longest common run of leading blocks,
  // in tokens, capped by the shortest member.
  std::vector<int64_t> common(num, -1), shortest(num, INT64_MAX);
  for (int32_t i = 0; i < num; ++i) {
    const int32_t g = group_out[i];
    if (g < 0) continue;
    if (members[g] < 2) {
      group_out[i] = -1;
      continue;
    }
    const auto& lead = batch[g]->table;
    const auto& t = batch[i]->table;
    int64_t c = 0;
    while (c < (int64_t)t.size() && c < (int64_t)lead.size() && t[c] == lead[c]) ++c;
    common[g] = common[g] < 0 ? c : std::min(common[g], c);
    shortest[g] = std::min<int64_t>(shortest[g], batch[i]->len);
  }
  for (int32_t i = 0; i < num; ++i) {
    const int32_t g = group_out[i];
    if (g >= 0) prefix_tokens_out[i] = (int32_t)std::min<int64_t>(common[g] * bm->block_size, shortest[g]);
  }
  return PA_OK;
}

extern "C" int32_t pa_bm_block_size(const pa_bm* bm) { return bm ? bm->block_size : -1; }

extern "C" int32_t pa_bm_len(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

extern "C" int32_t pa_bm_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->dev.refcount[block];
}

extern "C" void pa_bm_get_stats(const pa_bm* bm, pa_bm_stats* out) {
  if (!bm || !out) return;
  std::memset(out, 0, sizeof(*out));
  out->num_blocks = bm->num_blocks;
  out->free_blocks = (int32_t)bm->dev.free_stack.size();
  out->used_blocks = bm->num_blocks - out->free_blocks - (int32_t)bm->evictable.size();
  out->num_seqs = (int32_t)bm->seqs.size();
  for (const auto& kv : bm->seqs) out->logical_tokens += kv.second.len;
  for (int32_t c : bm->dev.refcount) out->shared_blocks += c > 1;
  out->alloc_failures = bm->alloc_failures;
  out->cow_copies = bm->cow_copies;
  out->host_blocks = (int32_t)bm->host.refcount.size();
  out->free_host_blocks = (int32_t)bm->host.free_stack.size();
  out->swapped_seqs = bm->num_swapped;
  out->swap_out_blocks = bm->swap_out_blocks;
  out->swap_in_blocks = bm->swap_in_blocks;
  out->cached_blocks = (int32_t)bm->cached.size();
  out->evictable_blocks = (int32_t)bm->evictable.size();
  out->prefix_query_tokens = bm->prefix_query_tokens;
  out->prefix_hit_tokens = bm->prefix_hit_tokens;
}

namespace {

// Counts of one pool against the tables of the sequences in `swapped` state.
pa_status check_pool(const pa_bm* bm, const pa_bm::Pool& pool, bool swapped, const char* what) {
  const int32_t n = (int32_t)pool.refcount.size();
  std::vector<int32_t> named(n, 0);
  for (const auto& kv : bm->seqs) {
    const auto& s = kv.second;
    if (s.swapped != swapped) continue;
    const int64_t expect = ((int64_t)s.len + bm->block_size - 1) / bm->block_size;
    if ((int64_t)s.table.size() != expect)
      return fail(PA_ERR_INVALID, "pa_bm_check: sequence %lld length %d has %zu %s blocks, expected %lld",
                  (long long)kv.first, s.len, s.table.size(), what, (long long)expect);
    for (int32_t b : s.table) {
      if (b < 0 || b >= n)
        return fail(PA_ERR_INVALID, "pa_bm_check: sequence %lld names %s block %d", (long long)kv.first, what, b);
      named[b] += 1;
    }
  }
  std::vector<char> is_free(n, 0);
  for (int32_t b : pool.free_stack) {
    if (b < 0 || b >= n || is_free[b])
      return fail(PA_ERR_INVALID, "pa_bm_check: %s block %d is on the free list twice or out of range", what, b);
    is_free[b] = 1;
  }
  if (!swapped) {
    for (const auto& e : bm->evictable) {
      const int32_t b = e.second;
      if (b < 0 || b >= n || is_free[b] || bm->tick_of[b] != e.first)
        return fail(PA_ERR_INVALID, "pa_bm_check: evictable block %d is free, out of range or misranked", b);
      is_free[b] = 2;
    }
  }
  for (int32_t b = 0; b < n; ++b) {
    if (named[b] != pool.refcount[b])
      return fail(PA_ERR_INVALID, "pa_bm_check: %s block %d count %d but %d tables name it", what, b,
                  pool.refcount[b], named[b]);
    if ((named[b] == 0) != (is_free[b] != 0))
      return fail(PA_ERR_INVALID, "pa_bm_check: %s block %d is %s", what, b,
                  named[b] ? "named and free" : "neither named nor free (leaked)");
  }
  return PA_OK;
}

// The prefix cache's own invariants: entries and the hash index agree, every
// entry's parent is cached and lists it as a child, a cached block has count
// zero exactly when it is evictable, and only cached blocks are evictable.
pa_status check_cache(const pa_bm* bm) {
  if (bm->index.size() != bm->cached.size())
    return fail(PA_ERR_INVALID, "pa_bm_check: %zu index entries for %zu cached blocks", bm->index.size(),
                bm->cached.size());
  for (const auto& kv : bm->cached) {
    const int32_t b = kv.first;
    const auto& c = kv.second;
    if ((int32_t)c.tokens.size() != bm->block_size || c.hash != bm->key_hash(c.parent, c.tokens.data()) ||
        bm->lookup(c.parent, c.tokens.data()) != b)
      return fail(PA_ERR_INVALID, "pa_bm_check: cached block %d is not found by its own key", b);
    if (c.parent >= 0) {
      auto p = bm->cached.find(c.parent);
      if (p == bm->cached.end() ||
          std::count(p->second.children.begin(), p->second.children.end(), b) != 1)
        return fail(PA_ERR_INVALID, "pa_bm_check: cached block %d has no cached parent listing it", b);
    }
    for (int32_t ch : c.children)
      if (!bm->cached.count(ch) || bm->cached.at(ch).parent != b)
        return fail(PA_ERR_INVALID, "pa_bm_check: cached block %d lists a stale child %d", b, ch);
    if ((bm->dev.refcount[b] == 0) != (bm->tick_of[b] >= 0))
      return fail(PA_ERR_INVALID, "pa_bm_check: cached block %d count %d but %sevictable", b, bm->dev.refcount[b],
                  bm->tick_of[b] >= 0 ? "" : "not ");
  }
  for (int32_t b = 0; b < bm->num_blocks; ++b)
    if (bm->tick_of[b] >= 0 && !bm->cached.count(b))
      return fail(PA_ERR_INVALID, "pa_bm_check: block %d is evictable but not cached", b);
  return PA_OK;
}

// Copy the distinct blocks of the listed tables from pool `src` to pool
// `dst` (one destination block each, in batch and table order), point the
// tables at the copies and retire the source tables.  The caller has checked
// states, distinctness and capacity.
void move_tables(pa_bm* bm, const std::vector<pa_bm::Seq*>& list, pa_bm::Pool& dst, bool to_host,
                 int32_t* pairs) {
  std::unordered_map<int32_t, int32_t> mapping;
  int32_t n = 0;
  std::vector<std::vector<int32_t>> old(list.size());
  for (size_t i = 0; i < list.size(); ++i) {
    pa_bm::Seq* s = list[i];
    old[i] = s->table;
    for (int32_t& b : s->table) {
      auto ins = mapping.emplace(b, -1);
      if (ins.second) {
        int32_t d;
        if (to_host) {
          d = dst.free_stack.back();
          dst.free_stack.pop_back();
        } else {
          d = bm->pop();
          dst.refcount[d] = 0;
        }
        ins.first->second = d;
        pairs[2 * n] = b;
        pairs[2 * n + 1] = d;
        ++n;
      }
      b = ins.first->second;
      dst.refcount[b] += 1;
    }
    s->swapped = to_host;
  }
  for (const auto& t : old) {
    if (to_host)
      bm->release_dev(t);
    else
      bm->host.release(t);
  }
  bm->num_swapped += to_host ? (int32_t)list.size() : -(int32_t)list.size();
}

pa_status swap(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* pairs_out, int32_t cap_pairs,
               int32_t* n_pairs_out, bool to_host, const char* who) {
  if (!bm || num < 0 || (num > 0 && !seqs) || !n_pairs_out || cap_pairs < 0 || (cap_pairs > 0 && !pairs_out))
    return fail(PA_ERR_INVALID, "%s: bad arguments", who);
  *n_pairs_out = 0;
  std::vector<int64_t> sorted(seqs, seqs + num);
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
    return fail(PA_ERR_INVALID, "%s: a sequence is listed twice", who);
  std::vector<pa_bm::Seq*> list(num);
  std::unordered_map<int32_t, char> distinct;
  for (int32_t i = 0; i < num; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PA_ERR_NOT_FOUND, "%s: unknown sequence %lld", who, (long long)seqs[i]);
    if (it->second.swapped == to_host)
      return fail(PA_ERR_INVALID, "%s: sequence %lld is %s", who, (long long)seqs[i],
                  to_host ? "already swapped out" : "not swapped out");
    list[i] = &it->second;
    for (int32_t b : it->second.table) distinct.emplace(b, 0);
  }
  pa_bm::Pool& dst = to_host ? bm->host : bm->dev;
  const int64_t need = (int64_t)distinct.size();
  const int64_t room = to_host ? (int64_t)bm->host.free_stack.size() : bm->capacity();
  if (need > room)
    return fail(PA_ERR_OOM, "%s: %lld blocks to copy, %lld free %s blocks", who, (long long)need, (long long)room,
                to_host ? "host" : "device");
  if (need > cap_pairs)
    return fail(PA_ERR_INVALID, "%s: %lld pairs due, cap_pairs is %d", who, (long long)need, cap_pairs);
  move_tables(bm, list, dst, to_host, pairs_out);
  *n_pairs_out = (int32_t)need;
  (to_host ? bm->swap_out_blocks : bm->swap_in_blocks) += need;
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_bm_set_host_blocks(pa_bm* bm, int32_t num_host_blocks) {
  if (!bm || num_host_blocks < 0) return fail(PA_ERR_INVALID, "pa_bm_set_host_blocks: bad arguments");
  if (bm->num_swapped) return fail(PA_ERR_INVALID, "pa_bm_set_host_blocks: %d sequences are swapped out", bm->num_swapped);
  bm->host.reset(num_host_blocks);
  return PA_OK;
}

extern "C" pa_status pa_bm_swap_out(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* pairs_out, int32_t cap_pairs,
                                    int32_t* n_pairs_out) {
  return swap(bm, seqs, num, pairs_out, cap_pairs, n_pairs_out, true, "pa_bm_swap_out");
}

extern "C" pa_status pa_bm_swap_in(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* pairs_out, int32_t cap_pairs,
                                   int32_t* n_pairs_out) {
  return swap(bm, seqs, num, pairs_out, cap_pairs, n_pairs_out, false, "pa_bm_swap_in");
}

extern "C" int32_t pa_bm_swapped(const pa_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : (it->second.swapped ? 1 : 0);
}

extern "C" int32_t pa_bm_host_refcount(const pa_bm* bm, int32_t host_block) {
  if (!bm || host_block < 0 || host_block >= (int32_t)bm->host.refcount.size()) return -1;
  return bm->host.refcount[host_block];
}

extern "C" pa_status pa_bm_enable_prefix_cache(pa_bm* bm) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_enable_prefix_cache: null manager");
  if (!bm->seqs.empty())
    return fail(PA_ERR_INVALID, "pa_bm_enable_prefix_cache: enable it before any sequence exists");
  bm->prefix_cache = true;
  return PA_OK;
}

extern "C" pa_status pa_bm_append_prompt(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t n,
                                         int64_t* slots_out, int32_t* n_cached_out) {
  if (!bm || n < 0 || (n > 0 && (!tokens || !slots_out)) || !n_cached_out)
    return fail(PA_ERR_INVALID, "pa_bm_append_prompt: bad arguments");
  *n_cached_out = 0;
  if (!bm->prefix_cache) return fail(PA_ERR_INVALID, "pa_bm_append_prompt: the prefix cache is not enabled");
  if (bm->seqs.count(seq)) return fail(PA_ERR_INVALID, "pa_bm_append_prompt: sequence %lld exists", (long long)seq);
  const int32_t B = bm->block_size;
  const int64_t blocks = ((int64_t)n + B - 1) / B;
  // Leading full blocks already cached, at most (n - 1) / B of them: the
  // prompt's last token is always computed.
  std::vector<int32_t> hits;
  int32_t parent = -1;
  int64_t revived = 0;
  for (int64_t j = 0; n > 0 && j < (n - 1) / B; ++j) {
    const int32_t b = bm->lookup(parent, tokens + j * B);
    if (b < 0) break;
    hits.push_back(b);
    revived += bm->dev.refcount[b] == 0;
    parent = b;
  }
  const int64_t need = blocks - (int64_t)hits.size();
  if (need > bm->capacity() - revived) {
    bm->alloc_failures += 1;
    return fail(PA_ERR_OOM, "pa_bm_append_prompt: sequence %lld needs %lld blocks, %lld free", (long long)seq,
                (long long)need, (long long)(bm->capacity() - revived));
  }
  bm->prefix_query_tokens += n;
  bm->prefix_hit_tokens += (int64_t)hits.size() * B;
  for (int32_t b : hits) {
    if (bm->tick_of[b] >= 0) {
      bm->evictable.erase({bm->tick_of[b], b});
      bm->tick_of[b] = -1;
    }
    bm->dev.refcount[b] += 1;
  }
  pa_bm::Seq s;
  s.table = hits;
  s.len = n;
  while ((int64_t)s.table.size() < blocks) s.table.push_back(bm->pop());
  // The prompt's new full blocks become cached (unless that content already is).
  for (int64_t j = (int64_t)hits.size(); j < n / B; ++j) {
    const int32_t par = j ? s.table[j - 1] : -1;
    if ((par < 0 || bm->cached.count(par)) && bm->lookup(par, tokens + j * B) < 0)
      bm->insert_cached(s.table[j], par, tokens + j * B);
  }
  const int64_t cached_tokens = (int64_t)hits.size() * B;
  for (int64_t t = 0; t < n; ++t) slots_out[t] = t < cached_tokens ? -1 : (int64_t)s.table[t / B] * B + t % B;
  bm->seqs.emplace(seq, std::move(s));
  *n_cached_out = (int32_t)cached_tokens;
  return PA_OK;
}

extern "C" int32_t pa_bm_cached(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->cached.count(block) ? 1 : 0;
}

extern "C" pa_status pa_bm_check(const pa_bm* bm) {
  if (!bm) return fail(PA_ERR_INVALID, "pa_bm_check: null manager");
  int32_t swapped = 0;
  for (const auto& kv : bm->seqs) swapped += kv.second.swapped;
  if (swapped != bm->num_swapped)
    return fail(PA_ERR_INVALID, "pa_bm_check: %d swapped sequences, counter says %d", swapped, bm->num_swapped);
  if (pa_status st = check_pool(bm, bm->dev, false, "device")) return st;
  if (pa_status st = check_pool(bm, bm->host, true, "host")) return st;
  return check_cache(bm);
}
