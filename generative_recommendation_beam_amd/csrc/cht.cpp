// Host-side batch former: Feather's chunked hash structure (Feather page,
// "Requests of a Feather Must Flock Together", Metodologia 1). Requests are
// kept as cumulative hashes over full token blocks, so one 64-bit value names
// a whole prefix; the active batch is a working set of hash -> count; waiting
// requests sit in a min-heap keyed by (missing blocks, arrival). Admitting or
// finishing a request changes the coverage of only the hashes it holds, and
// only the waiting requests holding those hashes get a new key, pushed as a
// fresh heap entry (older entries become stale and are skipped when they
// reach the top). Finding the best request is a heap top: O(log W) amortized.
// Its batches map onto the attention path directly: a group of sequences with
// a common prefix is one request with its sequences as beams.
#include <cstdint>
#include <new>
#include <queue>
#include <set>
#include <unordered_map>
#include <vector>

#include "xattn.h"

namespace {

inline uint64_t mix64(uint64_t x) {  // splitmix64 finalizer
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

struct Req {
  std::vector<uint64_t> hashes;  // cumulative hash of blocks 0..i
  int64_t seq;                   // arrival order
  int64_t missing;
  uint32_t version;
  bool waiting;
};

struct Entry {
  int64_t missing, seq, id;
  uint32_t version;
  bool operator>(const Entry& o) const {
    if (missing != o.missing) return missing > o.missing;
    return seq > o.seq;
  }
};

}  // namespace

struct xattn_cht {
  int block;
  int64_t next_seq = 0;
  std::unordered_map<int64_t, Req> reqs;
  std::unordered_map<uint64_t, int64_t> working;                   // hash -> active requests holding it
  std::unordered_map<uint64_t, std::vector<int64_t>> holders;      // hash -> waiting requests holding it
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap;
  std::set<std::pair<int64_t, int64_t>> fifo;                      // waiting (seq, id)
  int64_t n_active = 0;

  void push(int64_t id, Req& r) {
    ++r.version;
    heap.push(Entry{r.missing, r.seq, id, r.version});
  }
  // Coverage of hash h changed between 0 and 1: every waiting holder moves.
  void recount(uint64_t h, int64_t delta) {
    auto it = holders.find(h);
    if (it == holders.end()) return;
    std::vector<int64_t>& v = it->second;
    size_t keep = 0;
    for (size_t i = 0; i < v.size(); ++i) {
      auto rq = reqs.find(v[i]);
      if (rq == reqs.end() || !rq->second.waiting) continue;  // drop ids no longer waiting
      v[keep++] = v[i];
      rq->second.missing += delta;
      push(v[i], rq->second);
    }
    v.resize(keep);
    if (v.empty()) holders.erase(it);
  }
  void skip_stale() {
    while (!heap.empty()) {
      const Entry& e = heap.top();
      auto it = reqs.find(e.id);
      if (it != reqs.end() && it->second.waiting && it->second.version == e.version) return;
      heap.pop();
    }
  }
  void admit(int64_t id, Req& r) {
    r.waiting = false;
    fifo.erase({r.seq, id});
    ++n_active;
    // A hash is listed once per request even if the request repeats it.
    for (size_t i = 0; i < r.hashes.size(); ++i) {
      const uint64_t h = r.hashes[i];
      if (++working[h] == 1) recount(h, -1);
    }
  }
};

extern "C" {

xattn_status xattn_cht_create(int32_t block_size, xattn_cht** out) {
  if (!out) return XATTN_ERR_INVALID_ARG;
  *out = nullptr;
  if (block_size < 1) return XATTN_ERR_INVALID_ARG;
  xattn_cht* c = new (std::nothrow) xattn_cht();
  if (!c) return XATTN_ERR_UNSUPPORTED;
  c->block = block_size;
  *out = c;
  return XATTN_OK;
}

xattn_status xattn_cht_destroy(xattn_cht* c) {
  delete c;
  return XATTN_OK;
}

xattn_status xattn_cht_insert(xattn_cht* c, int64_t id, const int32_t* tokens, int64_t n_tokens) {
  if (!c || n_tokens < 0 || (n_tokens > 0 && !tokens) || id < 0) return XATTN_ERR_INVALID_ARG;
  if (c->reqs.count(id)) return XATTN_ERR_INVALID_ARG;
  Req r;
  const int64_t nb = n_tokens / c->block;
  r.hashes.resize((size_t)nb);
  uint64_t h = 0x6A09E667F3BCC908ull;
  for (int64_t b = 0; b < nb; ++b) {
    for (int i = 0; i < c->block; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[b * c->block + i]);
    r.hashes[(size_t)b] = h;
  }
  r.seq = c->next_seq++;
  r.missing = 0;
  for (uint64_t x : r.hashes)
    if (!c->working.count(x)) ++r.missing;
  r.version = 0;
  r.waiting = true;
  for (uint64_t x : r.hashes) c->holders[x].push_back(id);
  auto it = c->reqs.emplace(id, std::move(r)).first;
  c->fifo.insert({it->second.seq, id});
  c->push(id, it->second);
  return XATTN_OK;
}

xattn_status xattn_cht_best(xattn_cht* c, int64_t* id, int64_t* missing) {
  if (!c || !id || !missing) return XATTN_ERR_INVALID_ARG;
  c->skip_stale();
  if (c->heap.empty()) {
    *id = -1;
    *missing = -1;
    return XATTN_OK;
  }
  *id = c->heap.top().id;
  *missing = c->heap.top().missing;
  return XATTN_OK;
}

xattn_status xattn_cht_admit(xattn_cht* c, int64_t id) {
  if (!c) return XATTN_ERR_INVALID_ARG;
  auto it = c->reqs.find(id);
  if (it == c->reqs.end() || !it->second.waiting) return XATTN_ERR_INVALID_ARG;
  c->admit(id, it->second);
  return XATTN_OK;
}

xattn_status xattn_cht_complete(xattn_cht* c, int64_t id) {
  if (!c) return XATTN_ERR_INVALID_ARG;
  auto it = c->reqs.find(id);
  if (it == c->reqs.end() || it->second.waiting) return XATTN_ERR_INVALID_ARG;
  std::vector<uint64_t> hs = std::move(it->second.hashes);
  c->reqs.erase(it);
  --c->n_active;
  for (uint64_t h : hs) {
    auto w = c->working.find(h);
    if (--w->second == 0) {
      c->working.erase(w);
      c->recount(h, +1);
    }
  }
  return XATTN_OK;
}

xattn_status xattn_cht_form_batch(xattn_cht* c, int32_t max_batch, int64_t max_missing, int64_t* out_ids,
                                  int32_t* out_n) {
  if (!c || !out_n || max_batch < 0 || (max_batch > 0 && !out_ids)) return XATTN_ERR_INVALID_ARG;
  int32_t n = 0;
  if (c->n_active == 0 && !c->fifo.empty() && max_batch > 0) {
    const int64_t first = c->fifo.begin()->second;
    c->admit(first, c->reqs[first]);
    out_ids[n++] = first;
  }
  while (c->n_active < max_batch) {
    c->skip_stale();
    if (c->heap.empty() || c->heap.top().missing > max_missing) break;
    const int64_t id = c->heap.top().id;
    c->admit(id, c->reqs[id]);
    out_ids[n++] = id;
  }
  *out_n = n;
  return XATTN_OK;
}

}  // extern "C"
