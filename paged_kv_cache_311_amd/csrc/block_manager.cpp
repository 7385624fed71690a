// Host-side management of a paged KV-cache pool, and a decode-loop
// simulator comparing paged allocation with maximum-length reservations.
// The interface and its behaviour are documented in pkv_block_manager.h.
//
// The pool is a free list of fixed-size blocks; each sequence is a table
// of block ids plus a length.  A block shared by several sequences (after
// a fork) carries a reference count, and the first write into a shared,
// partially filled block copies it ("Your GPU was mostly empty..." [TEQ],
// "Paging's second gift: copy-on-write"; "PagedAttention KV cache memory
// management" [AITJ], "A request lifecycle: allocation, growth, sharing and
// release").  A sequence can leave empty slots only in its last block
// ([TEQ], "The OS already solved this in the 1960s"), which the simulator
// checks at every step.

#include "../../include/pkv_block_manager.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

struct pkv_bm {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  int32_t num_blocks = 0, block_size = 0;
  std::vector<int32_t> free_list;  // a stack: the last block freed is taken first
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    refcount[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refcount[b] == 0) free_list.push_back(b);
  }
};

extern "C" {

int pkv_bm_abi_version(void) { return 3; }

pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_bm* bm = new (std::nothrow) pkv_bm();
  if (!bm) return nullptr;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->refcount.assign(num_blocks, 0);
    bm->free_list.resize(num_blocks);
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list[i] = num_blocks - 1 - i;
  } catch (...) {
    delete bm;
    return nullptr;
  }
  return bm;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

int32_t pkv_bm_num_blocks(const pkv_bm* bm) { return bm ? bm->num_blocks : 0; }
int32_t pkv_bm_block_size(const pkv_bm* bm) { return bm ? bm->block_size : 0; }
int32_t pkv_bm_num_free(const pkv_bm* bm) {
  return bm ? (int32_t)bm->free_list.size() : 0;
}
int32_t pkv_bm_num_sequences(const pkv_bm* bm) { return bm ? (int32_t)bm->seqs.size() : 0; }

int32_t pkv_bm_refcount(const pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

int32_t pkv_bm_shared_flags(const pkv_bm* bm, uint8_t* flags, int32_t n) {
  if (!bm || !flags || n < bm->num_blocks) return PKV_BM_INVALID;
  for (int32_t b = 0; b < bm->num_blocks; ++b) flags[b] = bm->refcount[b] > 1 ? 1 : 0;
  return bm->num_blocks;
}

int pkv_bm_prefix_groups(const pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* order,
                         int32_t* group_start, int32_t* prefix_blocks, int32_t* num_groups) {
  if (!bm || n < 0 || !group_start || !num_groups ||
      (n > 0 && (!seq_ids || !order || !prefix_blocks)))
    return PKV_BM_INVALID;
  std::vector<const pkv_bm::Seq*> q(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return PKV_BM_INVALID;
    q[i] = &it->second;
  }
  // a sequence's key: its first block when that block is full and shared
  const int64_t kNone = INT64_MAX;
  std::vector<int64_t> key(n);
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq& s = *q[i];
    key[i] = s.len >= bm->block_size && bm->refcount[s.blocks[0]] > 1 ? s.blocks[0] : kNone;
  }
  std::vector<int32_t> ord(n);
  for (int32_t i = 0; i < n; ++i) ord[i] = i;
  std::stable_sort(ord.begin(), ord.end(),
                   [&](int32_t a, int32_t b) { return key[a] < key[b]; });
  int32_t g = 0;
  group_start[0] = 0;
  for (int32_t i = 0; i < n;) {
    int32_t e = i + 1;
    if (key[ord[i]] != kNone)
      while (e < n && key[ord[e]] == key[ord[i]]) ++e;
    int32_t pb = 0;
    if (e - i >= 2) {
      int64_t full = INT64_MAX;
      for (int32_t k = i; k < e; ++k) full = std::min(full, q[ord[k]]->len / bm->block_size);
      const std::vector<int32_t>& lead = q[ord[i]]->blocks;
      while (pb < full) {
        bool same = true;
        for (int32_t k = i + 1; k < e && same; ++k) same = q[ord[k]]->blocks[pb] == lead[pb];
        if (!same) break;
        ++pb;
      }
    }
    prefix_blocks[g] = pb;
    group_start[++g] = e;
    i = e;
  }
  for (int32_t i = 0; i < n; ++i) order[i] = ord[i];
  *num_groups = g;
  return PKV_BM_OK;
}

int pkv_bm_add_sequence(pkv_bm* bm, int64_t seq_id, int64_t num_tokens) {
  if (!bm || num_tokens < 0 || bm->seqs.count(seq_id)) return PKV_BM_INVALID;
  const int64_t need = (num_tokens + bm->block_size - 1) / bm->block_size;
  if (need > (int64_t)bm->free_list.size()) return PKV_BM_NO_BLOCKS;
  pkv_bm::Seq q;
  q.blocks.reserve(need);
  for (int64_t i = 0; i < need; ++i) q.blocks.push_back(bm->take());
  q.len = num_tokens;
  bm->seqs.emplace(seq_id, std::move(q));
  return PKV_BM_OK;
}

int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child) {
  if (!bm || parent == child || bm->seqs.count(child)) return PKV_BM_INVALID;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PKV_BM_INVALID;
  pkv_bm::Seq q = it->second;
  for (int32_t b : q.blocks) ++bm->refcount[b];
  bm->seqs.emplace(child, std::move(q));
  return PKV_BM_OK;
}

int pkv_bm_append_slot(pkv_bm* bm, int64_t seq_id, int64_t* slot, int32_t* cow_src,
                       int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PKV_BM_INVALID;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_BM_INVALID;
  pkv_bm::Seq& q = it->second;
  const int64_t off = q.len % bm->block_size;
  *cow_src = *cow_dst = -1;
  if (off == 0) {  // no block yet, or the last one is full: a fresh block
    if (bm->free_list.empty()) return PKV_BM_NO_BLOCKS;
    q.blocks.push_back(bm->take());
  } else if (bm->refcount[q.blocks.back()] > 1) {  // first write into a shared block
    if (bm->free_list.empty()) return PKV_BM_NO_BLOCKS;
    const int32_t old = q.blocks.back();
    const int32_t fresh = bm->take();
    --bm->refcount[old];  // others still hold it
    q.blocks.back() = fresh;
    *cow_src = old;
    *cow_dst = fresh;
  }
  *slot = (int64_t)q.blocks.back() * bm->block_size + off;
  ++q.len;
  return PKV_BM_OK;
}

int pkv_bm_append_slots(pkv_bm* bm, const int64_t* seq_ids, int32_t n, int64_t* slots,
                        int64_t* cow_pairs, int32_t* num_pairs, int32_t* num_done) {
  if (!bm || n < 0 || (n > 0 && (!seq_ids || !slots || !cow_pairs)) || !num_pairs ||
      !num_done)
    return PKV_BM_INVALID;
  *num_pairs = 0;
  *num_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t src, dst;
    const int rc = pkv_bm_append_slot(bm, seq_ids[i], &slots[i], &src, &dst);
    if (rc != PKV_BM_OK) return rc;
    if (src >= 0) {
      cow_pairs[2 * *num_pairs] = src;
      cow_pairs[2 * *num_pairs + 1] = dst;
      ++*num_pairs;
    }
    *num_done = i + 1;
  }
  return PKV_BM_OK;
}

int pkv_bm_free_sequence(pkv_bm* bm, int64_t seq_id) {
  if (!bm) return PKV_BM_INVALID;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_BM_INVALID;
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (auto b = blocks.rbegin(); b != blocks.rend(); ++b) bm->drop(*b);
  bm->seqs.erase(it);
  return PKV_BM_OK;
}

int64_t pkv_bm_seq_len(const pkv_bm* bm, int64_t seq_id) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_bm_block_table(const pkv_bm* bm, int64_t seq_id, int32_t* table, int32_t width) {
  if (!bm || width < 0 || (width > 0 && !table)) return -1;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return -1;
  const std::vector<int32_t>& blocks = it->second.blocks;
  if ((int64_t)blocks.size() > width) return -1;
  std::copy(blocks.begin(), blocks.end(), table);
  std::fill(table + blocks.size(), table + width, -1);
  return (int32_t)blocks.size();
}

int pkv_bm_block_tables(const pkv_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* tables,
                        int32_t width, int32_t* lens) {
  if (!bm || n < 0 || width < 0 || (n > 0 && (!seq_ids || !tables || !lens)))
    return PKV_BM_INVALID;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t L = pkv_bm_seq_len(bm, seq_ids[i]);
    if (L < 0 || L > INT32_MAX) return PKV_BM_INVALID;
    if (pkv_bm_block_table(bm, seq_ids[i], tables + (int64_t)i * width, width) < 0)
      return PKV_BM_INVALID;
    lens[i] = (int32_t)L;
  }
  return PKV_BM_OK;
}

// ------------------------------------------------------------- simulator --
namespace {

// splitmix64: a small, fully specified generator, so a seed gives the same
// stream on every platform.
struct SplitMix {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double unit() { return (next() >> 11) * (1.0 / 9007199254740992.0); }  // [0, 1)
};

struct Request {
  int64_t L, P;  // final length, prompt length
};

std::vector<Request> draw_requests(const pkv_sim_config& c) {
  SplitMix g{c.seed};
  std::vector<Request> r(c.num_requests);
  const double pi2 = 6.283185307179586;
  for (auto& q : r) {
    int64_t L;
    if (c.lengths == PKV_SIM_UNIFORM) {
      L = c.min_len + (int64_t)(g.next() % (uint64_t)(c.max_len - c.min_len + 1));
    } else {  // Box-Muller
      const double u1 = 1.0 - g.unit(), u2 = g.unit();
      const double z = std::sqrt(-2.0 * std::log(u1)) * std::cos(pi2 * u2);
      L = (int64_t)std::nearbyint(std::exp(std::log(c.median) + c.sigma * z));
      L = std::min<int64_t>(std::max<int64_t>(L, c.min_len), c.max_len);
    }
    q.L = L;  // >= 2: at least one prompt token and one generated token
    q.P = std::max<int64_t>(1, std::min<int64_t>(L - 1, (int64_t)std::nearbyint(c.prompt_fraction * L)));
  }
  return r;
}

struct Tally {
  double held = 0, reserved = 0, batch = 0;
  int64_t steps = 0;
  int32_t max_batch = 0;
  void step(double h, double r, int32_t b) {
    held += h;
    reserved += r;
    batch += b;
    max_batch = std::max(max_batch, b);
    ++steps;
  }
  void finish(pkv_sim_result* out) const {
    out->steps = steps;
    out->utilization = reserved > 0 ? held / reserved : 0.0;
    out->mean_batch = steps > 0 ? batch / steps : 0.0;
    out->max_batch = max_batch;
  }
};

int simulate_paged(const pkv_sim_config& c, const std::vector<Request>& req, pkv_sim_result* out,
                   int64_t step_limit) {
  const int32_t bs = c.block_size;
  pkv_bm* bm = pkv_bm_create((int32_t)(c.pool_tokens / bs), bs);
  if (!bm) return PKV_BM_INVALID;
  std::deque<int64_t> waiting;
  std::vector<int64_t> prompt(req.size());  // tokens cached at (re)admission
  for (size_t i = 0; i < req.size(); ++i) {
    waiting.push_back((int64_t)i);
    prompt[i] = req[i].P;
  }
  std::vector<int64_t> running;  // in admission order
  const int64_t watermark = (pkv_bm_num_blocks(bm) + 99) / 100;
  Tally t;
  out->preemptions = 0;
  out->recomputed_tokens = 0;
  out->max_tail_waste = 0;
  int rc = PKV_BM_OK;
  while (!waiting.empty() || !running.empty()) {
    if (t.steps >= step_limit) {
      rc = PKV_BM_INVALID;
      break;
    }
    // admit in arrival order while the prompt's blocks plus one, plus a
    // watermark of 1% of the pool, are free (no watermark while nothing
    // runs, so the head of the queue always fits)
    while (!waiting.empty()) {
      const int64_t r = waiting.front();
      const int64_t need = (prompt[r] + bs - 1) / bs + 1 + (running.empty() ? 0 : watermark);
      if (need > pkv_bm_num_free(bm)) break;
      pkv_bm_add_sequence(bm, r, prompt[r]);
      running.push_back(r);
      waiting.pop_front();
    }
    // one token for every running sequence; preempt the newest when full
    for (size_t k = 0; k < running.size();) {
      const int64_t r = running[k];
      int64_t slot;
      int32_t src, dst;
      if (pkv_bm_append_slot(bm, r, &slot, &src, &dst) == PKV_BM_OK) {
        ++k;
        continue;
      }
      const int64_t victim = running.back();
      const int64_t held = pkv_bm_seq_len(bm, victim);
      pkv_bm_free_sequence(bm, victim);
      running.pop_back();
      prompt[victim] = held;  // everything it held is computed again
      out->recomputed_tokens += held;
      ++out->preemptions;
      waiting.push_front(victim);
      if (victim == r) continue;  // the sequence that needed a block was the newest
    }
    double held = 0;
    for (int64_t r : running) {
      const int64_t L = pkv_bm_seq_len(bm, r);
      held += (double)L;
      const int64_t tail = ((L + bs - 1) / bs) * bs - L;
      out->max_tail_waste = std::max<int32_t>(out->max_tail_waste, (int32_t)tail);
    }
    const double reserved = (double)(pkv_bm_num_blocks(bm) - pkv_bm_num_free(bm)) * bs;
    t.step(held, reserved, (int32_t)running.size());
    // release finished sequences
    for (size_t k = 0; k < running.size();) {
      const int64_t r = running[k];
      if (pkv_bm_seq_len(bm, r) >= req[r].L) {
        pkv_bm_free_sequence(bm, r);
        running.erase(running.begin() + k);
      } else {
        ++k;
      }
    }
  }
  pkv_bm_destroy(bm);
  t.finish(out);
  return rc;
}

int simulate_slab(const pkv_sim_config& c, const std::vector<Request>& req, pkv_sim_result* out,
                  int64_t step_limit) {
  const int64_t capacity = c.pool_tokens / c.max_len;
  std::deque<int64_t> waiting;
  for (size_t i = 0; i < req.size(); ++i) waiting.push_back((int64_t)i);
  std::vector<std::pair<int64_t, int64_t>> running;  // (request, tokens)
  Tally t;
  out->preemptions = 0;
  out->recomputed_tokens = 0;
  out->max_tail_waste = 0;
  while (!waiting.empty() || !running.empty()) {
    if (t.steps >= step_limit) return PKV_BM_INVALID;
    while (!waiting.empty() && (int64_t)running.size() < capacity) {
      const int64_t r = waiting.front();
      waiting.pop_front();
      running.push_back({r, req[r].P});
    }
    double held = 0;
    for (auto& q : running) {
      ++q.second;
      held += (double)q.second;
    }
    t.step(held, (double)running.size() * c.max_len, (int32_t)running.size());
    running.erase(std::remove_if(running.begin(), running.end(),
                                 [&](const std::pair<int64_t, int64_t>& q) {
                                   return q.second >= req[q.first].L;
                                 }),
                  running.end());
  }
  t.finish(out);
  return PKV_BM_OK;
}

}  // namespace

int pkv_sim_decode(const pkv_sim_config* cfg, pkv_sim_result* paged, pkv_sim_result* slab) {
  if (!cfg || !paged || !slab) return PKV_BM_INVALID;
  const pkv_sim_config& c = *cfg;
  if (c.num_requests <= 0 || c.block_size <= 0 || c.min_len < 2 || c.max_len < c.min_len ||
      c.prompt_fraction < 0.0 || c.prompt_fraction > 1.0 ||
      (c.lengths != PKV_SIM_UNIFORM && c.lengths != PKV_SIM_LOGNORMAL) ||
      (c.lengths == PKV_SIM_LOGNORMAL && (!(c.median > 0.0) || !(c.sigma >= 0.0))) ||
      c.pool_tokens < ((int64_t)c.max_len + 2 * c.block_size - 1) / c.block_size * c.block_size ||
      c.pool_tokens / c.block_size > INT32_MAX)
    return PKV_BM_INVALID;
  try {
    const std::vector<Request> req = draw_requests(c);
    int64_t tokens = 0, generated = 0;
    for (const Request& q : req) {
      tokens += q.L;
      generated += q.L - q.P;
    }
    // each step advances the oldest running sequence by one token, so this
    // bound is never reached by a working simulation
    const int64_t limit = 4 * (tokens + (int64_t)req.size()) + 16;
    int rc = simulate_paged(c, req, paged, limit);
    if (rc == PKV_BM_OK) rc = simulate_slab(c, req, slab, limit);
    paged->tokens_generated = slab->tokens_generated = generated;
    return rc;
  } catch (...) {
    return PKV_BM_INVALID;
  }
}

}  // extern "C"
