// pa_blocks.hip — host-side KV block manager (pa_blocks.h). Host code only:
// plain bookkeeping over a FIFO free list and reference counts.
#include <stdint.h>

#include <deque>
#include <unordered_map>
#include <vector>

#include "pa_blocks.h"

namespace {

enum class State { Running, SwappedOut, Swapping };

struct Seq {
  std::vector<int32_t> table;     // device blocks (running) / host blocks (swapped out)
  int32_t num_tokens = 0;
  State state = State::Running;
  uint64_t admitted = 0;          // admission order (newest-first victim choice)
  std::vector<int32_t> host;      // host blocks planned by a swap-out in flight
};

struct Pool {
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;

  int32_t allocate() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b) {       // contents stay as they are
    if (--refcount[b] == 0) free_list.push_back(b);
  }
};

}  // namespace

struct pa_bm {
  int32_t block_size = 0;
  Pool dev, host;
  std::unordered_map<int64_t, Seq> seqs;
  uint64_t clock = 0;

  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  // free device blocks the next n positions take: new blocks past the last
  // one, plus a copy of the last block when it is shared and partly filled
  int32_t needed(const Seq& s, int32_t n) const {
    const int64_t have = (int64_t)s.table.size() * block_size;
    const int64_t extra = (int64_t)s.num_tokens + n - have;
    int64_t need = extra > 0 ? (extra + block_size - 1) / block_size : 0;
    if (n > 0 && s.num_tokens % block_size != 0 && dev.refcount[s.table.back()] > 1) ++need;
    return (int32_t)need;
  }
};

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* order,
                       int32_t num_host_blocks, pa_bm** out) {
  if (!out || num_blocks < 0 || num_host_blocks < 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  std::vector<int32_t> ids(num_blocks);
  if (order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = order[i];
      if (b < 0 || b >= num_blocks || seen[b]) return PA_ERR_INVALID_ARG;
      seen[b] = 1;
      ids[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) ids[i] = i;
  }
  pa_bm* bm = new pa_bm();
  bm->block_size = block_size;
  bm->dev.free_list.assign(ids.begin(), ids.end());
  bm->dev.refcount.assign(num_blocks, 0);
  for (int32_t i = 0; i < num_host_blocks; ++i) bm->host.free_list.push_back(i);
  bm->host.refcount.assign(num_host_blocks, 0);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_bm* bm, int32_t host) {
  if (!bm) return -1;
  return (int32_t)(host ? bm->host.free_list.size() : bm->dev.free_list.size());
}

pa_status pa_bm_add(pa_bm* bm, int64_t seq) {
  if (!bm || bm->find(seq)) return PA_ERR_INVALID_ARG;
  Seq s;
  s.admitted = ++bm->clock;
  bm->seqs.emplace(seq, std::move(s));
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm || bm->find(child)) return PA_ERR_INVALID_ARG;
  const Seq* p = bm->find(parent);
  if (!p || p->state != State::Running) return PA_ERR_INVALID_ARG;
  Seq c;
  c.table = p->table;
  c.num_tokens = p->num_tokens;
  c.admitted = ++bm->clock;
  for (int32_t b : c.table) ++bm->dev.refcount[b];
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

int32_t pa_bm_blocks_needed(const pa_bm* bm, int64_t seq, int32_t n) {
  if (!bm || n < 0) return 0;
  const Seq* s = bm->find(seq);
  if (!s || s->state != State::Running) return 0;
  return bm->needed(*s, n);
}

pa_status pa_bm_append(pa_bm* bm, int64_t seq, int32_t n, int64_t* slots, int64_t* cow_pairs,
                       int32_t* num_cow) {
  if (!bm || n < 0 || (n > 0 && (!slots || !cow_pairs)) || !num_cow) return PA_ERR_INVALID_ARG;
  Seq* s = bm->find(seq);
  if (!s || s->state != State::Running) return PA_ERR_INVALID_ARG;
  *num_cow = 0;
  if (n == 0) return PA_OK;
  if (bm->needed(*s, n) > (int32_t)bm->dev.free_list.size()) return PA_ERR_NO_SPACE;
  const int32_t B = bm->block_size;
  for (int32_t i = 0; i < n; ++i) {
    if (s->num_tokens % B == 0) {
      s->table.push_back(bm->dev.allocate());
    } else if (bm->dev.refcount[s->table.back()] > 1) {
      const int32_t old = s->table.back();
      const int32_t nb = bm->dev.allocate();
      bm->dev.release(old);
      s->table.back() = nb;
      cow_pairs[2 * *num_cow] = old;
      cow_pairs[2 * *num_cow + 1] = nb;
      ++*num_cow;
    }
    slots[i] = (int64_t)s->table.back() * B + s->num_tokens % B;
    ++s->num_tokens;
  }
  return PA_OK;
}

pa_status pa_bm_copy_last_block(pa_bm* bm, int64_t seq, int64_t* pair) {
  if (!bm || !pair) return PA_ERR_INVALID_ARG;
  Seq* s = bm->find(seq);
  if (!s || s->state != State::Running || s->table.empty()) return PA_ERR_INVALID_ARG;
  // only a block another sequence also holds is copied
  if (bm->dev.refcount[s->table.back()] <= 1) return PA_ERR_INVALID_ARG;
  if (bm->dev.free_list.empty()) return PA_ERR_NO_SPACE;
  const int32_t old = s->table.back();
  const int32_t nb = bm->dev.allocate();
  bm->dev.release(old);
  s->table.back() = nb;
  pair[0] = old;
  pair[1] = nb;
  return PA_OK;
}

pa_status pa_bm_release(pa_bm* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID_ARG;
  Seq* s = bm->find(seq);
  if (!s) return PA_ERR_INVALID_ARG;
  if (s->state == State::Swapping) return PA_ERR_INVALID_ARG;    // copy still in flight
  Pool& pool = s->state == State::Running ? bm->dev : bm->host;
  for (int32_t b : s->table) pool.release(b);
  bm->seqs.erase(seq);
  return PA_OK;
}

pa_status pa_bm_table(const pa_bm* bm, int64_t seq, int32_t* table, int32_t capacity,
                      int32_t* num_blocks, int32_t* num_tokens) {
  if (!bm || !num_blocks || !num_tokens) return PA_ERR_INVALID_ARG;
  const Seq* s = bm->find(seq);
  if (!s) return PA_ERR_INVALID_ARG;
  const bool dev = s->state != State::SwappedOut;
  const int32_t nb = dev ? (int32_t)s->table.size() : 0;
  if (nb > capacity || (nb > 0 && !table)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < nb; ++i) table[i] = s->table[i];
  *num_blocks = nb;
  *num_tokens = s->num_tokens;
  return PA_OK;
}

pa_status pa_bm_newest_running(const pa_bm* bm, int64_t* seq) {
  if (!bm || !seq) return PA_ERR_INVALID_ARG;
  bool any = false;
  uint64_t best = 0;
  for (const auto& kv : bm->seqs) {
    if (kv.second.state == State::Running && kv.second.admitted > best) {
      best = kv.second.admitted;
      *seq = kv.first;
      any = true;
    }
  }
  return any ? PA_OK : PA_ERR_INVALID_ARG;
}

pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* n) {
  if (!bm || !n) return PA_ERR_INVALID_ARG;
  Seq* s = bm->find(seq);
  if (!s || s->state != State::Running) return PA_ERR_INVALID_ARG;
  const int32_t nb = (int32_t)s->table.size();
  if (nb > capacity || (nb > 0 && !pairs)) return PA_ERR_INVALID_ARG;
  if (nb > (int32_t)bm->host.free_list.size()) return PA_ERR_NO_SPACE;
  s->host.clear();
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t hb = bm->host.allocate();
    s->host.push_back(hb);
    pairs[2 * i] = s->table[i];
    pairs[2 * i + 1] = hb;
  }
  s->state = State::Swapping;
  *n = nb;
  return PA_OK;
}

pa_status pa_bm_swap_out_done(pa_bm* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID_ARG;
  Seq* s = bm->find(seq);
  if (!s || s->state != State::Swapping) return PA_ERR_INVALID_ARG;
  for (int32_t b : s->table) bm->dev.release(b);
  s->table = std::move(s->host);
  s->host.clear();
  s->state = State::SwappedOut;
  return PA_OK;
}

pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq, int64_t* pairs, int32_t capacity, int32_t* n) {
  if (!bm || !n) return PA_ERR_INVALID_ARG;
  Seq* s = bm->find(seq);
  if (!s || s->state != State::SwappedOut) return PA_ERR_INVALID_ARG;
  const int32_t nb = (int32_t)s->table.size();
  if (nb > capacity || (nb > 0 && !pairs)) return PA_ERR_INVALID_ARG;
  if (nb > (int32_t)bm->dev.free_list.size()) return PA_ERR_NO_SPACE;
  std::vector<int32_t> dev(nb);
  for (int32_t i = 0; i < nb; ++i) {
    dev[i] = bm->dev.allocate();
    pairs[2 * i] = s->table[i];
    pairs[2 * i + 1] = dev[i];
    bm->host.release(s->table[i]);
  }
  s->table = std::move(dev);
  s->state = State::Running;
  s->admitted = ++bm->clock;
  *n = nb;
  return PA_OK;
}

}  // extern "C"
