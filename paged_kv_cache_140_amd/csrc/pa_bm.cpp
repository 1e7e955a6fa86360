// Host block manager: free queue, block tables, refcounts, fork and
// copy-on-write -- the bookkeeping side of paging.
//
// Pages: [icarus] "PagedAttention" (icarus.shaojiemike.top), sections
// "Block Table 如何工作" (write into the current block, take a free block
// when it is full, return unreferenced blocks when a request ends) and
// "支持块级共享" (shared blocks with reference counts, copy on write);
// [ttlab] "llm-kv-cache-02-serving-engine-kv" (ttlab.hopto.org), sections
// "블록과 블록 표" and "블록을 함께 쓰기".
//
// The policy choices the pages leave open (which free block, who copies,
// failure atomicity) are fixed as declared in pa.h.  Instead of the
// token-by-token walk with a rollback snapshot, an append first counts the
// blocks it will take (one per new logical block, plus one when the partly
// filled last block is shared) and fails before touching anything; the
// batched form keeps an undo log.
#include <deque>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_host.h"

namespace {

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
};

}  // namespace

struct pa_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_q;
  std::vector<int32_t> ref;
  std::unordered_map<int32_t, Seq> seqs;

  Seq* find(int32_t s) {
    auto it = seqs.find(s);
    return it == seqs.end() ? nullptr : &it->second;
  }

  int32_t take() {
    int32_t b = free_q.front();
    free_q.pop_front();
    ref[b] = 1;
    return b;
  }

  // Blocks an append of n tokens to s would take, given the current state.
  int64_t need(const Seq& s, int32_t n) const {
    if (n <= 0) return 0;
    const int64_t bs = block_size;
    int64_t fresh = pa::ceil_div(s.len + n, bs) - static_cast<int64_t>(s.table.size());
    int64_t cow = (s.len % bs != 0 && ref[s.table.back()] > 1) ? 1 : 0;
    return fresh + cow;
  }

  struct Undo {
    Seq* seq;
    size_t old_size;
    int64_t old_len;
    int32_t cow_old;  // -1 if no copy-on-write
  };

  // Performs the append (capacity already checked).  Writes n slots and at
  // most one pair.  Returns the number of pairs written.
  int append(Seq& s, int32_t n, int32_t* slots, int32_t* pair, Undo* undo) {
    const int64_t bs = block_size;
    int npairs = 0;
    if (undo) *undo = Undo{&s, s.table.size(), s.len, -1};
    if (n <= 0) return 0;
    if (s.len % bs != 0 && ref[s.table.back()] > 1) {
      int32_t old = s.table.back();
      int32_t fresh = take();
      ref[old] -= 1;
      s.table.back() = fresh;
      pair[0] = old;
      pair[1] = fresh;
      npairs = 1;
      if (undo) undo->cow_old = old;
    }
    for (int64_t i = 0; i < n; ++i) {
      int64_t p = s.len + i;
      int64_t j = p / bs;
      if (j == static_cast<int64_t>(s.table.size())) s.table.push_back(take());
      slots[i] = static_cast<int32_t>(s.table[j] * bs + p % bs);
    }
    s.len += n;
    return npairs;
  }

  // Reverts appends recorded in undo[0..k) (newest first).  Blocks taken go
  // back to the front of the queue in the order they were taken.
  void revert(const Undo* undo, int k) {
    for (int i = k - 1; i >= 0; --i) {
      const Undo& u = undo[i];
      Seq& s = *u.seq;
      while (s.table.size() > u.old_size) {
        int32_t b = s.table.back();
        s.table.pop_back();
        ref[b] = 0;
        free_q.push_front(b);
      }
      if (u.cow_old >= 0) {
        int32_t b = s.table.back();
        ref[b] = 0;
        free_q.push_front(b);
        s.table.back() = u.cow_old;
        ref[u.cow_old] += 1;
      }
      s.len = u.old_len;
    }
  }
};

extern "C" {

int pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pa_bm** out) {
  if (!out || !free_order) return pa::fail(PA_EINVAL, "pa_bm_create: NULL argument");
  if (num_blocks <= 0 || block_size <= 0) return pa::fail(PA_EINVAL, "pa_bm_create: sizes must be positive");
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return pa::fail(PA_EINVAL, "pa_bm_create: num_blocks * block_size must fit in int32");
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order[i];
    if (b < 0 || b >= num_blocks || seen[b]) return pa::fail(PA_EINVAL, "pa_bm_create: free_order is not a permutation");
    seen[b] = 1;
  }
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return pa::fail(PA_ENOMEM, "pa_bm_create: host allocation failed");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->free_q.assign(free_order, free_order + num_blocks);
  bm->ref.assign(num_blocks, 0);
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_add_seq(pa_bm* bm, int32_t seq) {
  if (!bm) return pa::fail(PA_EINVAL, "NULL manager");
  if (bm->find(seq)) return pa::fail(PA_ENOENT, "sequence " + std::to_string(seq) + " already exists");
  bm->seqs.emplace(seq, Seq{});
  return PA_OK;
}

int pa_bm_fork(pa_bm* bm, int32_t parent, int32_t child) {
  if (!bm) return pa::fail(PA_EINVAL, "NULL manager");
  Seq* p = bm->find(parent);
  if (!p) return pa::fail(PA_ENOENT, "no parent sequence " + std::to_string(parent));
  if (bm->find(child)) return pa::fail(PA_ENOENT, "child sequence " + std::to_string(child) + " already exists");
  Seq c = *p;  // copy before emplace: emplace may rehash and move *p
  for (int32_t b : c.table) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(c));
  return PA_OK;
}

int pa_bm_append_slots(pa_bm* bm, int32_t seq, int32_t n, int32_t* slots_out, int32_t* cow_pairs_out,
                       int32_t* n_cow_out) {
  if (!bm || (n > 0 && !slots_out)) return pa::fail(PA_EINVAL, "NULL argument");
  if (n < 0) return pa::fail(PA_EINVAL, "negative token count");
  Seq* s = bm->find(seq);
  if (!s) return pa::fail(PA_ENOENT, "no sequence " + std::to_string(seq));
  if (s->len + n > INT32_MAX) return pa::fail(PA_EINVAL, "sequence length overflows int32");
  int64_t need = bm->need(*s, n);
  if (need > static_cast<int64_t>(bm->free_q.size()))
    return pa::fail(PA_ENOMEM, "need " + std::to_string(need) + " blocks, " + std::to_string(bm->free_q.size()) + " free");
  const bool will_cow = n > 0 && s->len % bm->block_size != 0 && bm->ref[s->table.back()] > 1;
  if (will_cow && !cow_pairs_out) return pa::fail(PA_EINVAL, "append needs a copy-on-write pair but cow_pairs_out is NULL");
  int32_t pair[2];
  int np = bm->append(*s, n, slots_out, pair, nullptr);
  if (np) {
    cow_pairs_out[0] = pair[0];
    cow_pairs_out[1] = pair[1];
  }
  if (n_cow_out) *n_cow_out = np;
  return PA_OK;
}

int pa_bm_append_slots_batch(pa_bm* bm, const int32_t* seqs, const int32_t* ns, int32_t count, int32_t* slots_out,
                             int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!bm || count < 0 || (count > 0 && (!seqs || !ns || !cow_pairs_out))) return pa::fail(PA_EINVAL, "NULL argument");
  std::vector<pa_bm::Undo> undo(count);
  int64_t off = 0;
  int npairs = 0;
  for (int32_t i = 0; i < count; ++i) {
    Seq* s = bm->find(seqs[i]);
    int err = PA_OK;
    std::string msg;
    if (!s) {
      err = PA_ENOENT;
      msg = "no sequence " + std::to_string(seqs[i]);
    } else if (ns[i] < 0) {
      err = PA_EINVAL;
      msg = "negative token count";
    } else if (ns[i] > 0 && !slots_out) {
      err = PA_EINVAL;
      msg = "NULL slots_out";
    } else if (s->len + ns[i] > INT32_MAX) {
      err = PA_EINVAL;
      msg = "sequence length overflows int32";
    } else if (bm->need(*s, ns[i]) > static_cast<int64_t>(bm->free_q.size())) {
      err = PA_ENOMEM;
      msg = "out of free blocks at batch entry " + std::to_string(i);
    }
    if (err != PA_OK) {
      bm->revert(undo.data(), i);
      return pa::fail(err, msg);
    }
    npairs += bm->append(*s, ns[i], slots_out + off, cow_pairs_out + 2 * npairs, &undo[i]);
    off += ns[i];
  }
  if (n_cow_out) *n_cow_out = npairs;
  return PA_OK;
}

int pa_bm_free_seq(pa_bm* bm, int32_t seq) {
  if (!bm) return pa::fail(PA_EINVAL, "NULL manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return pa::fail(PA_ENOENT, "no sequence " + std::to_string(seq));
  const std::vector<int32_t>& t = it->second.table;
  for (auto r = t.rbegin(); r != t.rend(); ++r) {
    if (--bm->ref[*r] == 0) bm->free_q.push_back(*r);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_block_table(pa_bm* bm, int32_t seq, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!bm || (cap > 0 && !out)) return pa::fail(PA_EINVAL, "NULL argument");
  Seq* s = bm->find(seq);
  if (!s) return pa::fail(PA_ENOENT, "no sequence " + std::to_string(seq));
  int32_t n = static_cast<int32_t>(s->table.size());
  for (int32_t i = 0; i < n && i < cap; ++i) out[i] = s->table[i];
  if (n_out) *n_out = n;
  return PA_OK;
}

int pa_bm_block_tables(pa_bm* bm, const int32_t* seqs, int32_t count, int32_t* out, int32_t max_blocks, int32_t pad) {
  if (!bm || count < 0 || max_blocks < 0 || (count > 0 && (!seqs || !out))) return pa::fail(PA_EINVAL, "NULL argument");
  for (int32_t i = 0; i < count; ++i) {
    Seq* s = bm->find(seqs[i]);
    if (!s) return pa::fail(PA_ENOENT, "no sequence " + std::to_string(seqs[i]));
    if (static_cast<int64_t>(s->table.size()) > max_blocks)
      return pa::fail(PA_ESPACE, "sequence " + std::to_string(seqs[i]) + " has more than max_blocks blocks");
  }
  for (int32_t i = 0; i < count; ++i) {
    const Seq& s = *bm->find(seqs[i]);
    int32_t* row = out + static_cast<int64_t>(i) * max_blocks;
    size_t j = 0;
    for (; j < s.table.size(); ++j) row[j] = s.table[j];
    for (; j < static_cast<size_t>(max_blocks); ++j) row[j] = pad;
  }
  return PA_OK;
}

int pa_bm_seq_len(pa_bm* bm, int32_t seq) {
  if (!bm) return pa::fail(PA_EINVAL, "NULL manager");
  Seq* s = bm->find(seq);
  if (!s) return pa::fail(PA_ENOENT, "no sequence " + std::to_string(seq));
  return static_cast<int>(s->len);
}

int pa_bm_refcount(pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return pa::fail(PA_EINVAL, "block out of range");
  return bm->ref[block];
}

int pa_bm_num_free(pa_bm* bm) {
  if (!bm) return pa::fail(PA_EINVAL, "NULL manager");
  return static_cast<int>(bm->free_q.size());
}

int pa_bm_free_list(pa_bm* bm, int32_t* out, int32_t cap) {
  if (!bm || (cap > 0 && !out)) return pa::fail(PA_EINVAL, "NULL argument");
  int32_t n = static_cast<int32_t>(bm->free_q.size());
  int32_t i = 0;
  for (auto it = bm->free_q.begin(); it != bm->free_q.end() && i < cap; ++it) out[i++] = *it;
  return n;
}

}  // extern "C"
