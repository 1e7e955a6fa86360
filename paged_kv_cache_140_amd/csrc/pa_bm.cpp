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
// Automatic prefix caching ([ttlab] section "4. 프리픽스 캐시"; [icarus]
// "支持块级共享"): every full block of a sequence whose token ids are known
// gets a key, sha256(previous block's key, the block's token ids, extra
// information), and a later request whose prompt produces the same keys
// reuses those blocks.  Freed blocks keep their keys while they wait in the
// free queue (tail first); taking a block from the front of the queue evicts
// its key.
//
// The policy choices the pages leave open (which free block, who copies,
// failure atomicity, the hashed bytes) are fixed as declared in pa.h.
// Instead of the token-by-token walk with a rollback snapshot, an append
// first counts the blocks it will take (one per new logical block, plus one
// when the partly filled last block is shared) and fails before touching
// anything; the batched form keeps an undo log (evicted keys included).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pa_host.h"

namespace {

// ------------------------------------------------------------- SHA-256
// FIPS 180-4: 512-bit blocks, 64 rounds.  The round constants are the first
// 32 bits of the fractional parts of the cube roots of the first 64 primes,
// the initial hash value those of the square roots of the first 8 primes;
// both are computed here from that definition.
struct Sha256Consts {
  uint32_t k[64];
  uint32_t h0[8];
  Sha256Consts() {
    int primes[64], n = 0;
    for (int c = 2; n < 64; ++c) {
      bool prime = true;
      for (int d = 2; d * d <= c; ++d) prime = prime && (c % d != 0);
      if (prime) primes[n++] = c;
    }
    for (int i = 0; i < 64; ++i) {
      const long double r = std::cbrt(static_cast<long double>(primes[i]));
      k[i] = static_cast<uint32_t>((r - std::floor(r)) * 4294967296.0L);
    }
    for (int i = 0; i < 8; ++i) {
      const long double r = std::sqrt(static_cast<long double>(primes[i]));
      h0[i] = static_cast<uint32_t>((r - std::floor(r)) * 4294967296.0L);
    }
  }
};

const Sha256Consts& sha_consts() {
  static const Sha256Consts c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

class Sha256 {
 public:
  Sha256() : k_(sha_consts().k) { std::memcpy(h_, sha_consts().h0, sizeof(h_)); }
  void update(const uint8_t* p, size_t n) {
    total_ += n;
    if (fill_ > 0) {
      const size_t take = std::min(n, sizeof(buf_) - fill_);
      std::memcpy(buf_ + fill_, p, take);
      fill_ += take, p += take, n -= take;
      if (fill_ < sizeof(buf_)) return;
      compress(buf_);
      fill_ = 0;
    }
    for (; n >= sizeof(buf_); p += sizeof(buf_), n -= sizeof(buf_)) compress(p);
    std::memcpy(buf_, p, n);
    fill_ = n;
  }
  void final(uint8_t out[32]) {
    const uint64_t bits = total_ * 8;
    buf_[fill_++] = 0x80;
    if (fill_ > 56) {
      std::memset(buf_ + fill_, 0, 64 - fill_);
      compress(buf_);
      fill_ = 0;
    }
    std::memset(buf_ + fill_, 0, 56 - fill_);
    for (int i = 0; i < 8; ++i) buf_[56 + i] = static_cast<uint8_t>(bits >> (56 - 8 * i));
    compress(buf_);
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = static_cast<uint8_t>(h_[i] >> (24 - 8 * j));
  }

 private:
  void compress(const uint8_t* blk) {
    const uint32_t* K = k_;
    uint32_t w[64];
    for (int t = 0; t < 16; ++t)
      w[t] = (uint32_t(blk[4 * t]) << 24) | (uint32_t(blk[4 * t + 1]) << 16) | (uint32_t(blk[4 * t + 2]) << 8) |
             uint32_t(blk[4 * t + 3]);
    for (int t = 16; t < 64; ++t) {
      const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
      const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
      w[t] = w[t - 16] + s0 + w[t - 7] + s1;
    }
    uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3], e = h_[4], f = h_[5], g = h_[6], h = h_[7];
    for (int t = 0; t < 64; ++t) {
      const uint32_t t1 = h + (rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25)) + ((e & f) ^ (~e & g)) + K[t] + w[t];
      const uint32_t t2 = (rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22)) + ((a & b) ^ (a & c) ^ (b & c));
      h = g, g = f, f = e, e = d + t1, d = c, c = b, b = a, a = t1 + t2;
    }
    h_[0] += a, h_[1] += b, h_[2] += c, h_[3] += d, h_[4] += e, h_[5] += f, h_[6] += g, h_[7] += h;
  }
  const uint32_t* k_;
  uint32_t h_[8];
  uint8_t buf_[64];
  size_t fill_ = 0;
  uint64_t total_ = 0;
};

// ------------------------------------------------------------- block keys
struct Key {
  uint8_t b[32];
  bool operator==(const Key& o) const { return std::memcmp(b, o.b, 32) == 0; }
};
struct KeyHash {
  size_t operator()(const Key& k) const {
    uint64_t v;
    std::memcpy(&v, k.b, sizeof(v));
    return static_cast<size_t>(v);
  }
};

// Key of one full block: sha256 over the previous key (32 zero bytes for
// the first block), the block's token ids as little-endian int32 and the
// extra information as a little-endian uint64.
Key block_key(const Key& prev, const int32_t* tokens, int32_t bs, uint64_t extra) {
  thread_local std::vector<uint8_t> msg;
  msg.resize(32 + 4 * static_cast<size_t>(bs) + 8);
  std::memcpy(msg.data(), prev.b, 32);
  uint8_t* t = msg.data() + 32;
  for (int32_t i = 0; i < bs; ++i) {
    const uint32_t v = static_cast<uint32_t>(tokens[i]);
    t[4 * i] = uint8_t(v), t[4 * i + 1] = uint8_t(v >> 8), t[4 * i + 2] = uint8_t(v >> 16), t[4 * i + 3] = uint8_t(v >> 24);
  }
  for (int i = 0; i < 8; ++i) t[4 * bs + i] = static_cast<uint8_t>(extra >> (8 * i));
  Sha256 h;
  h.update(msg.data(), msg.size());
  Key k;
  h.final(k.b);
  return k;
}

// ------------------------------------------------------------- free queue
// FIFO of free blocks as an intrusive doubly linked list over block ids, so
// that a cache hit can take a waiting block out of the middle.
struct FreeQueue {
  std::vector<int32_t> prev, next;
  std::vector<char> in;
  int32_t head = -1, tail = -1;
  int64_t count = 0;

  void init(int32_t n) {
    prev.assign(n, -1);
    next.assign(n, -1);
    in.assign(n, 0);
  }
  int64_t size() const { return count; }
  void push_back(int32_t b) {
    prev[b] = tail, next[b] = -1, in[b] = 1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    ++count;
  }
  void push_front(int32_t b) {
    prev[b] = -1, next[b] = head, in[b] = 1;
    if (head >= 0) prev[head] = b; else tail = b;
    head = b;
    ++count;
  }
  void remove(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1, in[b] = 0;
    --count;
  }
  int32_t pop_front() {
    const int32_t b = head;
    remove(b);
    return b;
  }
};

struct Seq {
  std::vector<int32_t> table;
  int64_t len = 0;
  // keying state: the extra information, the key of the last full block and
  // the token ids of the partly filled block; keyed is false once the
  // sequence was appended without token ids
  bool keyed = true;
  uint64_t extra = 0;
  Key last{};
  std::vector<int32_t> part;
};

}  // namespace

struct pa_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  FreeQueue free_q;
  std::vector<int32_t> ref;
  std::unordered_map<int32_t, Seq> seqs;
  std::unordered_map<Key, int32_t, KeyHash> cache;
  std::vector<Key> bkey;
  std::vector<char> has_key;
  // while a batch runs: the keys take() evicts, so that a failed batch can
  // put them back
  std::vector<std::pair<int32_t, Key>>* evict_log = nullptr;

  Seq* find(int32_t s) {
    auto it = seqs.find(s);
    return it == seqs.end() ? nullptr : &it->second;
  }

  int32_t take() {
    const int32_t b = free_q.pop_front();
    if (has_key[b]) {  // its contents are about to be overwritten
      if (evict_log) evict_log->emplace_back(b, bkey[b]);
      cache.erase(bkey[b]);
      has_key[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  // Keys the blocks that the tokens of an append (positions [from, from + n)
  // of s) fill, and caches each unless its key is cached already.
  void key_tokens(Seq& s, int64_t from, const int32_t* tokens, int32_t n) {
    if (!s.keyed) return;
    for (int32_t i = 0; i < n; ++i) {
      s.part.push_back(tokens[i]);
      if (static_cast<int32_t>(s.part.size()) == block_size) {
        const int32_t b = s.table[(from + i) / block_size];
        const Key k = block_key(s.last, s.part.data(), block_size, s.extra);
        if (cache.emplace(k, b).second) {
          bkey[b] = k;
          has_key[b] = 1;
        }
        s.last = k;
        s.part.clear();
      }
    }
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
    bool old_keyed;
  };

  // Performs the append (capacity already checked).  Writes n slots and at
  // most one pair.  Returns the number of pairs written.
  int append(Seq& s, int32_t n, int32_t* slots, int32_t* pair, Undo* undo) {
    const int64_t bs = block_size;
    int npairs = 0;
    if (undo) *undo = Undo{&s, s.table.size(), s.len, -1, s.keyed};
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
  // back to the front of the queue in the order they were taken, and the
  // keys their taking evicted are cached again.
  void revert(const Undo* undo, int k, const std::vector<std::pair<int32_t, Key>>& evicted) {
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
      s.keyed = u.old_keyed;
    }
    for (const auto& e : evicted) {
      cache.emplace(e.second, e.first);
      bkey[e.first] = e.second;
      has_key[e.first] = 1;
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
  bm->free_q.init(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) bm->free_q.push_back(free_order[i]);
  bm->ref.assign(num_blocks, 0);
  bm->bkey.assign(num_blocks, Key{});
  bm->has_key.assign(num_blocks, 0);
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
  s->keyed = false;  // no token ids: the blocks this fills cannot be keyed
  return PA_OK;
}

int pa_bm_append_slots_batch(pa_bm* bm, const int32_t* seqs, const int32_t* ns, int32_t count, int32_t* slots_out,
                             int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!bm || count < 0 || (count > 0 && (!seqs || !ns || !cow_pairs_out))) return pa::fail(PA_EINVAL, "NULL argument");
  std::vector<pa_bm::Undo> undo(count);
  std::vector<std::pair<int32_t, Key>> evicted;
  bm->evict_log = &evicted;
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
      bm->evict_log = nullptr;
      bm->revert(undo.data(), i, evicted);
      return pa::fail(err, msg);
    }
    npairs += bm->append(*s, ns[i], slots_out + off, cow_pairs_out + 2 * npairs, &undo[i]);
    s->keyed = false;
    off += ns[i];
  }
  bm->evict_log = nullptr;
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
  for (int32_t b = bm->free_q.head; b >= 0 && i < cap; b = bm->free_q.next[b]) out[i++] = b;
  return n;
}

// ------------------------------------------------------------- prefix cache

int pa_bm_add_seq_prefix(pa_bm* bm, int32_t seq, const int32_t* tokens, int32_t n, uint64_t extra,
                         int32_t* n_hit_out) {
  if (!bm || n < 0 || (n > 0 && !tokens)) return pa::fail(PA_EINVAL, "NULL argument or negative length");
  if (bm->find(seq)) return pa::fail(PA_ENOENT, "sequence " + std::to_string(seq) + " already exists");
  Seq s;
  s.extra = extra;
  const int32_t bs = bm->block_size;
  for (int32_t j = 0; j < n / bs; ++j) {
    const Key k = block_key(s.last, tokens + static_cast<int64_t>(j) * bs, bs, extra);
    auto it = bm->cache.find(k);
    if (it == bm->cache.end()) break;
    const int32_t b = it->second;
    if (bm->ref[b] == 0) bm->free_q.remove(b);
    bm->ref[b] += 1;
    s.table.push_back(b);
    s.len += bs;
    s.last = k;
  }
  const int32_t hit = static_cast<int32_t>(s.len);
  bm->seqs.emplace(seq, std::move(s));
  if (n_hit_out) *n_hit_out = hit;
  return PA_OK;
}

int pa_bm_append_tokens(pa_bm* bm, int32_t seq, const int32_t* tokens, int32_t n, int32_t* slots_out,
                        int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!bm || (n > 0 && (!slots_out || !tokens))) return pa::fail(PA_EINVAL, "NULL argument");
  if (n < 0) return pa::fail(PA_EINVAL, "negative token count");
  Seq* s = bm->find(seq);
  if (!s) return pa::fail(PA_ENOENT, "no sequence " + std::to_string(seq));
  if (s->len + n > INT32_MAX) return pa::fail(PA_EINVAL, "sequence length overflows int32");
  const int64_t need = bm->need(*s, n);
  if (need > bm->free_q.size())
    return pa::fail(PA_ENOMEM, "need " + std::to_string(need) + " blocks, " + std::to_string(bm->free_q.size()) + " free");
  const bool will_cow = n > 0 && s->len % bm->block_size != 0 && bm->ref[s->table.back()] > 1;
  if (will_cow && !cow_pairs_out) return pa::fail(PA_EINVAL, "append needs a copy-on-write pair but cow_pairs_out is NULL");
  const int64_t from = s->len;
  int32_t pair[2];
  const int np = bm->append(*s, n, slots_out, pair, nullptr);
  if (np) {
    cow_pairs_out[0] = pair[0];
    cow_pairs_out[1] = pair[1];
  }
  if (n_cow_out) *n_cow_out = np;
  bm->key_tokens(*s, from, tokens, n);
  return PA_OK;
}

int pa_bm_prefix_lookup(pa_bm* bm, const int32_t* tokens, int32_t n, uint64_t extra) {
  if (!bm || n < 0 || (n > 0 && !tokens)) return pa::fail(PA_EINVAL, "NULL argument or negative length");
  const int32_t bs = bm->block_size;
  Key prev{};
  int32_t hit = 0;
  for (int32_t j = 0; j < n / bs; ++j) {
    const Key k = block_key(prev, tokens + static_cast<int64_t>(j) * bs, bs, extra);
    if (bm->cache.find(k) == bm->cache.end()) break;
    hit += bs;
    prev = k;
  }
  return hit;
}

int pa_bm_blocks_needed(pa_bm* bm, int32_t seq, int32_t n) {
  if (!bm || n < 0) return pa::fail(PA_EINVAL, "NULL manager or negative token count");
  Seq* s = bm->find(seq);
  if (!s) return pa::fail(PA_ENOENT, "no sequence " + std::to_string(seq));
  return static_cast<int>(bm->need(*s, n));
}

int pa_bm_admit_cost(pa_bm* bm, const int32_t* tokens, int32_t n, uint64_t extra) {
  if (!bm || n < 0 || (n > 0 && !tokens)) return pa::fail(PA_EINVAL, "NULL argument or negative length");
  const int32_t bs = bm->block_size;
  Key prev{};
  int64_t hits = 0, waiting = 0;
  for (int32_t j = 0; j < n / bs; ++j) {
    const Key k = block_key(prev, tokens + static_cast<int64_t>(j) * bs, bs, extra);
    auto it = bm->cache.find(k);
    if (it == bm->cache.end()) break;
    ++hits;
    if (bm->ref[it->second] == 0) ++waiting;
    prev = k;
  }
  return static_cast<int>(waiting + pa::ceil_div(n, bs) - hits);
}

int pa_bm_num_cached(pa_bm* bm) {
  if (!bm) return pa::fail(PA_EINVAL, "NULL manager");
  return static_cast<int>(bm->cache.size());
}

int pa_bm_block_key(pa_bm* bm, int32_t block, uint8_t* key_out) {
  if (!bm || !key_out || block < 0 || block >= bm->num_blocks) return pa::fail(PA_EINVAL, "bad argument");
  if (!bm->has_key[block]) return 0;
  std::memcpy(key_out, bm->bkey[block].b, 32);
  return 1;
}

int pa_sha256(const void* data, size_t n, uint8_t* digest_out) {
  if ((n > 0 && !data) || !digest_out) return pa::fail(PA_EINVAL, "NULL argument");
  Sha256 h;
  h.update(static_cast<const uint8_t*>(data), n);
  h.final(digest_out);
  return PA_OK;
}

}  // extern "C"
