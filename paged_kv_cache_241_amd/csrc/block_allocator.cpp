// Host-side block allocator of the paged KV cache (see block_allocator.hpp).
#include "block_allocator.hpp"

#include <algorithm>

namespace pa {

namespace {
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

BlockAllocator::BlockAllocator(int32_t num_blocks, int32_t block_size, int32_t max_seqs,
                               int32_t max_seq_len, bool paged)
    : paged_(paged),
      num_blocks_(paged ? num_blocks : 0),
      block_size_(block_size),
      max_seqs_(max_seqs),
      max_seq_len_(max_seq_len) {
  free_.resize(num_blocks_);
  for (int32_t i = 0; i < num_blocks_; ++i) free_[i] = num_blocks_ - 1 - i;  // 0 on top
  refcount_.assign(num_blocks_, 0);
  fill_.assign(num_blocks_, 0);
  free_ids_.resize(max_seqs_);
  for (int32_t i = 0; i < max_seqs_; ++i) free_ids_[i] = max_seqs_ - 1 - i;
  seqs_.resize(max_seqs_);
  mark_.assign(max_seqs_, 0);
}

Status BlockAllocator::set_free_order(const int32_t* ids, int32_t n, std::string* err) {
  if (!paged_) {
    *err = "set_free_order: a contiguous pool has no blocks";
    return kInvalidArg;
  }
  if (static_cast<int32_t>(free_.size()) != num_blocks_) {
    *err = "set_free_order: blocks are in use";
    return kInvalidArg;
  }
  if (ids == nullptr || n != num_blocks_) {
    *err = "set_free_order: need a permutation of all num_blocks block ids";
    return kInvalidArg;
  }
  std::vector<uint8_t> seen(num_blocks_, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= num_blocks_ || seen[ids[i]]) {
      *err = "set_free_order: not a permutation of 0..num_blocks-1";
      return kInvalidArg;
    }
    seen[ids[i]] = 1;
  }
  for (int32_t i = 0; i < n; ++i) free_[i] = ids[n - 1 - i];
  return kOk;
}

Status BlockAllocator::check_live(int32_t rid, std::string* err) const {
  if (rid < 0 || rid >= max_seqs_ || !seqs_[rid].live) {
    *err = "request id " + std::to_string(rid) + " is not live";
    return kUnknownSeq;
  }
  return kOk;
}

Status BlockAllocator::check_resident(int32_t rid, std::string* err) const {
  Status st = check_live(rid, err);
  if (st != kOk) return st;
  if (seqs_[rid].swapped) {
    *err = "request id " + std::to_string(rid) + " is swapped out";
    return kInvalidArg;
  }
  return kOk;
}

// Gives a request's blocks back in table order (a block is free once no table
// holds it) and empties its table.
void BlockAllocator::release(Seq& s) {
  for (int32_t b : s.table) {
    const int32_t rc = --refcount_[b];
    if (rc == 1) --shared_blocks_;
    if (rc == 0) {
      fill_[b] = 0;
      free_.push_back(b);
    }
  }
  s.table.clear();
}

Status BlockAllocator::add(int32_t* rid, std::string* err) {
  if (rid == nullptr) {
    *err = "seq_add: null output";
    return kInvalidArg;
  }
  if (free_ids_.empty()) {
    *err = "seq_add: all request ids are live";
    return kNoReqId;
  }
  int32_t r = free_ids_.back();
  free_ids_.pop_back();
  Seq& s = seqs_[r];
  s.live = true;
  s.swapped = false;
  s.len = 0;
  s.table.clear();
  *rid = r;
  return kOk;
}

Status BlockAllocator::fork(int32_t parent, int32_t* child, std::string* err) {
  if (!paged_) {
    *err = "seq_fork: sharing needs the paged layout";
    return kInvalidArg;
  }
  if (child == nullptr) {
    *err = "seq_fork: null output";
    return kInvalidArg;
  }
  Status st = check_resident(parent, err);
  if (st != kOk) return st;
  if (free_ids_.empty()) {
    *err = "seq_fork: all request ids are live";
    return kNoReqId;
  }
  int32_t r = free_ids_.back();
  free_ids_.pop_back();
  Seq& c = seqs_[r];
  const Seq& p = seqs_[parent];
  c.live = true;
  c.swapped = false;
  c.len = p.len;
  c.table = p.table;
  for (int32_t b : c.table)
    if (++refcount_[b] == 2) ++shared_blocks_;
  *child = r;
  return kOk;
}

Status BlockAllocator::free_seq(int32_t rid, std::string* err) {
  Status st = check_live(rid, err);
  if (st != kOk) return st;
  Seq& s = seqs_[rid];
  release(s);
  s.live = false;
  s.swapped = false;
  s.len = 0;
  free_ids_.push_back(rid);
  return kOk;
}

int32_t BlockAllocator::pop_block() {
  int32_t b = free_.back();
  free_.pop_back();
  return b;
}

Status BlockAllocator::check_growth(const int32_t* rids, int32_t n, const int32_t* counts,
                                    int64_t* total, std::string* err) const {
  if (n < 0 || (n > 0 && rids == nullptr)) {
    *err = "reserve: bad request list";
    return kInvalidArg;
  }
  if (++epoch_ == 0) {
    std::fill(mark_.begin(), mark_.end(), 0);
    epoch_ = 1;
  }
  int64_t sum = 0;
  for (int32_t i = 0; i < n; ++i) {
    Status st = check_resident(rids[i], err);
    if (st != kOk) return st;
    if (mark_[rids[i]] == epoch_) {
      *err = "reserve: request " + std::to_string(rids[i]) + " listed twice";
      return kInvalidArg;
    }
    mark_[rids[i]] = epoch_;
    int32_t c = counts ? counts[i] : 1;
    if (c < 0) {
      *err = "reserve: negative token count";
      return kInvalidArg;
    }
    if (static_cast<int64_t>(seqs_[rids[i]].len) + c > max_seq_len_) {
      *err = "reserve: request " + std::to_string(rids[i]) + " would exceed max_seq_len";
      return kInvalidArg;
    }
    sum += c;
  }
  *total = sum;
  return kOk;
}

Status BlockAllocator::reserve(const int32_t* rids, int32_t n, const int32_t* counts,
                               int32_t* slots, int64_t slots_cap, int32_t* pairs,
                               int32_t pair_cap, int32_t* n_pairs, std::string* err) {
  if (n < 0 || (n > 0 && rids == nullptr) || pair_cap < 0) {
    *err = "reserve: bad request list";
    return kInvalidArg;
  }
  if (n_pairs) *n_pairs = 0;
  // validate everything before touching state
  int64_t total = 0;
  {
    Status st = check_growth(rids, n, counts, &total, err);
    if (st != kOk) return st;
  }
  if (total > slots_cap || (total > 0 && slots == nullptr)) {
    *err = "reserve: slots_out holds " + std::to_string(slots_cap) + " slots, " +
           std::to_string(total) + " needed";
    return kInvalidArg;
  }
  if (!paged_) {
    int64_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
      Seq& s = seqs_[rids[i]];
      int32_t c = counts ? counts[i] : 1;
      for (int32_t t = 0; t < c; ++t) {
        slots[k++] = rids[i] * max_seq_len_ + s.len;
        ++s.len;
      }
    }
    return kOk;
  }
  // dry run: fresh blocks for growth plus one per copy-on-write
  const int32_t bs = block_size_;
  touched_.clear();
  share_.clear();
  int64_t need = 0, copies = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = seqs_[rids[i]];
    int32_t c = counts ? counts[i] : 1;
    if (c == 0) continue;
    if (s.len % bs != 0) {
      int32_t last = s.table.back();
      size_t j = 0;
      while (j < touched_.size() && touched_[j] != last) ++j;
      if (j == touched_.size()) {
        touched_.push_back(last);
        share_.push_back(refcount_[last]);
      }
      if (share_[j] > 1) {
        ++copies;
        --share_[j];
      }
    }
    need += ceil_div(static_cast<int64_t>(s.len) + c, bs) - ceil_div(s.len, bs);
  }
  need += copies;
  if (copies > pair_cap || (copies > 0 && pairs == nullptr)) {
    *err = "reserve: cow_pairs_out holds " + std::to_string(pair_cap) + " pairs, " +
           std::to_string(copies) + " needed";
    return kInvalidArg;
  }
  if (need > static_cast<int64_t>(free_.size())) {
    *err = "reserve: need " + std::to_string(need) + " blocks, " +
           std::to_string(free_.size()) + " free";
    return kNoBlocks;
  }
  // commit
  int64_t k = 0;
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq& s = seqs_[rids[i]];
    int32_t c = counts ? counts[i] : 1;
    for (int32_t t = 0; t < c; ++t) {
      const int32_t pos = s.len;
      int32_t b;
      if (pos % bs == 0) {
        b = pop_block();
        refcount_[b] = 1;
        fill_[b] = 0;
        s.table.push_back(b);
      } else {
        b = s.table.back();
        if (refcount_[b] > 1) {
          const int32_t nb = pop_block();
          refcount_[nb] = 1;
          fill_[nb] = fill_[b];
          if (--refcount_[b] == 1) --shared_blocks_;
          s.table.back() = nb;
          pairs[2 * np] = b;
          pairs[2 * np + 1] = nb;
          ++np;
          ++cow_copies_;
          b = nb;
        }
      }
      slots[k++] = b * bs + pos % bs;
      fill_[b] = pos % bs + 1;
      ++s.len;
    }
  }
  if (n_pairs) *n_pairs = np;
  return kOk;
}

Status BlockAllocator::tables(const int32_t* rids, int32_t n, int32_t stride, int32_t* out,
                              int32_t* lens, std::string* err) const {
  if (n < 0 || (n > 0 && rids == nullptr) || stride < 0) {
    *err = "get_block_tables: bad arguments";
    return kInvalidArg;
  }
  for (int32_t i = 0; i < n; ++i) {
    Status st = check_resident(rids[i], err);
    if (st != kOk) return st;
    if (out && static_cast<int64_t>(seqs_[rids[i]].table.size()) > stride) {
      *err = "get_block_tables: request " + std::to_string(rids[i]) + " has " +
             std::to_string(seqs_[rids[i]].table.size()) + " blocks, stride is " +
             std::to_string(stride);
      return kInvalidArg;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = seqs_[rids[i]];
    if (out) {
      int32_t* row = out + static_cast<int64_t>(i) * stride;
      int32_t j = 0;
      for (; j < static_cast<int32_t>(s.table.size()); ++j) row[j] = s.table[j];
      for (; j < stride; ++j) row[j] = -1;
    }
    if (lens) lens[i] = s.len;
  }
  return kOk;
}

AllocStats BlockAllocator::stats() const {
  AllocStats st;
  for (const Seq& s : seqs_) {
    if (!s.live) continue;
    if (s.swapped) {
      ++st.swapped_seqs;
      st.swapped_tokens += s.len;
      continue;
    }
    ++st.live_seqs;
    st.logical_tokens += s.len;
  }
  st.cow_copies = cow_copies_;
  st.shared_blocks = shared_blocks_;
  if (paged_) {
    st.free_blocks = static_cast<int64_t>(free_.size());
    st.used_blocks = num_blocks_ - st.free_blocks;
    for (int32_t b = 0; b < num_blocks_; ++b)
      if (refcount_[b] > 0) st.tokens += fill_[b];
    st.reserved_tokens = st.used_blocks * block_size_;
  } else {
    st.tokens = st.logical_tokens;
    st.reserved_tokens = st.live_seqs * static_cast<int64_t>(max_seq_len_);
  }
  st.utilisation = st.reserved_tokens
                       ? static_cast<double>(st.tokens) / static_cast<double>(st.reserved_tokens)
                       : 0.0;
  return st;
}

Status BlockAllocator::swap_out_blocks(int32_t rid, std::vector<int32_t>* blocks, int32_t* len,
                                       std::string* err) const {
  if (!paged_) {
    *err = "swap_out: swapping needs the paged layout";
    return kInvalidArg;
  }
  Status st = check_resident(rid, err);
  if (st != kOk) return st;
  *blocks = seqs_[rid].table;
  *len = seqs_[rid].len;
  return kOk;
}

Status BlockAllocator::swap_out(int32_t rid, std::string* err) {
  std::vector<int32_t> blocks;
  int32_t len = 0;
  Status st = swap_out_blocks(rid, &blocks, &len, err);
  if (st != kOk) return st;
  Seq& s = seqs_[rid];
  release(s);
  s.swapped = true;
  return kOk;
}

Status BlockAllocator::swap_in(int32_t rid, std::vector<int32_t>* blocks, std::string* err) {
  if (!paged_) {
    *err = "swap_in: swapping needs the paged layout";
    return kInvalidArg;
  }
  Status st = check_live(rid, err);
  if (st != kOk) return st;
  Seq& s = seqs_[rid];
  if (!s.swapped) {
    *err = "swap_in: request " + std::to_string(rid) + " is not swapped out";
    return kInvalidArg;
  }
  const int64_t n = ceil_div(s.len, block_size_);
  if (n > static_cast<int64_t>(free_.size())) {
    *err = "swap_in: need " + std::to_string(n) + " blocks, " + std::to_string(free_.size()) +
           " free";
    return kNoBlocks;
  }
  s.table.clear();
  for (int64_t j = 0; j < n; ++j) {
    const int32_t b = pop_block();
    refcount_[b] = 1;
    fill_[b] = static_cast<int32_t>(std::min<int64_t>(block_size_, s.len - j * block_size_));
    s.table.push_back(b);
  }
  s.swapped = false;
  *blocks = s.table;
  return kOk;
}

void BlockAllocator::swap_in_undo(int32_t rid) {
  Seq& s = seqs_[rid];
  for (auto it = s.table.rbegin(); it != s.table.rend(); ++it) {
    refcount_[*it] = 0;
    fill_[*it] = 0;
    free_.push_back(*it);
  }
  s.table.clear();
  s.swapped = true;
}

Status BlockAllocator::shared_groups(const int32_t* rids, int32_t n, int32_t unit,
                                     int32_t* seq_shared, int32_t* groups, int32_t* n_groups,
                                     int32_t* max_members, int32_t* max_shared,
                                     std::string* err) const {
  if (!paged_ || n < 0 || (n > 0 && rids == nullptr) || unit <= 0) {
    *err = "shared_groups: bad arguments";
    return kInvalidArg;
  }
  for (int32_t i = 0; i < n; ++i) {
    Status st = check_resident(rids[i], err);
    if (st != kOk) return st;
  }
  *n_groups = 0;
  *max_members = 0;
  *max_shared = 0;
  int32_t i = 0;
  while (i < n) {
    const Seq& f = seqs_[rids[i]];
    int64_t common = f.len;
    int32_t j = i + 1;
    for (; j < n; ++j) {
      const Seq& o = seqs_[rids[j]];
      size_t k = 0;
      while (k < f.table.size() && k < o.table.size() && f.table[k] == o.table[k]) ++k;
      const int64_t c = std::min<int64_t>(static_cast<int64_t>(k) * block_size_, std::min(f.len, o.len));
      if (c < unit) break;
      common = std::min(common, c);
    }
    const int32_t members = j - i;
    const int32_t shared = members >= 2 ? static_cast<int32_t>(common / unit * unit) : 0;
    for (int32_t k = i; k < j; ++k) seq_shared[k] = shared;
    if (shared > 0) {
      groups[2 * *n_groups] = i;
      groups[2 * *n_groups + 1] = members;
      ++*n_groups;
      *max_members = std::max(*max_members, members);
      *max_shared = std::max(*max_shared, shared);
    }
    i = j;
  }
  return kOk;
}

}  // namespace pa
