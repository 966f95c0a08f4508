// Host-side block allocator of the paged KV cache.  Plain C++17, no HIP: it
// builds and runs on any CPU.
//
// Rules (pages: "Running Out of Cache" paging paragraph, block-size paragraph,
// "Fragmentation is lost users"; the PagedAttention summary page, Summary and
// Key points; "Leveraging Low-Level CUDA APIs for vAttention's Dynamic
// Memory" 5.2.3):
//   * fixed blocks of block_size tokens; a block table per request maps its
//     logical blocks to physical ones;
//   * allocate-on-fill: a request takes a block only when its last one is full;
//   * requests can share blocks (fork); a shared partially filled last block is
//     copied when a sharer first writes into it, the last holder writes in
//     place;
//   * finishing or pre-empting a request returns its unshared blocks;
//   * a pre-empted request can instead be swapped out: its blocks are given
//     back but it keeps its reqId and length, and swapping it in later takes
//     fresh blocks for its whole context;
//   * reqIds in [0, max_seqs) are handed out by the allocator.
// Choices where the pages are silent: the free list and the reqId list are
// stacks (last returned, first reused); reserve is all-or-nothing and handles
// requests in the order given.  Swap-out gives blocks back in table order, as
// freeing does; swap-in takes ceil(L / block_size) blocks off the free stack,
// all or nothing.  A swapped-out request cannot grow, fork or be read until it
// is swapped in; it can be freed.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace pa {

enum Status : int {
  kOk = 0,
  kInvalidArg = -1,
  kNoBlocks = -2,
  kNoReqId = -3,
  kUnknownSeq = -4,
};

struct AllocStats {
  int64_t free_blocks = 0, used_blocks = 0, tokens = 0, logical_tokens = 0;
  int64_t reserved_tokens = 0, live_seqs = 0, cow_copies = 0, shared_blocks = 0;
  double utilisation = 0.0;
  int64_t swapped_seqs = 0, swapped_tokens = 0;
};

class BlockAllocator {
 public:
  // paged == false: contiguous per-request layout (no blocks; slot = reqId*S + pos).
  BlockAllocator(int32_t num_blocks, int32_t block_size, int32_t max_seqs, int32_t max_seq_len,
                 bool paged);

  Status set_free_order(const int32_t* ids, int32_t n, std::string* err);
  Status add(int32_t* rid, std::string* err);
  Status fork(int32_t parent, int32_t* child, std::string* err);
  Status free_seq(int32_t rid, std::string* err);
  Status reserve(const int32_t* rids, int32_t n, const int32_t* counts, int32_t* slots,
                 int64_t slots_cap, int32_t* pairs, int32_t pair_cap, int32_t* n_pairs,
                 std::string* err);
  // The checks reserve makes before it changes anything (ids live and
  // resident, each listed once, counts >= 0, lengths within max_seq_len);
  // *total receives the number of slots the call would hand out.
  Status check_growth(const int32_t* rids, int32_t n, const int32_t* counts, int64_t* total,
                      std::string* err) const;
  Status tables(const int32_t* rids, int32_t n, int32_t stride, int32_t* out, int32_t* lens,
                std::string* err) const;
  AllocStats stats() const;

  // Groups of consecutive requests (in the order given) whose tables start
  // with the same blocks: each run of at least two whose common prefix, cut
  // to whole units of `unit` tokens and to every member's length, is at
  // least one unit.  seq_shared[i] gets request i's shared tokens (0 outside
  // groups), groups[2g], groups[2g+1] the first index and size of group g.
  Status shared_groups(const int32_t* rids, int32_t n, int32_t unit, int32_t* seq_shared,
                       int32_t* groups, int32_t* n_groups, int32_t* max_members,
                       int32_t* max_shared, std::string* err) const;

  // Swap-out, in two steps so that the caller can copy the blocks out first:
  // swap_out_blocks reads the resident request's table (its blocks in logical
  // order) and changes nothing; swap_out releases the blocks.
  Status swap_out_blocks(int32_t rid, std::vector<int32_t>* blocks, int32_t* len,
                         std::string* err) const;
  Status swap_out(int32_t rid, std::string* err);
  // Swap-in: fresh blocks for the swapped-out request's whole context, in
  // logical order.  swap_in_undo gives them back, restoring the free stack.
  Status swap_in(int32_t rid, std::vector<int32_t>* blocks, std::string* err);
  void swap_in_undo(int32_t rid);

  // Length of a live request (resident or swapped out); false if not live.
  bool length(int32_t rid, int32_t* len) const {
    if (rid < 0 || rid >= max_seqs_ || !seqs_[rid].live) return false;
    *len = seqs_[rid].len;
    return true;
  }
  bool swapped(int32_t rid) const {
    return rid >= 0 && rid < max_seqs_ && seqs_[rid].live && seqs_[rid].swapped;
  }

  // Blocks currently held by more than one request.
  int64_t shared_blocks() const { return shared_blocks_; }
  bool paged() const { return paged_; }
  int32_t block_size() const { return block_size_; }
  int32_t num_blocks() const { return num_blocks_; }
  int32_t max_seqs() const { return max_seqs_; }
  int32_t max_seq_len() const { return max_seq_len_; }

 private:
  struct Seq {
    bool live = false;
    bool swapped = false;  // live but holding no blocks
    int32_t len = 0;
    std::vector<int32_t> table;
  };

  Status check_live(int32_t rid, std::string* err) const;
  Status check_resident(int32_t rid, std::string* err) const;
  void release(Seq& s);
  int32_t pop_block();

  bool paged_;
  int32_t num_blocks_, block_size_, max_seqs_, max_seq_len_;
  std::vector<int32_t> free_;      // stack: back() is handed out next
  std::vector<int32_t> refcount_;  // share count per block
  std::vector<int32_t> fill_;      // token rows written per block
  std::vector<int32_t> free_ids_;  // stack of free reqIds
  std::vector<Seq> seqs_;          // indexed by reqId
  int64_t cow_copies_ = 0;
  int64_t shared_blocks_ = 0;      // blocks with refcount > 1
  // per-call scratch (kept to avoid reallocating on every reserve)
  mutable std::vector<uint32_t> mark_;
  mutable uint32_t epoch_ = 0;
  std::vector<int32_t> touched_;   // last blocks whose share count a dry run lowered
  std::vector<int32_t> share_;     // dry-run share count of touched blocks
};

}  // namespace pa
