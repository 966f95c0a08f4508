// Random-operation driver for the host block allocator, built by
// tests/test_allocator_asan.py with AddressSanitizer and UBSan (g++, CPU only).
//
// It drives one BlockAllocator through seeded random sequences of add, fork,
// reserve (allocate-on-fill and copy-on-write), free, swap-out / swap-in,
// shared-prefix grouping and deliberately invalid calls, and after every
// operation checks what the paging rules fix ("Running Out of Cache", paging
// paragraph: blocks are taken only when the last one is full, so a request
// wastes less than one block; the PagedAttention summary page, Summary:
// shared blocks are copied when a sharer first writes into them):
//   * every resident request holds ceil(len / block_size) blocks;
//   * distinct blocks held = used blocks, used + free = all blocks;
//   * blocks held by more than one request = the allocator's shared count;
//   * a slot handed out for position p of a request lies in its table entry
//     p / block_size, row p % block_size, in a block no other request holds;
//   * a copy-on-write destination is held by the writer alone, and its source
//     is still held by some other request;
//   * a failed call changes nothing;
//   * once every request is freed, every block is free again.
// Exit status 0 when every check held; otherwise the first failure is printed.
//
//   asan_allocator_driver <seed> <operations>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "block_allocator.hpp"

namespace {

int g_failures = 0;
// what the run exercised, printed at the end so that the test can require it
struct Counts {
  long reserves = 0, slots = 0, cow_pairs = 0, forks = 0, frees = 0, swaps_out = 0, swaps_in = 0,
       undone = 0, refused = 0, groups = 0;
} g_n;

#define CHECK(cond, ...)                                      \
  do {                                                        \
    if (!(cond)) {                                            \
      std::fprintf(stderr, "check failed (%s): ", #cond);     \
      std::fprintf(stderr, __VA_ARGS__);                      \
      std::fprintf(stderr, "\n");                             \
      ++g_failures;                                           \
      return false;                                           \
    }                                                         \
  } while (0)

struct Model {
  int32_t nb, bs, max_seqs, max_len;
  std::map<int32_t, bool> live;  // reqId -> swapped out
};

// Tables and lengths of every live resident request, as the allocator reports them.
bool snapshot(const pa::BlockAllocator& a, const Model& m, std::map<int32_t, std::vector<int32_t>>* tables,
              std::map<int32_t, int32_t>* lens) {
  const int32_t stride = (m.max_len + m.bs - 1) / m.bs;
  for (const auto& kv : m.live) {
    int32_t len = -1;
    CHECK(a.length(kv.first, &len), "request %d should be live", kv.first);
    (*lens)[kv.first] = len;
    if (kv.second) continue;
    std::vector<int32_t> t(stride, -7);
    int32_t l2 = -1;
    std::string err;
    CHECK(a.tables(&kv.first, 1, stride, t.data(), &l2, &err) == pa::kOk, "tables: %s", err.c_str());
    CHECK(l2 == len, "length %d vs %d", l2, len);
    const int32_t held = (len + m.bs - 1) / m.bs;
    for (int32_t j = 0; j < stride; ++j) {
      if (j < held) {
        CHECK(t[j] >= 0 && t[j] < m.nb, "request %d entry %d = %d", kv.first, j, t[j]);
      } else {
        CHECK(t[j] == -1, "request %d padding entry %d = %d", kv.first, j, t[j]);
      }
    }
    t.resize(held);
    (*tables)[kv.first] = t;
  }
  return true;
}

bool invariants(const pa::BlockAllocator& a, const Model& m) {
  std::map<int32_t, std::vector<int32_t>> tables;
  std::map<int32_t, int32_t> lens;
  if (!snapshot(a, m, &tables, &lens)) return false;
  std::map<int32_t, int> holders;
  for (const auto& kv : tables) {
    std::set<int32_t> own(kv.second.begin(), kv.second.end());
    CHECK(own.size() == kv.second.size(), "request %d holds a block twice", kv.first);
    for (int32_t b : own) ++holders[b];
  }
  int64_t shared = 0;
  for (const auto& kv : holders) shared += kv.second > 1;
  const pa::AllocStats st = a.stats();
  CHECK(st.used_blocks == static_cast<int64_t>(holders.size()), "used %lld vs %zu distinct",
        static_cast<long long>(st.used_blocks), holders.size());
  CHECK(st.used_blocks + st.free_blocks == m.nb, "used %lld + free %lld != %d",
        static_cast<long long>(st.used_blocks), static_cast<long long>(st.free_blocks), m.nb);
  CHECK(st.shared_blocks == shared && a.shared_blocks() == shared, "shared %lld vs %lld",
        static_cast<long long>(st.shared_blocks), static_cast<long long>(shared));
  int64_t resident = 0, swapped = 0;
  for (const auto& kv : m.live) (kv.second ? swapped : resident) += 1;
  CHECK(st.live_seqs == resident && st.swapped_seqs == swapped, "live %lld/%lld swapped %lld/%lld",
        static_cast<long long>(st.live_seqs), static_cast<long long>(resident),
        static_cast<long long>(st.swapped_seqs), static_cast<long long>(swapped));
  return true;
}

bool run(uint32_t seed, int ops) {
  std::mt19937 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  Model m;
  m.bs = std::vector<int>{8, 16, 32}[uni(0, 2)];
  m.nb = uni(1, 96);
  m.max_seqs = uni(1, 12);
  m.max_len = uni(1, 12) * m.bs + uni(0, m.bs - 1);
  pa::BlockAllocator a(m.nb, m.bs, m.max_seqs, m.max_len, true);
  std::string err;
  if (uni(0, 1)) {
    std::vector<int32_t> order(m.nb);
    for (int32_t i = 0; i < m.nb; ++i) order[i] = i;
    std::shuffle(order.begin(), order.end(), rng);
    CHECK(a.set_free_order(order.data(), m.nb, &err) == pa::kOk, "set_free_order: %s", err.c_str());
  }
  // invalid free orders: a repeated id, an id out of range, a short list
  if (m.nb >= 2) {
    std::vector<int32_t> bad(m.nb, 0);
    CHECK(a.set_free_order(bad.data(), m.nb, &err) != pa::kOk, "repeated ids accepted");
    bad[0] = m.nb;
    CHECK(a.set_free_order(bad.data(), m.nb, &err) != pa::kOk, "out-of-range id accepted");
    CHECK(a.set_free_order(bad.data(), m.nb - 1, &err) != pa::kOk, "short list accepted");
  }
  if (!invariants(a, m)) return false;

  auto pick_live = [&](bool resident_only) -> int32_t {
    std::vector<int32_t> ids;
    for (const auto& kv : m.live)
      if (!resident_only || !kv.second) ids.push_back(kv.first);
    if (ids.empty()) return -1;
    return ids[uni(0, static_cast<int>(ids.size()) - 1)];
  };

  for (int op = 0; op < ops; ++op) {
    const int kind = uni(0, 9);
    std::map<int32_t, std::vector<int32_t>> before_t;
    std::map<int32_t, int32_t> before_l;
    if (!snapshot(a, m, &before_t, &before_l)) return false;
    const pa::AllocStats before = a.stats();
    bool failed_call = false;
    if (kind == 0 || m.live.empty()) {
      int32_t rid = -1;
      const pa::Status s = a.add(&rid, &err);
      if (s == pa::kOk) {
        CHECK(rid >= 0 && rid < m.max_seqs && !m.live.count(rid), "add gave %d", rid);
        m.live[rid] = false;
      } else {
        CHECK(s == pa::kNoReqId && static_cast<int32_t>(m.live.size()) == m.max_seqs, "add: %s", err.c_str());
        failed_call = true;
      }
    } else if (kind == 1) {
      const int32_t p = pick_live(true);
      if (p < 0) continue;
      int32_t c = -1;
      const pa::Status s = a.fork(p, &c, &err);
      if (s == pa::kOk) {
        m.live[c] = false;
        std::map<int32_t, std::vector<int32_t>> t;
        std::map<int32_t, int32_t> l;
        if (!snapshot(a, m, &t, &l)) return false;
        CHECK(t[c] == t[p] && l[c] == l[p], "fork: child %d differs from parent %d", c, p);
        ++g_n.forks;
      } else {
        failed_call = true;
      }
    } else if (kind <= 5) {
      // reserve for a random subset, one to a few tokens each (sometimes
      // more than fit, sometimes a duplicate or dead id)
      std::vector<int32_t> rids, counts;
      for (const auto& kv : m.live)
        if (!kv.second && uni(0, 2) > 0) {
          rids.push_back(kv.first);
          counts.push_back(uni(0, 4) == 0 ? uni(0, 3 * m.bs) : uni(0, 2));
        }
      const int mess = uni(0, 9);
      bool bad = true;  // the list breaks a rule: reserve must refuse it
      if (mess == 0 && !rids.empty()) {
        rids.push_back(rids[0]);
        counts.push_back(1);
      } else if (mess == 1) {
        rids.push_back(m.max_seqs + 3);
        counts.push_back(1);
      } else if (mess == 2 && !rids.empty()) {
        counts[0] = -1;
      } else {
        bad = false;
      }
      int64_t total = 0;
      for (int32_t c : counts) total += std::max(c, 0);
      std::vector<int32_t> slots(static_cast<size_t>(total) + 1, -9);
      std::vector<int32_t> pairs(2 * rids.size() + 2, -9);
      int32_t n_pairs = -1;
      const int32_t pair_cap = uni(0, 5) == 0 ? 0 : static_cast<int32_t>(rids.size());
      const pa::Status s = a.reserve(rids.data(), static_cast<int32_t>(rids.size()), counts.data(),
                                     slots.data(), total, pairs.data(), pair_cap, &n_pairs, &err);
      if (s == pa::kOk) {
        CHECK(!bad, "reserve accepted a bad list (case %d)", mess);
        ++g_n.reserves;
        g_n.slots += total;
        g_n.cow_pairs += n_pairs;
        std::map<int32_t, std::vector<int32_t>> t;
        std::map<int32_t, int32_t> l;
        if (!snapshot(a, m, &t, &l)) return false;
        int64_t k = 0;
        for (size_t i = 0; i < rids.size(); ++i) {
          const int32_t r = rids[i];
          CHECK(l[r] == before_l[r] + counts[i], "request %d length %d, expected %d", r, l[r],
                before_l[r] + counts[i]);
          for (int32_t j = 0; j < counts[i]; ++j, ++k) {
            const int32_t p = before_l[r] + j;
            const int32_t slot = slots[k];
            CHECK(slot / m.bs == t[r][p / m.bs] && slot % m.bs == p % m.bs,
                  "request %d position %d got slot %d, table entry %d", r, p, slot, t[r][p / m.bs]);
            // nobody else may hold a block that is written into
            int holders = 0;
            for (const auto& kv : t) holders += std::count(kv.second.begin(), kv.second.end(), slot / m.bs) > 0;
            CHECK(holders == 1, "request %d wrote into block %d, held by %d requests", r, slot / m.bs, holders);
          }
        }
        CHECK(n_pairs >= 0 && n_pairs <= pair_cap, "%d copy pairs, cap %d", n_pairs, pair_cap);
        for (int32_t q = 0; q < n_pairs; ++q) {
          const int32_t src = pairs[2 * q], dst = pairs[2 * q + 1];
          CHECK(src != dst && src >= 0 && dst >= 0 && src < m.nb && dst < m.nb, "pair %d -> %d", src, dst);
          int holders_dst = 0, holders_src = 0;
          for (const auto& kv : t) {
            holders_dst += std::count(kv.second.begin(), kv.second.end(), dst) > 0;
            holders_src += std::count(kv.second.begin(), kv.second.end(), src) > 0;
          }
          CHECK(holders_dst == 1, "copy destination %d held by %d requests", dst, holders_dst);
          CHECK(holders_src >= 1, "copy source %d no longer held", src);
        }
      } else {
        failed_call = true;
      }
    } else if (kind == 6) {
      const int32_t r = uni(0, 5) == 0 ? m.max_seqs + uni(0, 3) : pick_live(false);
      if (r < 0) continue;
      const pa::Status s = a.free_seq(r, &err);
      if (s == pa::kOk) {
        CHECK(m.live.count(r), "freed a request that was not live: %d", r);
        m.live.erase(r);
        ++g_n.frees;
      } else {
        CHECK(!m.live.count(r), "free of live request %d failed: %s", r, err.c_str());
        failed_call = true;
      }
    } else if (kind == 7) {
      const int32_t r = pick_live(true);
      if (r < 0) continue;
      std::vector<int32_t> blocks;
      int32_t len = -1;
      CHECK(a.swap_out_blocks(r, &blocks, &len, &err) == pa::kOk, "swap_out_blocks: %s", err.c_str());
      CHECK(blocks == before_t[r] && len == before_l[r], "swap_out_blocks of %d differs from its table", r);
      CHECK(a.swap_out(r, &err) == pa::kOk, "swap_out: %s", err.c_str());
      m.live[r] = true;
      ++g_n.swaps_out;
      CHECK(a.swap_out(r, &err) != pa::kOk, "second swap_out of %d accepted", r);
    } else if (kind == 8) {
      std::vector<int32_t> ids;
      for (const auto& kv : m.live)
        if (kv.second) ids.push_back(kv.first);
      if (ids.empty()) continue;
      const int32_t r = ids[uni(0, static_cast<int>(ids.size()) - 1)];
      std::vector<int32_t> blocks;
      const pa::Status s = a.swap_in(r, &blocks, &err);
      if (s == pa::kOk) {
        CHECK(static_cast<int32_t>(blocks.size()) == (before_l[r] + m.bs - 1) / m.bs, "swap_in of %d: %zu blocks",
              r, blocks.size());
        if (uni(0, 3) == 0) {
          a.swap_in_undo(r);
          ++g_n.undone;
        } else {
          m.live[r] = false;
          ++g_n.swaps_in;
        }
      } else {
        CHECK(s == pa::kNoBlocks, "swap_in of %d: %s", r, err.c_str());
        failed_call = true;
      }
    } else {
      std::vector<int32_t> rids;
      for (const auto& kv : m.live)
        if (!kv.second) rids.push_back(kv.first);
      const int32_t n = static_cast<int32_t>(rids.size());
      std::vector<int32_t> seq_shared(n + 1, -9), groups(2 * n + 2, -9);
      int32_t ng = -1, mm = -1, ms = -1;
      const pa::Status s = a.shared_groups(rids.data(), n, m.bs * uni(1, 2), seq_shared.data(), groups.data(),
                                           &ng, &mm, &ms, &err);
      CHECK(s == pa::kOk, "shared_groups: %s", err.c_str());
      CHECK(ng >= 0 && 2 * ng <= n, "%d groups of %d requests", ng, n);
      for (int32_t g = 0; g < ng; ++g)
        CHECK(groups[2 * g] >= 0 && groups[2 * g + 1] >= 2 && groups[2 * g] + groups[2 * g + 1] <= n,
              "group %d = (%d, %d)", g, groups[2 * g], groups[2 * g + 1]);
      g_n.groups += ng;
      continue;  // read-only
    }
    if (failed_call) {
      ++g_n.refused;
      // a refused call changes nothing
      std::map<int32_t, std::vector<int32_t>> t;
      std::map<int32_t, int32_t> l;
      if (!snapshot(a, m, &t, &l)) return false;
      const pa::AllocStats after = a.stats();
      CHECK(t == before_t && l == before_l, "a refused call (operation %d) changed the tables", kind);
      CHECK(after.free_blocks == before.free_blocks && after.cow_copies == before.cow_copies,
            "a refused call (operation %d) changed the free list or the copy count", kind);
    }
    if (!invariants(a, m)) return false;
  }
  // free everything: every block comes back
  while (!m.live.empty()) {
    const int32_t r = m.live.begin()->first;
    CHECK(a.free_seq(r, &err) == pa::kOk, "final free of %d: %s", r, err.c_str());
    m.live.erase(r);
  }
  CHECK(a.stats().free_blocks == m.nb, "%lld of %d blocks free at the end",
        static_cast<long long>(a.stats().free_blocks), m.nb);
  return invariants(a, m);
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s <seed> <operations>\n", argv[0]);
    return 2;
  }
  const uint32_t seed = static_cast<uint32_t>(std::strtoul(argv[1], nullptr, 10));
  const int ops = std::atoi(argv[2]);
  if (!run(seed, ops)) {
    std::fprintf(stderr, "seed %u failed\n", seed);
    return 1;
  }
  std::printf("reserves=%ld slots=%ld cow_pairs=%ld forks=%ld frees=%ld swaps_out=%ld swaps_in=%ld "
              "undone=%ld refused=%ld groups=%ld\n",
              g_n.reserves, g_n.slots, g_n.cow_pairs, g_n.forks, g_n.frees, g_n.swaps_out, g_n.swaps_in,
              g_n.undone, g_n.refused, g_n.groups);
  return g_failures == 0 ? 0 : 1;
}
