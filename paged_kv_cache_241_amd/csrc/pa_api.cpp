// C ABI of libpa.so (include/pa.h): argument checks, error text, the host
// block allocator and kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <exception>
#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "../../include/pa.h"
#include "block_allocator.hpp"
#include "kernels.hpp"
#include "vmm.hpp"

static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::kStaticScratchBytes,
              "pa.h states the scratch size of pa_append_decode_noalloc");

struct pa_pool {
  pa_pool_desc desc;
  pa::CacheGeom geom;
  pa::BlockAllocator alloc;
  pa::VirtualCache* vmm = nullptr;  // demand-paged contiguous caches (owned), or null
  pa_pool(const pa_pool_desc& d, const pa::CacheGeom& g)
      : desc(d),
        geom(g),
        alloc(d.num_blocks, d.block_size, d.max_seqs, d.max_seq_len, d.layout == PA_PAGED) {}
  ~pa_pool() { delete vmm; }
  pa_pool(const pa_pool&) = delete;
  pa_pool& operator=(const pa_pool&) = delete;
};

namespace {

thread_local std::string g_err;

pa_status fail(pa_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

// Every pa_status entry point runs its body through guarded(): nothing
// throws across the C ABI.  A failed host allocation (the allocator's tables,
// error text) becomes PA_ERR_NO_MEMORY, anything else PA_ERR_INVALID_ARG.
template <class F>
pa_status guarded(const char* who, F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(PA_ERR_NO_MEMORY, std::string(who) + ": out of host memory");
  } catch (const std::exception& e) {
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": " + e.what());
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": unexpected error");
  }
}

pa_status from_alloc(pa::Status st, const std::string& msg) {
  if (st == pa::kOk) return PA_OK;
  g_err = msg;
  return static_cast<pa_status>(static_cast<int>(st));
}

int32_t elt_bytes(pa_dtype t) { return t == PA_BF16 ? 2 : (t == PA_F32 ? 4 : 0); }

// Empty string if desc is valid, else the reason.
std::string check_desc(const pa_pool_desc* d) {
  if (d == nullptr) return "null pool descriptor";
  if (d->num_layers < 1) return "num_layers must be >= 1";
  if (d->block_size != 8 && d->block_size != 16 && d->block_size != 32)
    return "block_size must be 8, 16 or 32";
  if (d->num_kv_heads < 1) return "num_kv_heads must be >= 1";
  if (d->head_dim != 64 && d->head_dim != 128) return "head_dim must be 64 or 128";
  if (elt_bytes(d->kv_dtype) == 0) return "kv_dtype must be PA_F32 or PA_BF16";
  if (d->layout != PA_PAGED && d->layout != PA_CONTIGUOUS) return "unknown layout";
  if (d->max_seqs < 1) return "max_seqs must be >= 1";
  if (d->max_seq_len < 1) return "max_seq_len must be >= 1";
  if (d->layout == PA_PAGED) {
    if (d->num_blocks < 1) return "num_blocks must be >= 1";
    if (static_cast<int64_t>(d->num_blocks) * d->block_size > INT32_MAX)
      return "num_blocks * block_size must fit in int32 slots";
  } else {
    if (d->max_seq_len % d->block_size != 0)
      return "contiguous layout: max_seq_len must be a multiple of block_size";
    if (static_cast<int64_t>(d->max_seqs) * d->max_seq_len > INT32_MAX)
      return "max_seqs * max_seq_len must fit in int32 slots";
  }
  return "";
}

// Bytes of one block of one layer: every KV head's K and V tiles.
int64_t block_bytes(const pa_pool_desc* d) {
  return static_cast<int64_t>(d->num_kv_heads) * 2 * d->head_dim * d->block_size * elt_bytes(d->kv_dtype);
}

// Bytes of one layer of the cache (K and V).
int64_t layer_bytes(const pa_pool_desc* d) {
  const int64_t blocks = d->layout == PA_PAGED ? d->num_blocks
                                               : static_cast<int64_t>(d->max_seqs) * (d->max_seq_len / d->block_size);
  return blocks * block_bytes(d);
}

// Decode launch shape.  A workgroup of W waves handles one (sequence, KV
// head, context partition).  The grid aims at about kTargetWaves waves (8 per
// CU, all resident at once) so that one launch covers the chip without a
// split-K merge where it can: on MI355X one partition per sequence beats two
// by 12% at batch 64 x 8 KV heads x 1024 tokens and by 28% on 2304-token
// shared-prompt samples.  Only long contexts (> kSplitAbove tokens, where a
// ragged batch's few longest sequences would otherwise run alone at the end)
// are cut into kSplitTokens partitions (22% faster on the ragged
// Exp(1024)+Exp(256) mix than one partition).  Partitions hold at least
// kMinTokens so that every wave streams several chunks.
constexpr int64_t kTargetWaves = 2048;
constexpr int32_t kSplitAbove = 4096;
constexpr int32_t kSplitTokens = 1024;
constexpr int32_t kMinTokens = 256;

int32_t partition_unit(const pa_pool* p) { return p->desc.block_size > 16 ? p->desc.block_size : 16; }

int32_t choose_partition_tokens(const pa_pool* p, int32_t num_seqs, int32_t max_context,
                                int32_t partition_tokens) {
  const int32_t unit = partition_unit(p);
  if (partition_tokens > 0) return partition_tokens;
  if (max_context <= 0) return unit;
  const int64_t waves = static_cast<int64_t>(num_seqs) * p->desc.num_kv_heads * pa::kDecodeWaves;
  const int64_t parts = (kTargetWaves + waves - 1) / waves;
  int64_t tokens = (max_context + parts - 1) / parts;
  if (max_context > kSplitAbove && tokens > kSplitTokens) tokens = kSplitTokens;
  if (tokens < kMinTokens) tokens = kMinTokens;
  tokens = (tokens + unit - 1) / unit * unit;
  return static_cast<int32_t>(tokens);
}

int32_t num_partitions(int32_t max_context, int32_t ptokens) {
  return max_context <= 0 ? 1 : (max_context + ptokens - 1) / ptokens;
}

bool bad_partition(const pa_pool* p, int32_t partition_tokens) {
  return partition_tokens < 0 || partition_tokens % partition_unit(p) != 0;
}


int32_t num_queries_per_kv(int32_t num_q_heads, int32_t num_kv_heads) { return num_q_heads / num_kv_heads; }

pa::CacheGeom make_geom(const pa_pool_desc* desc, void* cache) {
  pa::CacheGeom g;
  g.base = static_cast<char*>(cache);
  g.layer_bytes = layer_bytes(desc);
  g.tile_bytes = static_cast<int64_t>(desc->head_dim) * desc->block_size * elt_bytes(desc->kv_dtype);
  g.num_layers = desc->num_layers;
  g.num_kv_heads = desc->num_kv_heads;
  g.head_dim = desc->head_dim;
  g.elt = elt_bytes(desc->kv_dtype);
  g.block_size = desc->block_size;
  g.paged = desc->layout == PA_PAGED ? 1 : 0;
  g.blocks_per_seq = g.paged ? 0 : desc->max_seq_len / desc->block_size;
  return g;
}

// Length of a live request of a paged pool (resident or swapped out).
pa_status swap_length(const pa_pool* pool, int32_t req_id, const char* who, int32_t* len) {
  if (!pool->geom.paged)
    return fail(PA_ERR_INVALID_ARG, std::string(who) + ": swapping needs the paged layout");
  if (!pool->alloc.length(req_id, len))
    return fail(PA_ERR_UNKNOWN_SEQ, std::string(who) + ": request id " + std::to_string(req_id) +
                                        " is not live");
  return PA_OK;
}

size_t image_bytes(const pa_pool* pool, int32_t len) {
  const pa_pool_desc& d = pool->desc;
  const int64_t blocks = (static_cast<int64_t>(len) + d.block_size - 1) / d.block_size;
  return static_cast<size_t>(static_cast<int64_t>(d.num_layers) * blocks * 2 * d.num_kv_heads *
                             d.head_dim * d.block_size * elt_bytes(d.kv_dtype));
}

// The image must hold the request's blocks and be reachable by the kernels:
// device memory as it is, pinned host memory through its device mapping.
// Anything else (pageable host memory) is refused here rather than faulted on.
// No image at all (NULL with capacity 0) means no copy: *dev stays NULL.
pa_status check_image(const pa_pool* pool, const void* image, size_t cap, int32_t len,
                      const char* who, char** dev) {
  const std::string w(who);
  const size_t need = image_bytes(pool, len);
  *dev = nullptr;
  if (image == nullptr && cap == 0) return PA_OK;
  if (need == 0) return PA_OK;
  if (image == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null image with a nonzero capacity");
  if (cap < need)
    return fail(PA_ERR_INVALID_ARG, w + ": image holds " + std::to_string(cap) + " bytes, " +
                                        std::to_string(need) + " needed");
  if (reinterpret_cast<uintptr_t>(image) & 15) return fail(PA_ERR_INVALID_ARG, w + ": image must be 16-byte aligned");
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, image) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the next launch
    return fail(PA_ERR_INVALID_ARG, w + ": image is neither device nor pinned host memory");
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *dev = static_cast<char*>(const_cast<void*>(image));
  } else if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    const char* hp = static_cast<const char*>(attr.hostPointer ? attr.hostPointer : image);
    *dev = static_cast<char*>(attr.devicePointer) + (static_cast<const char*>(image) - hp);
  } else {
    return fail(PA_ERR_INVALID_ARG, w + ": image is neither device nor pinned host memory");
  }
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_cache_bytes(const pa_pool_desc* desc) {
  if (!check_desc(desc).empty()) return 0;
  return static_cast<size_t>(layer_bytes(desc) * desc->num_layers);
}

size_t pa_bytes_per_token(const pa_pool_desc* desc) {
  if (!check_desc(desc).empty()) return 0;
  return static_cast<size_t>(2) * desc->num_layers * desc->num_kv_heads * desc->head_dim *
         elt_bytes(desc->kv_dtype);
}

pa_status pa_create_pool(const pa_pool_desc* desc, void* d_cache, pa_pool** out) {
  return guarded("create_pool", [&]() -> pa_status {
    if (out == nullptr) return fail(PA_ERR_INVALID_ARG, "create_pool: null output");
    *out = nullptr;
    const std::string why = check_desc(desc);
    if (!why.empty()) return fail(PA_ERR_INVALID_ARG, "create_pool: " + why);
    if (d_cache == nullptr) return fail(PA_ERR_INVALID_ARG, "create_pool: null cache pointer");
    if (reinterpret_cast<uintptr_t>(d_cache) & 15)
      return fail(PA_ERR_INVALID_ARG, "create_pool: the cache must be 16-byte aligned");
    pa_pool* p = new (std::nothrow) pa_pool(*desc, make_geom(desc, d_cache));
    if (p == nullptr) return fail(PA_ERR_NO_MEMORY, "create_pool: out of host memory");
    *out = p;
    return PA_OK;
  });
}

pa_status pa_create_pool_vmm(const pa_pool_desc* desc, size_t physical_bytes, pa_pool** out) {
  return guarded("create_pool_vmm", [&]() -> pa_status {
    if (out == nullptr) return fail(PA_ERR_INVALID_ARG, "create_pool_vmm: null output");
    *out = nullptr;
    const std::string why = check_desc(desc);
    if (!why.empty()) return fail(PA_ERR_INVALID_ARG, "create_pool_vmm: " + why);
    if (desc->layout != PA_CONTIGUOUS)
      return fail(PA_ERR_INVALID_ARG, "create_pool_vmm: demand paging backs the contiguous layout");
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(PA_ERR_HIP, std::string("create_pool_vmm: ") + hipGetErrorString(e));
    }
    const int64_t region = layer_bytes(desc) / desc->max_seqs;
    pa::VirtualCache* vc = nullptr;
    const std::string err =
        pa::VirtualCache::create(desc->num_layers, desc->max_seqs, region, physical_bytes, device, &vc);
    if (!err.empty()) return fail(PA_ERR_UNSUPPORTED, "create_pool_vmm: " + err);
    pa_pool* p = new (std::nothrow) pa_pool(*desc, make_geom(desc, vc->base()));
    if (p == nullptr) {
      delete vc;
      return fail(PA_ERR_NO_MEMORY, "create_pool_vmm: out of host memory");
    }
    p->vmm = vc;
    *out = p;
    return PA_OK;
  });
}

pa_status pa_vmm_info(const pa_pool* pool, pa_vmm_stats* out) {
  return guarded("vmm_info", [&]() -> pa_status {
    if (pool == nullptr || out == nullptr) return fail(PA_ERR_INVALID_ARG, "vmm_info: null argument");
    if (pool->vmm == nullptr) return fail(PA_ERR_INVALID_ARG, "vmm_info: not a demand-paged pool");
    out->page_bytes = pool->vmm->page_bytes();
    out->mapped_bytes = pool->vmm->bytes_mapped();
    out->budget_bytes = pool->vmm->bytes_budget();
    out->region_bytes = pool->vmm->region_bytes();
    return PA_OK;
  });
}

pa_status pa_vmm_trim(pa_pool* pool, int64_t* freed_bytes_out) {
  return guarded("vmm_trim", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "vmm_trim: null pool");
    if (pool->vmm == nullptr) return fail(PA_ERR_INVALID_ARG, "vmm_trim: not a demand-paged pool");
    const int64_t before = pool->vmm->bytes_mapped();
    for (int32_t r = 0; r < pool->desc.max_seqs; ++r) {
      int32_t len = 0;
      if (!pool->alloc.length(r, &len)) pool->vmm->trim(r);
    }
    if (freed_bytes_out) *freed_bytes_out = before - pool->vmm->bytes_mapped();
    return PA_OK;
  });
}

pa_status pa_destroy_pool(pa_pool* pool) {
  return guarded("destroy_pool", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "destroy_pool: null pool");
    delete pool;
    return PA_OK;
  });
}

pa_status pa_set_free_order(pa_pool* pool, const int32_t* block_ids, int32_t n) {
  return guarded("set_free_order", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "set_free_order: null pool");
    std::string err;
    pa::Status st = pool->alloc.set_free_order(block_ids, n, &err);
    return from_alloc(st, err);
  });
}

pa_status pa_seq_add(pa_pool* pool, int32_t* req_id_out) {
  return guarded("seq_add", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "seq_add: null pool");
    std::string err;
    pa::Status st = pool->alloc.add(req_id_out, &err);
    return from_alloc(st, err);
  });
}

pa_status pa_seq_fork(pa_pool* pool, int32_t parent, int32_t* child_out) {
  return guarded("seq_fork", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "seq_fork: null pool");
    std::string err;
    pa::Status st = pool->alloc.fork(parent, child_out, &err);
    return from_alloc(st, err);
  });
}

pa_status pa_seq_free(pa_pool* pool, int32_t req_id) {
  return guarded("seq_free", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "seq_free: null pool");
    std::string err;
    pa::Status st = pool->alloc.free_seq(req_id, &err);
    return from_alloc(st, err);
  });
}

pa_status pa_reserve(pa_pool* pool, const int32_t* req_ids, int32_t n, const int32_t* counts,
                     int32_t* slots_out, int64_t slots_cap, int32_t* cow_pairs_out,
                     int32_t cow_cap, int32_t* n_cow_out) {
  return guarded("reserve", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "reserve: null pool");
    std::string err;
    if (pool->vmm != nullptr) {
      // demand paging: back every listed request's grown prefix first, all or
      // nothing against the physical budget
      int64_t total = 0;
      pa::Status st = pool->alloc.check_growth(req_ids, n, counts, &total, &err);
      if (st != pa::kOk) return from_alloc(st, err);
      if (total > slots_cap || (total > 0 && slots_out == nullptr))
        return fail(PA_ERR_INVALID_ARG, "reserve: slots_out holds " + std::to_string(slots_cap) +
                                            " slots, " + std::to_string(total) + " needed");
      const int64_t unit = block_bytes(&pool->desc);
      std::vector<int64_t> bytes(n);
      int64_t more = 0;
      for (int32_t i = 0; i < n; ++i) {
        int32_t len = 0;
        pool->alloc.length(req_ids[i], &len);
        const int64_t grown = static_cast<int64_t>(len) + (counts ? counts[i] : 1);
        bytes[i] = (grown + pool->desc.block_size - 1) / pool->desc.block_size * unit;
        more += pool->vmm->bytes_short(req_ids[i], bytes[i]);
      }
      if (more > pool->vmm->bytes_free())
        return fail(PA_ERR_NO_BLOCKS, "reserve: needs " + std::to_string(more) +
                                          " more bytes of physical memory, " +
                                          std::to_string(pool->vmm->bytes_free()) + " left");
      for (int32_t i = 0; i < n; ++i) {
        const std::string e = pool->vmm->grow(req_ids[i], bytes[i]);
        if (!e.empty()) return fail(PA_ERR_HIP, "reserve: " + e);
      }
    }
    pa::Status st = pool->alloc.reserve(req_ids, n, counts, slots_out, slots_cap, cow_pairs_out,
                                        cow_cap, n_cow_out, &err);
    return from_alloc(st, err);
  });
}

pa_status pa_get_block_tables(const pa_pool* pool, const int32_t* req_ids, int32_t n,
                              int32_t stride, int32_t* tables_out, int32_t* lens_out) {
  return guarded("get_block_tables", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "get_block_tables: null pool");
    std::string err;
    pa::Status st = pool->alloc.tables(req_ids, n, stride, tables_out, lens_out, &err);
    return from_alloc(st, err);
  });
}

pa_status pa_get_stats(const pa_pool* pool, pa_stats* out) {
  return guarded("get_stats", [&]() -> pa_status {
    if (pool == nullptr || out == nullptr) return fail(PA_ERR_INVALID_ARG, "get_stats: null argument");
    const pa::AllocStats s = pool->alloc.stats();
    out->free_blocks = s.free_blocks;
    out->used_blocks = s.used_blocks;
    out->tokens = s.tokens;
    out->logical_tokens = s.logical_tokens;
    out->reserved_tokens = s.reserved_tokens;
    out->live_seqs = s.live_seqs;
    out->cow_copies = s.cow_copies;
    out->shared_blocks = s.shared_blocks;
    out->utilisation = s.utilisation;
    out->swapped_seqs = s.swapped_seqs;
    out->swapped_tokens = s.swapped_tokens;
    return PA_OK;
  });
}

pa_status pa_swap_bytes(const pa_pool* pool, int32_t req_id, size_t* bytes_out) {
  return guarded("swap_bytes", [&]() -> pa_status {
    if (pool == nullptr || bytes_out == nullptr) return fail(PA_ERR_INVALID_ARG, "swap_bytes: null argument");
    int32_t len = 0;
    pa_status st = swap_length(pool, req_id, "swap_bytes", &len);
    if (st != PA_OK) return st;
    *bytes_out = image_bytes(pool, len);
    return PA_OK;
  });
}

pa_status pa_swap_out(pa_pool* pool, int32_t req_id, void* d_image, size_t image_bytes_cap,
                      void* stream) {
  return guarded("swap_out", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "swap_out: null pool");
    std::vector<int32_t> blocks;
    int32_t len = 0;
    std::string err;
    pa::Status s = pool->alloc.swap_out_blocks(req_id, &blocks, &len, &err);
    if (s != pa::kOk) return fail(static_cast<pa_status>(s), "swap_out: " + err);
    char* dev = nullptr;
    pa_status st = check_image(pool, d_image, image_bytes_cap, len, "swap_out", &dev);
    if (st != PA_OK) return st;
    if (dev != nullptr) {
      hipError_t e = pa::launch_swap(pool->geom, blocks.data(), static_cast<int32_t>(blocks.size()),
                                     dev, true, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("swap_out: ") + hipGetErrorString(e));
    }
    s = pool->alloc.swap_out(req_id, &err);
    if (s != pa::kOk) return fail(static_cast<pa_status>(s), "swap_out: " + err);
    return PA_OK;
  });
}

pa_status pa_swap_in(pa_pool* pool, int32_t req_id, const void* d_image, size_t image_bytes_cap,
                     void* stream) {
  return guarded("swap_in", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "swap_in: null pool");
    int32_t len = 0;
    pa_status st = swap_length(pool, req_id, "swap_in", &len);
    if (st != PA_OK) return st;
    if (!pool->alloc.swapped(req_id))
      return fail(PA_ERR_INVALID_ARG, "swap_in: request " + std::to_string(req_id) + " is not swapped out");
    char* dev = nullptr;
    st = check_image(pool, d_image, image_bytes_cap, len, "swap_in", &dev);
    if (st != PA_OK) return st;
    std::vector<int32_t> blocks;
    std::string err;
    pa::Status s = pool->alloc.swap_in(req_id, &blocks, &err);
    if (s != pa::kOk) return fail(static_cast<pa_status>(s), "swap_in: " + err);
    if (dev != nullptr) {
      hipError_t e = pa::launch_swap(pool->geom, blocks.data(), static_cast<int32_t>(blocks.size()),
                                     dev, false, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) {
        pool->alloc.swap_in_undo(req_id);
        return fail(PA_ERR_HIP, std::string("swap_in: ") + hipGetErrorString(e));
      }
    }
    return PA_OK;
  });
}

pa_status pa_copy_blocks(pa_pool* pool, const int32_t* d_pairs, int32_t n, void* stream) {
  return guarded("copy_blocks", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "copy_blocks: null pool");
    if (n < 0) return fail(PA_ERR_INVALID_ARG, "copy_blocks: negative pair count");
    if (n == 0) return PA_OK;
    if (!pool->geom.paged) return fail(PA_ERR_INVALID_ARG, "copy_blocks: contiguous pool has no blocks");
    if (d_pairs == nullptr) return fail(PA_ERR_INVALID_ARG, "copy_blocks: null pairs");
    hipError_t e = pa::launch_copy_blocks(pool->geom, d_pairs, n, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("copy_blocks: ") + hipGetErrorString(e));
    return PA_OK;
  });
}

pa_status pa_append_kv(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                       const int32_t* d_slots, int32_t n, void* stream) {
  return guarded("append_kv", [&]() -> pa_status {
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, "append_kv: null pool");
    if (layer < 0 || layer >= pool->desc.num_layers)
      return fail(PA_ERR_INVALID_ARG, "append_kv: layer out of range");
    if (n < 0) return fail(PA_ERR_INVALID_ARG, "append_kv: negative token count");
    if (n == 0) return PA_OK;
    if (d_k == nullptr || d_v == nullptr || d_slots == nullptr)
      return fail(PA_ERR_INVALID_ARG, "append_kv: null device pointer");
    if ((reinterpret_cast<uintptr_t>(d_k) | reinterpret_cast<uintptr_t>(d_v)) & 15)
      return fail(PA_ERR_INVALID_ARG, "append_kv: k and v must be 16-byte aligned");
    hipError_t e = pa::launch_append(pool->geom, layer, d_k, d_v, d_slots, n,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, std::string("append_kv: ") + hipGetErrorString(e));
    return PA_OK;
  });
}

int32_t pa_decode_partition_tokens(const pa_pool* pool, int32_t num_seqs, int32_t max_context,
                                   int32_t partition_tokens) {
  if (pool == nullptr || num_seqs < 0 || max_context < 0 || bad_partition(pool, partition_tokens)) return 0;
  return choose_partition_tokens(pool, num_seqs, max_context, partition_tokens);
}

size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_context, int32_t partition_tokens) {
  if (pool == nullptr || num_seqs < 0 || max_context < 0 || bad_partition(pool, partition_tokens)) return 0;
  const int32_t pt = choose_partition_tokens(pool, num_seqs, max_context, partition_tokens);
  return pa::decode_workspace_bytes(num_seqs, num_q_heads, pool->desc.head_dim,
                                    num_partitions(max_context, pt));
}

}  // extern "C"

namespace {
pa_status decode_impl(const char* who, pa_pool* pool, int32_t layer, const void* d_k_new,
                      const void* d_v_new, const int32_t* d_slots, const void* d_q,
                      pa_dtype q_dtype, int32_t num_q_heads, float scale,
                      const int32_t* d_block_tables, int32_t table_stride,
                      const int32_t* d_req_ids, const int32_t* d_context_lens, int32_t num_seqs,
                      int32_t max_context, int32_t partition_tokens, float* d_out,
                      void* d_workspace, size_t workspace_bytes, void* stream,
                      const int32_t* d_seq_shared = nullptr, const int32_t* d_groups = nullptr,
                      int32_t num_groups = 0, int32_t max_members = 0, int32_t max_shared = 0,
                      bool static_workspace = false, bool plan_made = false) {
  const std::string w(who);
  const bool shared = d_seq_shared != nullptr;
  if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null pool");
  const pa_pool_desc& d = pool->desc;
  if (layer < 0 || layer >= d.num_layers) return fail(PA_ERR_INVALID_ARG, w + ": layer out of range");
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, w + ": negative num_seqs");
  if (num_seqs == 0) return PA_OK;
  if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, w + ": num_q_heads must be a positive multiple of num_kv_heads");
  if (q_dtype != d.kv_dtype)
    return fail(PA_ERR_UNSUPPORTED, w + ": q_dtype must equal the cache's kv_dtype");
  if (num_q_heads / d.num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, w + ": GQA groups of more than 16 query heads");
  if (max_context < 0 || max_context > d.max_seq_len)
    return fail(PA_ERR_INVALID_ARG, w + ": max_context must be in [0, max_seq_len]");
  if (bad_partition(pool, partition_tokens))
    return fail(PA_ERR_INVALID_ARG,
                w + ": partition_tokens must be 0 or a positive multiple of 16 and of block_size");
  if (d_q == nullptr || d_context_lens == nullptr || d_out == nullptr)
    return fail(PA_ERR_INVALID_ARG, w + ": null device pointer");
  if (reinterpret_cast<uintptr_t>(d_q) & 15) return fail(PA_ERR_INVALID_ARG, w + ": q must be 16-byte aligned");
  const int32_t bs = d.block_size;
  const int32_t nblk = (max_context + bs - 1) / bs;
  if (d.layout == PA_PAGED) {
    if (d_block_tables == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null block tables");
    if (table_stride < nblk)
      return fail(PA_ERR_INVALID_ARG, w + ": table_stride is shorter than ceil(max_context / block_size)");
  } else if (d_req_ids == nullptr && num_seqs > d.max_seqs) {
    // without request ids sequence s reads request s's sub-tensor, which
    // exists for s < max_seqs only
    return fail(PA_ERR_INVALID_ARG, w + ": num_seqs " + std::to_string(num_seqs) + " exceeds max_seqs " +
                                        std::to_string(d.max_seqs) + " and no request ids are given");
  }
  if (!(scale == scale)) return fail(PA_ERR_INVALID_ARG, w + ": scale is NaN");
  if (shared) {
    if (d.layout != PA_PAGED) return fail(PA_ERR_INVALID_ARG, w + ": shared prefixes need the paged layout");
    if (partition_tokens <= 0)
      return fail(PA_ERR_INVALID_ARG, w + ": give partition_tokens (the shared prefixes are whole partitions)");
    if (num_groups < 0 || max_shared < 0 || max_shared % partition_tokens != 0 || max_shared > max_context)
      return fail(PA_ERR_INVALID_ARG, w + ": max_shared must be a multiple of partition_tokens within max_context");
    if (num_groups > 0 && (d_groups == nullptr || max_members < 1))
      return fail(PA_ERR_INVALID_ARG, w + ": null groups or max_members < 1");
  }
  const int64_t grid = static_cast<int64_t>(num_seqs) * d.num_kv_heads;
  pa::DecodeArgs a;
  a.q = d_q;
  a.tables = d.layout == PA_PAGED ? d_block_tables : nullptr;
  a.req_ids = d.layout == PA_PAGED ? nullptr : d_req_ids;
  a.lens = d_context_lens;
  a.out = d_out;
  a.layer = layer;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.table_stride = table_stride;
  const int32_t pt = choose_partition_tokens(pool, num_seqs, max_context, partition_tokens);
  a.partition_chunks = pt / 16;
  a.num_partitions = num_partitions(max_context, pt);
  a.max_context = max_context;
  if (shared) {
    // partials and the merge even where one partition would cover a context
    a.num_partitions = std::max(a.num_partitions, 2);
    a.seq_shared = d_seq_shared;
  }
  if (d_k_new != nullptr) {
    a.new_k = d_k_new;
    a.new_v = d_v_new;
    a.new_slots = d_slots;
  }
  // the shared pass reads shared blocks once; the partition kernel then reads
  // private blocks only
  a.streaming = shared || pool->alloc.shared_blocks() == 0 ? 1 : 0;
  a.scale = scale;
  if (grid * a.num_partitions > INT32_MAX) return fail(PA_ERR_INVALID_ARG, w + ": launch too large");
  const size_t need = pa::decode_workspace_bytes(num_seqs, num_q_heads, d.head_dim, a.num_partitions);
  if (need > 0 && static_workspace) {
    // the library's own device array instead of a caller's workspace
    if (need > pa::kStaticScratchBytes)
      return fail(PA_ERR_WORKSPACE, w + ": the split-K partials need " + std::to_string(need) +
                                        " bytes, more than the " + std::to_string(pa::kStaticScratchBytes) +
                                        " bytes of the library's scratch (use pa_append_decode with a workspace)");
    void* p = nullptr;
    const hipError_t e = pa::static_scratch(&p);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(PA_ERR_HIP, w + ": scratch address: " + hipGetErrorString(e));
    }
    a.ws = static_cast<float*>(p);
  } else if (need > 0) {
    if (d_workspace == nullptr || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, w + ": workspace needs " + std::to_string(need) + " bytes, got " +
                                        std::to_string(d_workspace ? workspace_bytes : 0));
    if (reinterpret_cast<uintptr_t>(d_workspace) & 15)
      return fail(PA_ERR_INVALID_ARG, w + ": workspace must be 16-byte aligned");
    a.ws = static_cast<float*>(d_workspace);
  }
  bool supported = true;
  const int kind = d.kv_dtype == PA_BF16 ? pa::kBF16 : pa::kF32;
  if (shared && num_groups > 0 && max_shared > 0) {
    pa::SharedArgs sh;
    sh.groups = d_groups;
    sh.num_groups = num_groups;
    const int64_t cols = static_cast<int64_t>(max_members) * (num_queries_per_kv(num_q_heads, d.num_kv_heads));
    sh.col_blocks = static_cast<int32_t>((cols + 63) / 64);
    sh.shared_parts = max_shared / pt;
    const int64_t n_shared = static_cast<int64_t>(num_groups) * d.num_kv_heads * sh.col_blocks * sh.shared_parts;
    if (n_shared + grid * a.num_partitions > INT32_MAX) return fail(PA_ERR_INVALID_ARG, w + ": launch too large");
    sh.n_shared = static_cast<int32_t>(n_shared);
    // one launch for the shared pass and the private partitions, then the merge
    hipError_t es = pa::launch_decode_shared(pool->geom, kind, a, sh, &supported,
                                             static_cast<hipStream_t>(stream));
    if (!supported) return fail(PA_ERR_UNSUPPORTED, w + ": no kernel for this shape");
    if (es == hipSuccess) es = pa::launch_merge(pool->geom, a, static_cast<hipStream_t>(stream));
    if (es != hipSuccess) return fail(PA_ERR_HIP, std::string(w + ": ") + hipGetErrorString(es));
    return PA_OK;
  }
  hipError_t e = pa::launch_decode(pool->geom, kind, a, &supported, static_cast<hipStream_t>(stream),
                                   plan_made);
  if (!supported) return fail(PA_ERR_UNSUPPORTED, w + ": no kernel for this shape");
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string(w + ": ") + hipGetErrorString(e));
  return PA_OK;
}
}  // namespace

extern "C" {

pa_status pa_decode(pa_pool* pool, int32_t layer, const void* d_q, pa_dtype q_dtype,
                    int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                    int32_t table_stride, const int32_t* d_req_ids,
                    const int32_t* d_context_lens, int32_t num_seqs, int32_t max_context,
                    int32_t partition_tokens, float* d_out, void* d_workspace,
                    size_t workspace_bytes, void* stream) {
  return guarded("decode", [&]() -> pa_status {
    return decode_impl("decode", pool, layer, nullptr, nullptr, nullptr, d_q, q_dtype, num_q_heads,
                       scale, d_block_tables, table_stride, d_req_ids, d_context_lens, num_seqs,
                       max_context, partition_tokens, d_out, d_workspace, workspace_bytes, stream);
  });
}

pa_status pa_append_decode(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                           const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                           int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                           int32_t table_stride, const int32_t* d_req_ids,
                           const int32_t* d_context_lens, int32_t num_seqs, int32_t max_context,
                           int32_t partition_tokens, float* d_out, void* d_workspace,
                           size_t workspace_bytes, void* stream) {
  return guarded("append_decode", [&]() -> pa_status {
    if (d_k == nullptr || d_v == nullptr || d_slots == nullptr)
      return fail(PA_ERR_INVALID_ARG, "append_decode: null k, v or slots");
    if ((reinterpret_cast<uintptr_t>(d_k) | reinterpret_cast<uintptr_t>(d_v)) & 15)
      return fail(PA_ERR_INVALID_ARG, "append_decode: k and v must be 16-byte aligned");
    return decode_impl("append_decode", pool, layer, d_k, d_v, d_slots, d_q, q_dtype, num_q_heads,
                       scale, d_block_tables, table_stride, d_req_ids, d_context_lens, num_seqs,
                       max_context, partition_tokens, d_out, d_workspace, workspace_bytes, stream);
  });
}

pa_status pa_decode_plan(pa_pool* pool, const int32_t* d_context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_context, int32_t partition_tokens,
                         void* d_workspace, size_t workspace_bytes, int32_t* planned_out, void* stream) {
  return guarded("decode_plan", [&]() -> pa_status {
    const std::string w = "decode_plan";
    if (planned_out != nullptr) *planned_out = 0;
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null pool");
    const pa_pool_desc& d = pool->desc;
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, w + ": negative num_seqs");
    if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
      return fail(PA_ERR_INVALID_ARG, w + ": num_q_heads must be a positive multiple of num_kv_heads");
    if (max_context < 0 || max_context > d.max_seq_len)
      return fail(PA_ERR_INVALID_ARG, w + ": max_context must be in [0, max_seq_len]");
    if (bad_partition(pool, partition_tokens))
      return fail(PA_ERR_INVALID_ARG,
                  w + ": partition_tokens must be 0 or a positive multiple of 16 and of block_size");
    if (num_seqs == 0) return PA_OK;
    if (d_context_lens == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null context lengths");
    pa::DecodeArgs a;
    a.lens = d_context_lens;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    const int32_t pt = choose_partition_tokens(pool, num_seqs, max_context, partition_tokens);
    a.partition_chunks = pt / 16;
    a.num_partitions = num_partitions(max_context, pt);
    a.max_context = max_context;
    if (static_cast<int64_t>(num_seqs) * d.num_kv_heads * a.num_partitions > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, w + ": launch too large");
    if (!pa::decode_uses_plan(pool->geom, a)) return PA_OK;
    const size_t need = pa::decode_workspace_bytes(num_seqs, num_q_heads, d.head_dim, a.num_partitions);
    if (d_workspace == nullptr || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, w + ": workspace needs " + std::to_string(need) + " bytes, got " +
                                        std::to_string(d_workspace ? workspace_bytes : 0));
    if (reinterpret_cast<uintptr_t>(d_workspace) & 15)
      return fail(PA_ERR_INVALID_ARG, w + ": workspace must be 16-byte aligned");
    a.ws = static_cast<float*>(d_workspace);
    const hipError_t e = pa::launch_decode_plan(pool->geom, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_HIP, w + ": " + hipGetErrorString(e));
    if (planned_out != nullptr) *planned_out = 1;
    return PA_OK;
  });
}

pa_status pa_decode_planned(pa_pool* pool, int32_t layer, const void* d_q, pa_dtype q_dtype,
                            int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                            int32_t table_stride, const int32_t* d_req_ids,
                            const int32_t* d_context_lens, int32_t num_seqs, int32_t max_context,
                            int32_t partition_tokens, float* d_out, void* d_workspace,
                            size_t workspace_bytes, void* stream) {
  return guarded("decode_planned", [&]() -> pa_status {
    return decode_impl("decode_planned", pool, layer, nullptr, nullptr, nullptr, d_q, q_dtype,
                       num_q_heads, scale, d_block_tables, table_stride, d_req_ids, d_context_lens,
                       num_seqs, max_context, partition_tokens, d_out, d_workspace, workspace_bytes,
                       stream, nullptr, nullptr, 0, 0, 0, false, /*plan_made=*/true);
  });
}

pa_status pa_append_decode_planned(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                   const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                                   int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                                   int32_t table_stride, const int32_t* d_req_ids,
                                   const int32_t* d_context_lens, int32_t num_seqs,
                                   int32_t max_context, int32_t partition_tokens, float* d_out,
                                   void* d_workspace, size_t workspace_bytes, void* stream) {
  return guarded("append_decode_planned", [&]() -> pa_status {
    if (d_k == nullptr || d_v == nullptr || d_slots == nullptr)
      return fail(PA_ERR_INVALID_ARG, "append_decode_planned: null k, v or slots");
    if ((reinterpret_cast<uintptr_t>(d_k) | reinterpret_cast<uintptr_t>(d_v)) & 15)
      return fail(PA_ERR_INVALID_ARG, "append_decode_planned: k and v must be 16-byte aligned");
    return decode_impl("append_decode_planned", pool, layer, d_k, d_v, d_slots, d_q, q_dtype,
                       num_q_heads, scale, d_block_tables, table_stride, d_req_ids, d_context_lens,
                       num_seqs, max_context, partition_tokens, d_out, d_workspace, workspace_bytes,
                       stream, nullptr, nullptr, 0, 0, 0, false, /*plan_made=*/true);
  });
}

pa_status pa_append_decode_noalloc(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                   const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                                   int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                                   int32_t table_stride, const int32_t* d_req_ids,
                                   const int32_t* d_context_lens, int32_t num_seqs,
                                   int32_t max_context, int32_t partition_tokens, float* d_out,
                                   void* stream) {
  return guarded("append_decode_noalloc", [&]() -> pa_status {
    if (d_k == nullptr || d_v == nullptr || d_slots == nullptr)
      return fail(PA_ERR_INVALID_ARG, "append_decode_noalloc: null k, v or slots");
    if ((reinterpret_cast<uintptr_t>(d_k) | reinterpret_cast<uintptr_t>(d_v)) & 15)
      return fail(PA_ERR_INVALID_ARG, "append_decode_noalloc: k and v must be 16-byte aligned");
    return decode_impl("append_decode_noalloc", pool, layer, d_k, d_v, d_slots, d_q, q_dtype,
                       num_q_heads, scale, d_block_tables, table_stride, d_req_ids, d_context_lens,
                       num_seqs, max_context, partition_tokens, d_out, nullptr, 0, stream, nullptr,
                       nullptr, 0, 0, 0, /*static_workspace=*/true);
  });
}

pa_status pa_shared_groups(const pa_pool* pool, const int32_t* req_ids, int32_t n,
                           int32_t partition_tokens, int32_t* seq_shared_out, int32_t* groups_out,
                           int32_t* n_groups_out, int32_t* max_members_out, int32_t* max_shared_out) {
  return guarded("shared_groups", [&]() -> pa_status {
    if (pool == nullptr || seq_shared_out == nullptr || groups_out == nullptr || n_groups_out == nullptr ||
        max_members_out == nullptr || max_shared_out == nullptr)
      return fail(PA_ERR_INVALID_ARG, "shared_groups: null argument");
    if (!pool->geom.paged) return fail(PA_ERR_INVALID_ARG, "shared_groups: sharing needs the paged layout");
    if (bad_partition(pool, partition_tokens) || partition_tokens <= 0)
      return fail(PA_ERR_INVALID_ARG, "shared_groups: partition_tokens must be a positive multiple of 16 and of block_size");
    std::string err;
    pa::Status st = pool->alloc.shared_groups(req_ids, n, partition_tokens, seq_shared_out, groups_out,
                                              n_groups_out, max_members_out, max_shared_out, &err);
    return from_alloc(st, err);
  });
}

pa_status pa_append_decode_shared(pa_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                  const int32_t* d_slots, const void* d_q, pa_dtype q_dtype,
                                  int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                                  int32_t table_stride, const int32_t* d_context_lens, int32_t num_seqs,
                                  int32_t max_context, int32_t partition_tokens, const int32_t* d_seq_shared,
                                  const int32_t* d_groups, int32_t num_groups, int32_t max_members,
                                  int32_t max_shared, float* d_out, void* d_workspace,
                                  size_t workspace_bytes, void* stream) {
  return guarded("append_decode_shared", [&]() -> pa_status {
    if (d_seq_shared == nullptr) return fail(PA_ERR_INVALID_ARG, "append_decode_shared: null seq_shared");
    if (d_k == nullptr || d_v == nullptr || d_slots == nullptr)
      return fail(PA_ERR_INVALID_ARG, "append_decode_shared: null k, v or slots");
    if ((reinterpret_cast<uintptr_t>(d_k) | reinterpret_cast<uintptr_t>(d_v)) & 15)
      return fail(PA_ERR_INVALID_ARG, "append_decode_shared: k and v must be 16-byte aligned");
    return decode_impl("append_decode_shared", pool, layer, d_k, d_v, d_slots, d_q, q_dtype, num_q_heads,
                       scale, d_block_tables, table_stride, nullptr, d_context_lens, num_seqs, max_context,
                       partition_tokens, d_out, d_workspace, workspace_bytes, stream, d_seq_shared, d_groups,
                       num_groups, max_members, max_shared);
  });
}

pa_status pa_check_shared_args(const pa_pool* pool, const int32_t* h_seq_shared,
                               const int32_t* h_context_lens, const int32_t* h_slots, int32_t num_seqs,
                               int32_t partition_tokens) {
  return guarded("check_shared_args", [&]() -> pa_status {
    const std::string w = "check_shared_args";
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null pool");
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, w + ": negative num_seqs");
    if (partition_tokens <= 0 || bad_partition(pool, partition_tokens))
      return fail(PA_ERR_INVALID_ARG, w + ": partition_tokens must be a positive multiple of 16 and of block_size");
    if (num_seqs == 0) return PA_OK;
    if (h_seq_shared == nullptr || h_context_lens == nullptr)
      return fail(PA_ERR_INVALID_ARG, w + ": null seq_shared or lengths");
    for (int32_t s = 0; s < num_seqs; ++s) {
      const std::string at = w + ": sequence " + std::to_string(s);
      const int32_t sh = h_seq_shared[s], L = h_context_lens[s];
      if (sh < 0 || sh % partition_tokens != 0 || sh > L)
        return fail(PA_ERR_INVALID_ARG, at + ": shared prefix " + std::to_string(sh) +
                                            " is not a multiple of partition_tokens within the context");
      if (h_slots != nullptr && h_slots[s] >= 0 && sh > L - 1)
        return fail(PA_ERR_INVALID_ARG, at + ": its new token (position " + std::to_string(L - 1) +
                                            ") lies in its shared prefix: find the groups after pa_reserve");
    }
    return PA_OK;
  });
}

pa_status pa_decode_shared(pa_pool* pool, int32_t layer, const void* d_q, pa_dtype q_dtype,
                           int32_t num_q_heads, float scale, const int32_t* d_block_tables,
                           int32_t table_stride, const int32_t* d_context_lens, int32_t num_seqs,
                           int32_t max_context, int32_t partition_tokens, const int32_t* d_seq_shared,
                           const int32_t* d_groups, int32_t num_groups, int32_t max_members,
                           int32_t max_shared, float* d_out, void* d_workspace,
                           size_t workspace_bytes, void* stream) {
  return guarded("decode_shared", [&]() -> pa_status {
    if (d_seq_shared == nullptr) return fail(PA_ERR_INVALID_ARG, "decode_shared: null seq_shared");
    return decode_impl("decode_shared", pool, layer, nullptr, nullptr, nullptr, d_q, q_dtype, num_q_heads,
                       scale, d_block_tables, table_stride, nullptr, d_context_lens, num_seqs,
                       max_context, partition_tokens, d_out, d_workspace, workspace_bytes, stream,
                       d_seq_shared, d_groups, num_groups, max_members, max_shared);
  });
}

// ---- host-side checks of device arrays (nothing is launched) -------------

pa_status pa_check_decode_args(const pa_pool* pool, const int32_t* h_block_tables,
                               int32_t table_stride, const int32_t* h_req_ids,
                               const int32_t* h_context_lens, const int32_t* h_slots,
                               int32_t num_seqs, int32_t max_context) {
  return guarded("check_decode_args", [&]() -> pa_status {
    const std::string w = "check_decode_args";
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null pool");
    const pa_pool_desc& d = pool->desc;
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, w + ": negative num_seqs");
    if (max_context < 0 || max_context > d.max_seq_len)
      return fail(PA_ERR_INVALID_ARG, w + ": max_context must be in [0, max_seq_len]");
    if (num_seqs == 0) return PA_OK;
    if (h_context_lens == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null lengths");
    const int32_t bs = d.block_size;
    const bool paged = d.layout == PA_PAGED;
    if (paged) {
      if (h_block_tables == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null block tables");
      if (table_stride < (max_context + bs - 1) / bs)
        return fail(PA_ERR_INVALID_ARG, w + ": table_stride is shorter than ceil(max_context / block_size)");
    } else if (h_req_ids == nullptr && num_seqs > d.max_seqs) {
      return fail(PA_ERR_INVALID_ARG, w + ": num_seqs exceeds max_seqs and no request ids are given");
    }
    std::vector<int64_t> taken;  // slots appended to, to find repeats
    for (int32_t s = 0; s < num_seqs; ++s) {
      const std::string at = w + ": sequence " + std::to_string(s);
      const int32_t L = h_context_lens[s];
      if (L < 0 || L > max_context)
        return fail(PA_ERR_INVALID_ARG, at + ": length " + std::to_string(L) + " outside [0, max_context]");
      const int32_t nblk = (L + bs - 1) / bs;
      int64_t last_slot = -1;  // slot of position L - 1
      if (paged) {
        const int32_t* row = h_block_tables + static_cast<int64_t>(s) * table_stride;
        for (int32_t j = 0; j < nblk; ++j) {
          if (row[j] < 0 || row[j] >= d.num_blocks)
            return fail(PA_ERR_INVALID_ARG, at + ": block table entry " + std::to_string(j) + " = " +
                                                std::to_string(row[j]) + " is not a block of the pool");
        }
        if (L > 0) last_slot = static_cast<int64_t>(row[(L - 1) / bs]) * bs + (L - 1) % bs;
      } else {
        const int32_t rid = h_req_ids ? h_req_ids[s] : s;
        if (rid < 0 || rid >= d.max_seqs)
          return fail(PA_ERR_INVALID_ARG, at + ": request id " + std::to_string(rid) + " outside [0, max_seqs)");
        if (pool->vmm != nullptr) {
          if (nblk * block_bytes(&d) > pool->vmm->region_mapped(rid))
            return fail(PA_ERR_INVALID_ARG, at + ": length " + std::to_string(L) + " reaches past the pages mapped for request " +
                                                std::to_string(rid));
        }
        if (L > 0) last_slot = static_cast<int64_t>(rid) * d.max_seq_len + L - 1;
      }
      if (h_slots != nullptr && h_slots[s] >= 0) {
        if (L < 1) return fail(PA_ERR_INVALID_ARG, at + ": appends a token but its length is 0");
        if (h_slots[s] != last_slot)
          return fail(PA_ERR_INVALID_ARG, at + ": slot " + std::to_string(h_slots[s]) + " is not the slot of position L-1 (" +
                                              std::to_string(last_slot) + ")");
        taken.push_back(h_slots[s]);
      }
    }
    std::sort(taken.begin(), taken.end());
    if (std::adjacent_find(taken.begin(), taken.end()) != taken.end())
      return fail(PA_ERR_INVALID_ARG, w + ": two sequences append to the same slot");
    return PA_OK;
  });
}

pa_status pa_check_slots(const pa_pool* pool, const int32_t* h_slots, int32_t n) {
  return guarded("check_slots", [&]() -> pa_status {
    const std::string w = "check_slots";
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null pool");
    if (n < 0) return fail(PA_ERR_INVALID_ARG, w + ": negative count");
    if (n == 0) return PA_OK;
    if (h_slots == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null slots");
    const pa_pool_desc& d = pool->desc;
    const int64_t rows = d.layout == PA_PAGED ? static_cast<int64_t>(d.num_blocks) * d.block_size
                                              : static_cast<int64_t>(d.max_seqs) * d.max_seq_len;
    std::vector<int32_t> taken;
    taken.reserve(n);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t slot = h_slots[i];
      if (slot < 0) continue;
      if (slot >= rows)
        return fail(PA_ERR_INVALID_ARG, w + ": slot " + std::to_string(slot) + " (token " + std::to_string(i) +
                                            ") is not a row of the pool");
      if (pool->vmm != nullptr) {
        const int32_t rid = slot / d.max_seq_len;
        const int64_t pos = slot % d.max_seq_len;
        if ((pos / d.block_size + 1) * block_bytes(&d) > pool->vmm->region_mapped(rid))
          return fail(PA_ERR_INVALID_ARG, w + ": slot " + std::to_string(slot) + " lies in an unmapped page");
      }
      taken.push_back(slot);
    }
    std::sort(taken.begin(), taken.end());
    if (std::adjacent_find(taken.begin(), taken.end()) != taken.end())
      return fail(PA_ERR_INVALID_ARG, w + ": a slot appears twice");
    return PA_OK;
  });
}

pa_status pa_check_block_pairs(const pa_pool* pool, const int32_t* h_pairs, int32_t n) {
  return guarded("check_block_pairs", [&]() -> pa_status {
    const std::string w = "check_block_pairs";
    if (pool == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null pool");
    if (n < 0) return fail(PA_ERR_INVALID_ARG, w + ": negative count");
    if (n == 0) return PA_OK;
    if (pool->desc.layout != PA_PAGED) return fail(PA_ERR_INVALID_ARG, w + ": contiguous pool has no blocks");
    if (h_pairs == nullptr) return fail(PA_ERR_INVALID_ARG, w + ": null pairs");
    std::vector<int32_t> srcs, dsts;
    for (int32_t i = 0; i < n; ++i) {
      for (int k = 0; k < 2; ++k) {
        const int32_t b = h_pairs[2 * i + k];
        if (b < 0 || b >= pool->desc.num_blocks)
          return fail(PA_ERR_INVALID_ARG, w + ": pair " + std::to_string(i) + " names block " + std::to_string(b) +
                                              ", not a block of the pool");
      }
      if (h_pairs[2 * i] == h_pairs[2 * i + 1])
        return fail(PA_ERR_INVALID_ARG, w + ": pair " + std::to_string(i) + " copies a block onto itself");
      srcs.push_back(h_pairs[2 * i]);
      dsts.push_back(h_pairs[2 * i + 1]);
    }
    std::sort(srcs.begin(), srcs.end());
    std::sort(dsts.begin(), dsts.end());
    if (std::adjacent_find(dsts.begin(), dsts.end()) != dsts.end())
      return fail(PA_ERR_INVALID_ARG, w + ": a block is the destination of two pairs");
    for (int32_t b : dsts)
      if (std::binary_search(srcs.begin(), srcs.end(), b))
        return fail(PA_ERR_INVALID_ARG, w + ": block " + std::to_string(b) + " is both a source and a destination");
    return PA_OK;
  });
}

const char* pa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
