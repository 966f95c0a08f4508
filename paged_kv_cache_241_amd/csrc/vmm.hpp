// Demand-paged contiguous KV cache ("Leveraging Low-Level CUDA APIs for
// vAttention's Dynamic Memory", 5.2.1-5.2.3): per layer a virtual tensor (K
// and V tile pairs) for the maximum batch in which request reqId owns the
// sub-range at reqId x region_bytes; virtual memory is reserved once, and physical pages
// are mapped into a request's sub-range as it grows (sub-ranges are backed
// independently, one physical allocation per page: 2 MiB where the sub-ranges
// allow, else the allocation granularity).  Built on
// ROCm's virtual memory calls (hipMemAddressReserve, hipMemCreate, hipMemMap,
// hipMemSetAccess).  Host code; no kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

namespace pa {

class VirtualCache {
 public:
  // Reserves num_layers * max_seqs * region_bytes of virtual memory on
  // `device`, with no physical memory.  physical_bytes caps the memory mapped
  // over all layers.  Returns "" on success, else the reason (and *out stays
  // null).
  static std::string create(int32_t num_layers, int32_t max_seqs, int64_t region_bytes,
                            size_t physical_bytes, int device, VirtualCache** out);
  ~VirtualCache();
  VirtualCache(const VirtualCache&) = delete;
  VirtualCache& operator=(const VirtualCache&) = delete;

  char* base() const { return base_; }
  int64_t page_bytes() const { return page_; }
  int64_t region_bytes() const { return region_; }

  // Physical bytes request rid's growth to hold its first `bytes` bytes (in
  // every layer) would add.
  int64_t bytes_short(int32_t rid, int64_t bytes) const;
  int64_t bytes_free() const { return budget_ - mapped_; }
  int64_t bytes_mapped() const { return mapped_; }
  int64_t bytes_budget() const { return budget_; }
  int64_t region_mapped(int32_t rid) const { return static_cast<int64_t>(pages_[rid]) * page_; }

  // Back the first `bytes` bytes of rid's sub-range in every layer.
  // The caller has checked bytes_short against bytes_free.  On a HIP error,
  // whatever this call mapped is taken back and the reason returned.
  std::string grow(int32_t rid, int64_t bytes);

  // Unmap and free rid's pages.  No queued or running work may touch them.
  std::string trim(int32_t rid);

 private:
  struct Mapping {
    char* addr;
    size_t size;
    hipMemGenericAllocationHandle_t handle;
  };
  VirtualCache() = default;
  std::string map_range(char* addr, size_t size, Mapping* m) const;
  static void unmap(const Mapping& m);

  int device_ = 0;
  int32_t num_layers_ = 0, max_seqs_ = 0;
  int64_t region_ = 0, page_ = 0, budget_ = 0, mapped_ = 0;
  size_t reserved_ = 0;  // bytes of the virtual range
  char* base_ = nullptr;
  std::vector<int32_t> pages_;              // pages backed per sub-range, per request id
  std::vector<std::vector<Mapping>> maps_;  // per request id
};

}  // namespace pa
