// Demand-paged contiguous KV cache (see vmm.hpp).
#include "vmm.hpp"

namespace pa {

namespace {

std::string hip_err(const char* what, hipError_t e) {
  (void)hipGetLastError();  // leave no error behind for the next launch
  return std::string(what) + ": " + hipGetErrorString(e);
}

hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop{};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

}  // namespace

std::string VirtualCache::create(int32_t num_layers, int32_t max_seqs, int64_t region_bytes,
                                 size_t physical_bytes, int device, VirtualCache** out) {
  *out = nullptr;
  int supported = 0;
  hipError_t e = hipDeviceGetAttribute(&supported, hipDeviceAttributeVirtualMemoryManagementSupported,
                                       device);
  if (e != hipSuccess) return hip_err("hipDeviceGetAttribute", e);
  if (!supported) return "the device has no virtual memory management";
  const hipMemAllocationProp prop = device_prop(device);
  size_t gran = 0;
  e = hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityRecommended);
  if (e != hipSuccess) return hip_err("hipMemGetAllocationGranularity", e);
  if (gran == 0) return "zero allocation granularity";
  // 2 MiB pages where the sub-ranges allow (fewer mapping calls, wider TLB
  // reach), else the granularity itself
  constexpr size_t kLargePage = size_t{2} << 20;
  if (kLargePage % gran == 0 && region_bytes % static_cast<int64_t>(kLargePage) == 0) gran = kLargePage;
  if (region_bytes <= 0 || region_bytes % static_cast<int64_t>(gran) != 0)
    return "a request's sub-range (" + std::to_string(region_bytes) +
           " bytes) must be a multiple of the page size (" + std::to_string(gran) + " bytes)";
  VirtualCache* vc = new VirtualCache();
  vc->device_ = device;
  vc->num_layers_ = num_layers;
  vc->max_seqs_ = max_seqs;
  vc->region_ = region_bytes;
  vc->page_ = static_cast<int64_t>(gran);
  vc->budget_ = static_cast<int64_t>(physical_bytes / gran) * vc->page_;
  vc->reserved_ = static_cast<size_t>(num_layers) * max_seqs * region_bytes;
  vc->pages_.assign(max_seqs, 0);
  vc->maps_.resize(max_seqs);
  void* base = nullptr;
  e = hipMemAddressReserve(&base, vc->reserved_, gran, nullptr, 0);
  if (e != hipSuccess) {
    delete vc;
    return hip_err("hipMemAddressReserve", e);
  }
  vc->base_ = static_cast<char*>(base);
  *out = vc;
  return "";
}

VirtualCache::~VirtualCache() {
  for (auto& list : maps_)
    for (const Mapping& m : list) unmap(m);
  if (base_) (void)hipMemAddressFree(base_, reserved_);
  (void)hipGetLastError();
}

int64_t VirtualCache::bytes_short(int32_t rid, int64_t bytes) const {
  const int64_t want = (bytes + page_ - 1) / page_;
  const int64_t more = want > pages_[rid] ? want - pages_[rid] : 0;
  return more * page_ * num_layers_;
}

std::string VirtualCache::map_range(char* addr, size_t size, Mapping* m) const {
  const hipMemAllocationProp prop = device_prop(device_);
  hipMemGenericAllocationHandle_t h{};
  hipError_t e = hipMemCreate(&h, size, &prop, 0);
  if (e != hipSuccess) return hip_err("hipMemCreate", e);
  e = hipMemMap(addr, size, 0, h, 0);
  if (e != hipSuccess) {
    (void)hipMemRelease(h);
    return hip_err("hipMemMap", e);
  }
  hipMemAccessDesc access{};
  access.location.type = hipMemLocationTypeDevice;
  access.location.id = device_;
  access.flags = hipMemAccessFlagsProtReadWrite;
  e = hipMemSetAccess(addr, size, &access, 1);
  if (e != hipSuccess) {
    (void)hipMemUnmap(addr, size);
    (void)hipMemRelease(h);
    return hip_err("hipMemSetAccess", e);
  }
  *m = Mapping{addr, size, h};
  return "";
}

void VirtualCache::unmap(const Mapping& m) {
  (void)hipMemUnmap(m.addr, m.size);
  (void)hipMemRelease(m.handle);
}

// One physical allocation per page: a handle spanning several pages is
// mapped fine but its access can be refused once other mappings share the
// reservation (measured on MI355X with ROCm 7.2).
std::string VirtualCache::grow(int32_t rid, int64_t bytes) {
  const int64_t want = (bytes + page_ - 1) / page_;
  const int64_t have = pages_[rid];
  if (want <= have) return "";
  std::vector<Mapping>& list = maps_[rid];
  const size_t before = list.size();
  for (int32_t l = 0; l < num_layers_; ++l) {
    char* region = base_ + (static_cast<int64_t>(l) * max_seqs_ + rid) * region_;
    for (int64_t pg = have; pg < want; ++pg) {
      Mapping m{};
      const std::string err = map_range(region + pg * page_, static_cast<size_t>(page_), &m);
      if (!err.empty()) {
        while (list.size() > before) {
          unmap(list.back());
          list.pop_back();
        }
        return err;
      }
      list.push_back(m);
    }
  }
  pages_[rid] = static_cast<int32_t>(want);
  mapped_ += (want - have) * page_ * num_layers_;
  return "";
}

std::string VirtualCache::trim(int32_t rid) {
  for (const Mapping& m : maps_[rid]) unmap(m);
  mapped_ -= static_cast<int64_t>(pages_[rid]) * page_ * num_layers_;
  maps_[rid].clear();
  pages_[rid] = 0;
  return "";
}

}  // namespace pa
