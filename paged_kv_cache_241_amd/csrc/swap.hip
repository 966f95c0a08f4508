// HIP kernel of pre-emption by swapping ("Running Out of Cache": when paging
// runs out, a request's cache is evicted and swapped back in later, section
// "Fragmentation is lost users" and the Pre-emption term): a request's blocks
// move between the pool and an image the caller owns, in pinned host memory
// (written and read through its device mapping) or in device memory.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace pa {
namespace {

// Block ids of one swap launch, passed by value (kernel arguments).
constexpr int kSwapBatch = 256;
struct SwapBlocks {
  int32_t id[kSwapBatch];
};

// Workgroup (j, layer) moves block ids.id[j] of `layer` between the pool and
// the image: its num_kv_heads tile pairs (K, V), contiguous in both.  j0 is
// the first logical block of the launch, n_total the request's block count
// (the image's second dimension).
__global__ __launch_bounds__(256) void swap_blocks_kernel(CacheGeom g, SwapBlocks ids, int32_t j0,
                                                          int32_t n_total, char* image,
                                                          int32_t to_image) {
  const int j = blockIdx.x;
  const int layer = blockIdx.y;
  const int64_t bb = static_cast<int64_t>(g.num_kv_heads) * 2 * g.tile_bytes;
  char* blk = g.base + static_cast<int64_t>(layer) * g.layer_bytes + static_cast<int64_t>(ids.id[j]) * bb;
  char* img = image + (static_cast<int64_t>(layer) * n_total + j0 + j) * bb;
  const uint4* src = reinterpret_cast<const uint4*>(to_image ? blk : img);
  uint4* dst = reinterpret_cast<uint4*>(to_image ? img : blk);
  for (int64_t x = threadIdx.x; x < bb / 16; x += 256) dst[x] = src[x];
}

}  // namespace

hipError_t launch_swap(const CacheGeom& g, const int32_t* blocks, int32_t n, char* image,
                       bool to_image, hipStream_t stream) {
  for (int32_t j0 = 0; j0 < n; j0 += kSwapBatch) {
    const int32_t cnt = n - j0 < kSwapBatch ? n - j0 : kSwapBatch;
    SwapBlocks ids{};
    for (int32_t j = 0; j < cnt; ++j) ids.id[j] = blocks[j0 + j];
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(static_cast<uint32_t>(cnt), g.num_layers),
                       dim3(256), 0, stream, g, ids, j0, n, image, to_image ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pa
