// Achievable HBM read rate of the GPU, next to the datasheet peak: a plain
// streaming read and a read of 4 KiB tiles (the size of one bf16 cache tile of
// 16 tokens x 128 dims) in order and in a random order.  Prints one line per
// case, "<case> <workgroups> <GB/s>", for bench.py.  Every index is < n
// (grid-stride loops; tile ids are a permutation of all tiles).
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <algorithm>
#include <random>
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("hip error %s line %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__global__ void stream_read(const u32x4* __restrict__ b, size_t n, unsigned* out, int nt) {
  u32x4 acc = {0, 0, 0, 0};
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x, st = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += st) acc ^= nt ? __builtin_nontemporal_load(b + i) : b[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}
// one wave reads whole 4 KiB tiles (256 x 16 B): tile = perm[t]
__global__ void tile_read(const u32x4* __restrict__ b, const int* __restrict__ perm, int ntiles, unsigned* out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  u32x4 acc = {0, 0, 0, 0};
  for (int t = wave; t < ntiles; t += nw) {
    const u32x4* p = b + (size_t)perm[t] * 256;
    acc ^= __builtin_nontemporal_load(p + lane) ^ __builtin_nontemporal_load(p + 64 + lane) ^
           __builtin_nontemporal_load(p + 128 + lane) ^ __builtin_nontemporal_load(p + 192 + lane);
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}
int main() {
  const size_t bytes = (size_t)4 << 30, n = bytes / 16;
  const int ntiles = (int)(bytes / 4096);
  u32x4* b; unsigned* out; int* perm;
  CK(hipMalloc(&b, bytes)); CK(hipMemset(b, 1, bytes));
  const int maxthreads = 256 * 64 * 256;
  CK(hipMalloc(&out, (size_t)maxthreads * 4));
  std::vector<int> hp(ntiles); for (int i = 0; i < ntiles; ++i) hp[i] = i;
  CK(hipMalloc(&perm, (size_t)ntiles * 4));
  hipEvent_t ev0, ev1; CK(hipEventCreate(&ev0)); CK(hipEventCreate(&ev1));
  for (int nt = 0; nt < 2; ++nt) for (int wg : {1024, 2048, 4096, 8192}) {
    hipLaunchKernelGGL(stream_read, dim3(wg), dim3(256), 0, 0, b, n, out, nt); CK(hipGetLastError());
    CK(hipEventRecord(ev0));
    for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(stream_read, dim3(wg), dim3(256), 0, 0, b, n, out, nt);
    CK(hipEventRecord(ev1)); CK(hipEventSynchronize(ev1));
    float ms; CK(hipEventElapsedTime(&ms, ev0, ev1));
    printf("stream%s %d %.0f\n", nt ? "_nt" : "", wg, 5.0 * bytes / (ms / 1e3) / 1e9);
  }
  for (int shuffle = 0; shuffle < 2; ++shuffle) {
    if (shuffle) { std::mt19937 g(1); std::shuffle(hp.begin(), hp.end(), g); }
    CK(hipMemcpy(perm, hp.data(), (size_t)ntiles * 4, hipMemcpyHostToDevice));
    for (int wg : {512, 1024, 2048, 4096}) {
      hipLaunchKernelGGL(tile_read, dim3(wg), dim3(256), 0, 0, b, perm, ntiles, out); CK(hipGetLastError());
      CK(hipEventRecord(ev0));
      for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(tile_read, dim3(wg), dim3(256), 0, 0, b, perm, ntiles, out);
      CK(hipEventRecord(ev1)); CK(hipEventSynchronize(ev1));
      float ms; CK(hipEventElapsedTime(&ms, ev0, ev1));
      printf("tiles_%s %d %.0f\n", shuffle ? "random" : "in_order", wg, 5.0 * bytes / (ms / 1e3) / 1e9);
    }
  }
  return 0;
}
