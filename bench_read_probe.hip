// Achievable HBM read rate of the GPU, next to the datasheet peak: a plain
// streaming read, a read of 4 KiB tiles (the size of one bf16 cache tile of
// 16 tokens x 128 dims) in order and in a random order, and the decode's own
// read patterns without their arithmetic.  Prints one line per
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
// The decode's own read pattern without its arithmetic: 512 workgroups x 4
// waves, each wave walks 16 random blocks and reads, per block, a 4 KiB K
// tile (4 x 16 B per lane) and a 4 KiB V tile (8 x 8 B per lane) from two
// arrays.  ids[] holds block ids < nblocks.
__global__ void kv_pattern(const char* __restrict__ K, const char* __restrict__ V,
                           const int* __restrict__ ids, int per_wave, unsigned* out) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  u32x4 acc = {0, 0, 0, 0};
  for (int i = 0; i < per_wave; ++i) {
    const long tile = (long)ids[gw * per_wave + i] * 4096;
    u32x4 k[4];
    u32x2 v[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) k[x] = __builtin_nontemporal_load((const u32x4*)(K + tile + x * 1024 + lane * 16));
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = __builtin_nontemporal_load((const u32x2*)(V + tile + x * 512 + lane * 8));
#pragma unroll
    for (int x = 0; x < 4; ++x) acc ^= k[x];
#pragma unroll
    for (int x = 0; x < 8; ++x) { acc.x ^= v[x].x; acc.y ^= v[x].y; }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// The decode's exact mapping on the Llama-3-8B batch-64 layer, without its
// arithmetic: K and V pools of [4096 blocks][8 heads][4 KiB tile] per layer,
// 64 sequences of 64 blocks each (a seeded permutation), workgroup
// s * 8 + h of 4 waves, wave w reading chunks 63 - w, 59 - w, ... down to 0.
// table[] holds block ids < 4096, so every tile lies inside its pool.
__global__ void decode_mapped(const char* __restrict__ K, const char* __restrict__ V,
                              const int* __restrict__ table, unsigned* out) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.x / 8, h = blockIdx.x % 8;
  u32x4 acc = {0, 0, 0, 0};
  for (int c = 63 - wave; c >= 0; c -= 4) {
    const long tile = ((long)table[s * 64 + c] * 8 + h) * 4096;
    u32x4 k[4];
    u32x2 v[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) k[x] = __builtin_nontemporal_load((const u32x4*)(K + tile + x * 1024 + lane * 16));
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = __builtin_nontemporal_load((const u32x2*)(V + tile + x * 512 + lane * 8));
#pragma unroll
    for (int x = 0; x < 4; ++x) acc ^= k[x];
#pragma unroll
    for (int x = 0; x < 8; ++x) { acc.x ^= v[x].x; acc.y ^= v[x].y; }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Variants of decode_mapped, each changing one thing (same 268 MB per launch,
// 8 rotated layer pools, 64 sequences x 8 heads x 64 blocks, table[] < 4096):
//   KV8K  K and V of one (block, head) side by side, one 8 KiB run
//         ([4096][8][K 4 KiB | V 4 KiB] per layer);
//   TWO   each wave keeps two chunks' loads in flight (chunks c and c - 4);
//   W8    8 waves per workgroup (4096 waves, 8 chunks each).
// Every wave of every variant reads exactly the tiles decode_mapped reads.
template <bool KV8K, bool TWO, int W>
__global__ void decode_mapped_var(const char* __restrict__ K, const char* __restrict__ V,
                                  const int* __restrict__ table, unsigned* out) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.x / 8, h = blockIdx.x % 8;
  u32x4 acc = {0, 0, 0, 0};
  auto read = [&](int c) {
    const long blk = (long)table[s * 64 + c] * 8 + h;
    const char* kt = KV8K ? K + blk * 8192 : K + blk * 4096;
    const char* vt = KV8K ? K + blk * 8192 + 4096 : V + blk * 4096;
    u32x4 k[4];
    u32x2 v[8];
#pragma unroll
    for (int x = 0; x < 4; ++x) k[x] = __builtin_nontemporal_load((const u32x4*)(kt + x * 1024 + lane * 16));
#pragma unroll
    for (int x = 0; x < 8; ++x) v[x] = __builtin_nontemporal_load((const u32x2*)(vt + x * 512 + lane * 8));
#pragma unroll
    for (int x = 0; x < 4; ++x) acc ^= k[x];
#pragma unroll
    for (int x = 0; x < 8; ++x) { acc.x ^= v[x].x; acc.y ^= v[x].y; }
  };
  if (TWO) {
    // chunks c and c - W together; with W = 4 and c from 63 - wave down by
    // 8, c - 4 >= 3 - wave >= 0
    for (int c = 63 - wave; c >= 0; c -= 2 * W) {
      const long b0 = (long)table[s * 64 + c] * 8 + h, b1 = (long)table[s * 64 + c - W] * 8 + h;
      u32x4 k0[4], k1[4];
      u32x2 v0[8], v1[8];
      const char* kt0 = KV8K ? K + b0 * 8192 : K + b0 * 4096;
      const char* vt0 = KV8K ? K + b0 * 8192 + 4096 : V + b0 * 4096;
      const char* kt1 = KV8K ? K + b1 * 8192 : K + b1 * 4096;
      const char* vt1 = KV8K ? K + b1 * 8192 + 4096 : V + b1 * 4096;
#pragma unroll
      for (int x = 0; x < 4; ++x) k0[x] = __builtin_nontemporal_load((const u32x4*)(kt0 + x * 1024 + lane * 16));
#pragma unroll
      for (int x = 0; x < 8; ++x) v0[x] = __builtin_nontemporal_load((const u32x2*)(vt0 + x * 512 + lane * 8));
#pragma unroll
      for (int x = 0; x < 4; ++x) k1[x] = __builtin_nontemporal_load((const u32x4*)(kt1 + x * 1024 + lane * 16));
#pragma unroll
      for (int x = 0; x < 8; ++x) v1[x] = __builtin_nontemporal_load((const u32x2*)(vt1 + x * 512 + lane * 8));
#pragma unroll
      for (int x = 0; x < 4; ++x) acc ^= k0[x] ^ k1[x];
#pragma unroll
      for (int x = 0; x < 8; ++x) { acc.x ^= v0[x].x ^ v1[x].x; acc.y ^= v0[x].y ^ v1[x].y; }
    }
  } else {
    for (int c = 63 - wave; c >= 0; c -= W) read(c);
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// 4 KiB tiles in a random order, one wave per tile, over one 256 MiB layer
// pool per launch (8 pools rotated): the tile probe at the decode's launch
// size.  perm[] is a permutation of the 65536 tiles of a pool.
__global__ void tile_read_pool(const u32x4* __restrict__ b, const int* __restrict__ perm, int ntiles, unsigned* out) {
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
  {
    // decode-shaped pattern: K and V tiles from the two halves of the buffer
    const char* Kp = reinterpret_cast<const char*>(b);
    const char* Vp = Kp + bytes / 2;
    const int nblocks = (int)(bytes / 2 / 4096), per_wave = 16, wg = 512, waves = wg * 4;
    std::vector<int> ids((size_t)waves * per_wave);
    std::mt19937 g(7);
    std::uniform_int_distribution<int> U(0, nblocks - 1);
    for (auto& x : ids) x = U(g);
    int* dids;
    CK(hipMalloc(&dids, ids.size() * 4));
    CK(hipMemcpy(dids, ids.data(), ids.size() * 4, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(kv_pattern, dim3(wg), dim3(256), 0, 0, Kp, Vp, dids, per_wave, out);
    CK(hipGetLastError());
    CK(hipEventRecord(ev0));
    for (int r = 0; r < 20; ++r) hipLaunchKernelGGL(kv_pattern, dim3(wg), dim3(256), 0, 0, Kp, Vp, dids, per_wave, out);
    CK(hipEventRecord(ev1)); CK(hipEventSynchronize(ev1));
    float ms; CK(hipEventElapsedTime(&ms, ev0, ev1));
    const double moved = (double)waves * per_wave * 8192;
    printf("decode_pattern %d %.0f\n", wg, moved * 20 / (ms / 1e3) / 1e9);
    printf("decode_pattern_us %d %.2f\n", wg, ms * 1e3 / 20);
  }
  {
    // the decode's exact mapping, 8 layer pools rotated as the benchmark
    // rotates them (2 GiB of the 4 GiB buffer)
    const size_t pool = (size_t)4096 * 8 * 4096;
    const int layers = 8;
    std::vector<int> blocks(4096);
    for (int i = 0; i < 4096; ++i) blocks[i] = i;
    std::mt19937 g(2412);
    std::shuffle(blocks.begin(), blocks.end(), g);
    int* table;
    CK(hipMalloc(&table, 4096 * 4));
    CK(hipMemcpy(table, blocks.data(), 4096 * 4, hipMemcpyHostToDevice));
    const char* base = reinterpret_cast<const char*>(b);
    for (int l = 0; l < layers; ++l)
      hipLaunchKernelGGL(decode_mapped, dim3(512), dim3(256), 0, 0, base + l * 2 * pool, base + l * 2 * pool + pool,
                         table, out);
    CK(hipGetLastError());
    CK(hipDeviceSynchronize());
    CK(hipEventRecord(ev0));
    for (int r = 0; r < 5; ++r)
      for (int l = 0; l < layers; ++l)
        hipLaunchKernelGGL(decode_mapped, dim3(512), dim3(256), 0, 0, base + l * 2 * pool,
                           base + l * 2 * pool + pool, table, out);
    CK(hipEventRecord(ev1));
    CK(hipEventSynchronize(ev1));
    float ms;
    CK(hipEventElapsedTime(&ms, ev0, ev1));
    const double moved = 512.0 * 64 * 8192;
    printf("decode_mapped 512 %.0f\n", moved * 5 * layers / (ms / 1e3) / 1e9);
    printf("decode_mapped_us 512 %.2f\n", ms * 1e3 / (5 * layers));
    // one-change variants; each pool pair [K 128 MiB][V 128 MiB] of the
    // rotation serves as one 256 MiB interleaved pool for KV8K
    std::vector<int> ident(4096);
    for (int i = 0; i < 4096; ++i) ident[i] = i;
    int* table_in_order;
    CK(hipMalloc(&table_in_order, 4096 * 4));
    CK(hipMemcpy(table_in_order, ident.data(), 4096 * 4, hipMemcpyHostToDevice));
    auto run = [&](const char* name, auto kern, int threads, const int* tb) -> int {
      for (int l = 0; l < layers; ++l)
        hipLaunchKernelGGL(kern, dim3(512), dim3(threads), 0, 0, base + l * 2 * pool, base + l * 2 * pool + pool, tb, out);
      CK(hipGetLastError());
      CK(hipDeviceSynchronize());
      CK(hipEventRecord(ev0));
      for (int r = 0; r < 5; ++r)
        for (int l = 0; l < layers; ++l)
          hipLaunchKernelGGL(kern, dim3(512), dim3(threads), 0, 0, base + l * 2 * pool, base + l * 2 * pool + pool, tb, out);
      CK(hipEventRecord(ev1));
      CK(hipEventSynchronize(ev1));
      float t;
      CK(hipEventElapsedTime(&t, ev0, ev1));
      printf("%s 512 %.0f\n", name, moved * 5 * layers / (t / 1e3) / 1e9);
      printf("%s_us 512 %.2f\n", name, t * 1e3 / (5 * layers));
      return 0;
    };
    if (run("decode_mapped_kv8k", decode_mapped_var<true, false, 4>, 256, table)) return 1;
    if (run("decode_mapped_two", decode_mapped_var<false, true, 4>, 256, table)) return 1;
    if (run("decode_mapped_kv8k_two", decode_mapped_var<true, true, 4>, 256, table)) return 1;
    if (run("decode_mapped_w8", decode_mapped_var<false, false, 8>, 512, table)) return 1;
    if (run("decode_mapped_in_order", decode_mapped_var<false, false, 4>, 256, table_in_order)) return 1;
    // random 4 KiB tiles at the decode's launch size: 2048 waves over one
    // 256 MiB pool per launch
    {
      const int nt = (int)(2 * pool / 4096);
      std::vector<int> pp(nt);
      for (int i = 0; i < nt; ++i) pp[i] = i;
      std::mt19937 g2(11);
      std::shuffle(pp.begin(), pp.end(), g2);
      int* dperm;
      CK(hipMalloc(&dperm, (size_t)nt * 4));
      CK(hipMemcpy(dperm, pp.data(), (size_t)nt * 4, hipMemcpyHostToDevice));
      for (int l = 0; l < layers; ++l)
        hipLaunchKernelGGL(tile_read_pool, dim3(512), dim3(256), 0, 0, (const u32x4*)(base + l * 2 * pool), dperm, nt, out);
      CK(hipGetLastError());
      CK(hipDeviceSynchronize());
      CK(hipEventRecord(ev0));
      for (int r = 0; r < 5; ++r)
        for (int l = 0; l < layers; ++l)
          hipLaunchKernelGGL(tile_read_pool, dim3(512), dim3(256), 0, 0, (const u32x4*)(base + l * 2 * pool), dperm, nt, out);
      CK(hipEventRecord(ev1));
      CK(hipEventSynchronize(ev1));
      float t;
      CK(hipEventElapsedTime(&t, ev0, ev1));
      printf("tiles_random_pool 512 %.0f\n", 2.0 * pool * 5 * layers / (t / 1e3) / 1e9);
      printf("tiles_random_pool_us 512 %.2f\n", t * 1e3 / (5 * layers));
    }
  }
  return 0;
}
